"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer
(CPU only): the oracle test files run against a copy of fp4_oracle.c built
with -fsanitize=address,undefined (every report fatal) in a child process.
The two exhaustive format sweeps are left out (their code paths are the
scalar encoders every other test calls); a strided sample of the same sweeps
runs instead."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "fp4_oracle.c")
TESTS = ["tests/test_oracle_pins.py", "tests/test_oracle_msed.py", "tests/test_oracle_rows.py",
         "tests/test_oracle_requant.py", "tests/test_oracle_gemm.py", "tests/test_error_study.py",
         "tests/test_rotated_tolerance.py"]

SAMPLE = r"""
import numpy as np, oracle, os
assert oracle.loaded_path() == os.environ["FP4Q_ORACLE_LIB"]
bits = np.arange(0, 2**32, 4099, dtype=np.uint64).astype(np.uint32)   # every 4099th fp32
f = bits.view(np.float32)
c = oracle.e2m1_encode(f)
e = oracle.e4m3_encode(np.abs(f[np.isfinite(f)]))
assert c.max() <= 15 and e.max() <= 0x7F
print("sample ok", f.size)
"""


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("no gcc")
    asan = subprocess.check_output([gcc, "-print-file-name=libasan.so"], text=True).strip()
    if not os.path.isabs(asan) or not os.path.exists(asan):
        pytest.skip("gcc has no libasan")
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.check_call([gcc, "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
                           "-fPIC", "-shared", "-fsanitize=address,undefined",
                           "-fno-sanitize-recover=all", "-fno-omit-frame-pointer", SRC, "-o", lib,
                           "-lm"])
    env = dict(os.environ, LD_PRELOAD=asan, FP4Q_ORACLE_LIB=lib,
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1:alloc_dealloc_mismatch=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-c", SAMPLE], env=env, cwd=ROOT, capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 0 and "sample ok" in r.stdout, r.stdout[-2000:] + r.stderr[-4000:]
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "-m", "not gpu", "-k", "not exhaustive and not every_fp32", *TESTS],
                       env=env, cwd=ROOT, capture_output=True, text=True, timeout=900)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-4000:]
    assert " passed" in r.stdout
