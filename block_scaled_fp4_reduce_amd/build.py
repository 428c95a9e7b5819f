"""Build libfp4q.so (HIP, gfx950) in-tree with hipcc.

    python -m block_scaled_fp4_reduce_amd.build [--asm]

Flags: gfx950 only; no fp contraction (every fused multiply-add in the
kernels is an explicit fmaf, so results are reproducible bit for bit);
packed fp32 instructions disabled; fp32 division stays correctly rounded
(the HIP default).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp4q.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-ffp-contract=off",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function", "-Wno-unused-command-line-argument",
]


def sources():
    return [os.path.join(CSRC, "fp4q.hip")]


def deps():
    out = [os.path.join(CSRC, f) for f in os.listdir(CSRC)]
    out.append(os.path.join(os.path.dirname(HERE), "include", "fp4q.h"))
    return out


def build(verbose: bool = False) -> str:
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *FLAGS, *sources(), "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


def up_to_date() -> bool:
    if not os.path.exists(LIB):
        return False
    t = os.path.getmtime(LIB)
    return all(os.path.getmtime(d) <= t for d in deps())


def dump_asm(out_dir: str) -> str:
    """Device assembly of the kernels, for inspection."""
    os.makedirs(out_dir, exist_ok=True)
    cmd = [HIPCC, *[f for f in FLAGS if f not in ("-shared", "-fPIC")],
           "--cuda-device-only", "-S", *sources(), "-o", os.path.join(out_dir, "fp4q-gfx950.s")]
    subprocess.check_call(cmd)
    return os.path.join(out_dir, "fp4q-gfx950.s")


if __name__ == "__main__":
    if "--asm" in sys.argv:
        print(dump_asm(os.path.join(os.path.dirname(HERE), "_build", "asm")))
    else:
        print(build(verbose=True))
