"""CPU oracle for block-scaled FP4 quantization (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The library under test never does,
and the two share no code: this module wraps ``fp4_oracle.c`` (plain C,
fp32 with the operation order written there) through ctypes and numpy.

Parity status per function is listed at the top of ``fp4_oracle.c``; the
functions here are marshalling only.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
# A prebuilt copy of this same source to load instead (the sanitizer test
# builds one with -fsanitize=address,undefined); never rebuilt here.
_LIB_OVERRIDE = os.environ.get("FP4Q_ORACLE_LIB")

FOUR_OVER_SIX = 1 << 0
SR = 1 << 1
RHT16 = 1 << 2
BLOCK2D = 1 << 3
HAD32 = 1 << 4
ROWWISE = 1 << 5
COLWISE = 1 << 6
MSEDEN = 1 << 7

_CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
           "-fPIC", "-shared", "-Wall", "-Wextra"]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no GPU code involved)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
            os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "fp4_oracle.h"))):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def loaded_path() -> str:
    """Path of the oracle library lib() loads."""
    return _LIB_OVERRIDE or _LIB


def lib():
    global _lib
    if _lib is None:
        if not _LIB_OVERRIDE:
            build()
        L = C.CDLL(loaded_path())
        u8p, f32p, u16p, u32p = (C.POINTER(C.c_uint8), C.POINTER(C.c_float),
                                 C.POINTER(C.c_uint16), C.POINTER(C.c_uint32))
        L.orc_e2m1_encode.restype = C.c_uint8
        L.orc_e2m1_encode.argtypes = [C.c_float]
        L.orc_e2m1_decode.restype = C.c_float
        L.orc_e2m1_decode.argtypes = [C.c_uint8]
        L.orc_e4m3_encode.restype = C.c_uint8
        L.orc_e4m3_encode.argtypes = [C.c_float]
        L.orc_e4m3_decode.restype = C.c_float
        L.orc_e4m3_decode.argtypes = [C.c_uint8]
        L.orc_ue8m0_decode.restype = C.c_float
        L.orc_ue8m0_decode.argtypes = [C.c_uint8]
        L.orc_e2m1_encode_array.argtypes = [f32p, C.c_int64, u8p]
        L.orc_e4m3_encode_array.argtypes = [f32p, C.c_int64, u8p]
        L.orc_philox4x32_10.argtypes = [u32p, u32p, u32p]
        L.orc_rht16_signs.restype = C.c_uint32
        L.orc_rht16_signs.argtypes = [C.c_uint64]
        L.orc_fwht.argtypes = [f32p, C.c_int]
        L.orc_rotate_rht16.argtypes = [f32p, C.c_uint32, f32p]
        L.orc_rotate_had32.argtypes = [f32p, f32p]
        L.orc_had32_norm.restype = C.c_float
        L.orc_tensor_amax.restype = C.c_float
        L.orc_tensor_amax.argtypes = [u16p, C.c_int64, C.c_int64, C.c_uint32, C.c_uint64]
        L.orc_nvfp4_quantize.restype = C.c_int
        L.orc_nvfp4_quantize.argtypes = [u16p, C.c_int64, C.c_int64, C.c_uint32, C.c_uint64,
                                         f32p, f32p, u8p, u8p, u8p, u8p, u8p, C.c_void_p]
        L.orc_nvfp4_quantize_f32.restype = C.c_int
        L.orc_nvfp4_quantize_f32.argtypes = [f32p, C.c_int64, C.c_int64, C.c_uint32, C.c_uint64,
                                             f32p, f32p, u8p, u8p, u8p]
        L.orc_nvfp4_quantize_rows.restype = C.c_int
        L.orc_nvfp4_quantize_rows.argtypes = [u16p, C.c_int64, C.c_int64, C.c_uint32, C.c_uint64,
                                              f32p, u8p, u8p, u8p]
        L.orc_nvfp4_quantize_at.restype = C.c_int
        L.orc_nvfp4_quantize_at.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int64, C.c_uint32,
                                            C.c_uint64, f32p, f32p, u8p, u8p, u8p]
        L.orc_nvfp4_quantize_rows_at.restype = C.c_int
        L.orc_nvfp4_quantize_rows_at.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int64,
                                                 C.c_uint32, C.c_uint64, f32p, u8p, u8p, u8p]
        L.orc_nvfp4_requantize_t_at.restype = C.c_int
        L.orc_nvfp4_requantize_t_at.argtypes = [u8p, u8p, C.c_float, C.c_int64, C.c_int64,
                                                C.c_int64, C.c_uint32, C.c_uint64, f32p, f32p,
                                                u8p, u8p, u8p]
        L.orc_nvfp4_requantize_t.restype = C.c_int
        L.orc_nvfp4_requantize_t.argtypes = [u8p, u8p, C.c_float, C.c_int64, C.c_int64,
                                             C.c_uint32, C.c_uint64, f32p, u8p, u8p, u8p]
        L.orc_mxfp4_quantize.restype = C.c_int
        L.orc_mxfp4_quantize.argtypes = [u16p, C.c_int64, C.c_int64, C.c_uint32,
                                         u8p, u8p, u8p, u8p, f32p, f32p]
        L.orc_nvfp4_simulate.restype = C.c_int
        L.orc_nvfp4_simulate.argtypes = [u16p, C.c_int64, C.c_int64, C.c_int, C.c_float, f32p]
        L.orc_dequantize.restype = C.c_int
        L.orc_dequantize.argtypes = [C.c_int, u8p, u8p, C.c_float, C.c_int64, C.c_int64,
                                     C.c_uint32, f32p]
        _lib = L
    return _lib


class _Debug(C.Structure):
    _fields_ = [(n, C.POINTER(C.c_float)) for n in
                ("t", "u", "p", "dpre6", "dpre4", "err6", "err4")]


def _p(a, ct):
    return None if a is None else a.ctypes.data_as(C.POINTER(ct))


# --------------------------------------------------------------- formats
def e2m1_encode(t):
    t = np.ascontiguousarray(np.asarray(t, dtype=np.float32)).ravel()
    out = np.empty(t.size, np.uint8)
    lib().orc_e2m1_encode_array(_p(t, C.c_float), t.size, _p(out, C.c_uint8))
    return out


def e2m1_decode(codes):
    table = np.array([lib().orc_e2m1_decode(c) for c in range(16)], np.float32)
    return table[np.asarray(codes, np.uint8) & 0xF]


def e4m3_encode(x):
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).ravel()
    out = np.empty(x.size, np.uint8)
    lib().orc_e4m3_encode_array(_p(x, C.c_float), x.size, _p(out, C.c_uint8))
    return out


def e4m3_decode(codes):
    table = np.array([lib().orc_e4m3_decode(c) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def ue8m0_decode(codes):
    table = np.array([lib().orc_ue8m0_decode(c) for c in range(256)], np.float32)
    return table[np.asarray(codes, np.uint8)]


def philox4x32_10(ctr, key):
    c = np.asarray(ctr, np.uint32).copy()
    k = np.asarray(key, np.uint32).copy()
    o = np.zeros(4, np.uint32)
    lib().orc_philox4x32_10(_p(c, C.c_uint32), _p(k, C.c_uint32), _p(o, C.c_uint32))
    return o


def rht16_signs(seed: int) -> int:
    return int(lib().orc_rht16_signs(C.c_uint64(seed & (2**64 - 1))))


def fwht(v):
    v = np.ascontiguousarray(np.asarray(v, np.float32)).copy()
    lib().orc_fwht(_p(v, C.c_float), v.size)
    return v


def rotate_rht16(x, signs):
    x = np.ascontiguousarray(np.asarray(x, np.float32))
    y = np.empty(16, np.float32)
    lib().orc_rotate_rht16(_p(x, C.c_float), signs, _p(y, C.c_float))
    return y


def rotate_had32(x):
    x = np.ascontiguousarray(np.asarray(x, np.float32))
    y = np.empty(32, np.float32)
    lib().orc_rotate_had32(_p(x, C.c_float), _p(y, C.c_float))
    return y


def had32_norm() -> np.float32:
    return np.float32(lib().orc_had32_norm())


# --------------------------------------------------------------- the path
def tensor_amax(x_bf16, flags=0, seed=0) -> float:
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    return float(lib().orc_tensor_amax(_p(x, C.c_uint16), rows, cols, flags,
                                       C.c_uint64(seed & (2**64 - 1))))


def nvfp4_quantize(x_bf16, flags=0, seed=0, amax=None, debug=False):
    """Returns dict(codes, scales, alpha, choice[, codes_t, scales_t][, dbg...])."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    two_d = bool(flags & BLOCK2D)
    srows = rows // 16 if two_d else rows
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((srows, cols // 16), np.uint8)
    choice = np.zeros((srows, cols // 16), np.uint8)
    alpha = np.zeros(1, np.float32)
    codes_t = scales_t = None
    if two_d and (flags & COLWISE):
        codes_t = np.zeros((cols, rows // 2), np.uint8)
        scales_t = np.zeros((cols // 16, rows // 16), np.uint8)
    amax_arr = None if amax is None else np.array([amax], np.float32)
    dbg = None
    arrays = {}
    if debug:
        n = rows * cols
        nb = scales.size
        arrays = dict(t=np.zeros(n, np.float32), u=np.zeros(n, np.float32),
                      p=np.zeros(n, np.float32), dpre6=np.zeros(nb, np.float32),
                      dpre4=np.zeros(nb, np.float32), err6=np.zeros(nb, np.float32),
                      err4=np.zeros(nb, np.float32))
        dbg = _Debug(**{k: _p(v, C.c_float) for k, v in arrays.items()})
    rc = lib().orc_nvfp4_quantize(
        _p(x, C.c_uint16), rows, cols, flags, C.c_uint64(seed & (2**64 - 1)),
        _p(amax_arr, C.c_float), _p(alpha, C.c_float), _p(codes, C.c_uint8),
        _p(scales, C.c_uint8), _p(choice, C.c_uint8), _p(codes_t, C.c_uint8),
        _p(scales_t, C.c_uint8), C.byref(dbg) if dbg is not None else None)
    if rc != 0:
        raise ValueError("oracle nvfp4_quantize rejected the arguments (%d)" % rc)
    out = dict(codes=codes, scales=scales, alpha=np.float32(alpha[0]), choice=choice)
    if codes_t is not None:
        out.update(codes_t=codes_t, scales_t=scales_t)
    for k, v in arrays.items():
        out["dbg_" + k] = v.reshape((rows, cols) if k in ("t", "u", "p") else scales.shape)
    return out


def nvfp4_quantize_at(x_bf16, row0, amax, flags=0, seed=0):
    """nvfp4_quantize (1D flags) of rows row0 .. row0 + len(x) - 1 of a larger
    tensor, given alone: SR and MS-EDEN draw with the whole tensor's element
    and block indices, and `amax` is the whole tensor's.  row0 = 0 is
    nvfp4_quantize(x, flags, seed, amax)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    choice = np.zeros((rows, cols // 16), np.uint8)
    alpha = np.zeros(1, np.float32)
    amax_arr = np.array([amax], np.float32)
    rc = lib().orc_nvfp4_quantize_at(
        _p(x, C.c_uint16), rows, cols, int(row0), flags, C.c_uint64(seed & (2**64 - 1)),
        _p(amax_arr, C.c_float), _p(alpha, C.c_float), _p(codes, C.c_uint8),
        _p(scales, C.c_uint8), _p(choice, C.c_uint8))
    if rc != 0:
        raise ValueError("oracle nvfp4_quantize_at rejected the arguments (%d)" % rc)
    return dict(codes=codes, scales=scales, alpha=np.float32(alpha[0]), choice=choice)


def nvfp4_quantize_f32(x_f32, flags=0, seed=0, amax=None):
    """NVFP4 of an fp32 tensor (1D flags); dict(codes, scales, alpha, choice)."""
    x = np.ascontiguousarray(x_f32, dtype=np.float32)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    choice = np.zeros((rows, cols // 16), np.uint8)
    alpha = np.zeros(1, np.float32)
    amax_arr = None if amax is None else np.array([amax], np.float32)
    rc = lib().orc_nvfp4_quantize_f32(
        _p(x, C.c_float), rows, cols, flags, C.c_uint64(seed & (2**64 - 1)),
        _p(amax_arr, C.c_float), _p(alpha, C.c_float), _p(codes, C.c_uint8),
        _p(scales, C.c_uint8), _p(choice, C.c_uint8))
    if rc != 0:
        raise ValueError("oracle nvfp4_quantize_f32 rejected the arguments (%d)" % rc)
    return dict(codes=codes, scales=scales, alpha=np.float32(alpha[0]), choice=choice)


def nvfp4_quantize_rows(x_bf16, flags=0, seed=0):
    """NVFP4 with one FP32 scale per row (1D flags); dict(codes, scales,
    alpha [rows], choice)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    choice = np.zeros((rows, cols // 16), np.uint8)
    alpha = np.zeros(max(rows, 1), np.float32)
    rc = lib().orc_nvfp4_quantize_rows(
        _p(x, C.c_uint16), rows, cols, flags, C.c_uint64(seed & (2**64 - 1)), _p(alpha, C.c_float),
        _p(codes, C.c_uint8), _p(scales, C.c_uint8), _p(choice, C.c_uint8))
    if rc != 0:
        raise ValueError("orc_nvfp4_quantize_rows failed: %d" % rc)
    return {"codes": codes, "scales": scales, "alpha": alpha[:rows], "choice": choice}


def nvfp4_quantize_rows_at(x_bf16, row0, flags=0, seed=0):
    """nvfp4_quantize_rows of rows row0 .. row0 + len(x) - 1 of a larger
    tensor, given alone (SR counters are the whole tensor's element indices)."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    codes = np.zeros((rows, cols // 2), np.uint8)
    scales = np.zeros((rows, cols // 16), np.uint8)
    choice = np.zeros((rows, cols // 16), np.uint8)
    alpha = np.zeros(max(rows, 1), np.float32)
    rc = lib().orc_nvfp4_quantize_rows_at(
        _p(x, C.c_uint16), rows, cols, int(row0), flags, C.c_uint64(seed & (2**64 - 1)),
        _p(alpha, C.c_float), _p(codes, C.c_uint8), _p(scales, C.c_uint8), _p(choice, C.c_uint8))
    if rc != 0:
        raise ValueError("orc_nvfp4_quantize_rows_at failed: %d" % rc)
    return {"codes": codes, "scales": scales, "alpha": alpha[:rows], "choice": choice}


def nvfp4_requantize_t(codes, scales, alpha, rows, cols, flags=0, seed=0):
    """NVFP4 (flags) of dequantize(X)^T for a 1D NVFP4 X [rows][cols]:
    dict(codes [cols][rows/2], scales [cols][rows/16], alpha, choice)."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    ct = np.zeros((cols, rows // 2), np.uint8)
    st = np.zeros((cols, rows // 16), np.uint8)
    ch = np.zeros((cols, rows // 16), np.uint8)
    a = np.zeros(1, np.float32)
    rc = lib().orc_nvfp4_requantize_t(
        _p(codes, C.c_uint8), _p(scales, C.c_uint8), C.c_float(alpha), rows, cols, flags,
        C.c_uint64(seed & (2**64 - 1)), _p(a, C.c_float), _p(ct, C.c_uint8), _p(st, C.c_uint8),
        _p(ch, C.c_uint8))
    if rc != 0:
        raise ValueError("oracle nvfp4_requantize_t rejected the arguments (%d)" % rc)
    return dict(codes=ct, scales=st, alpha=np.float32(a[0]), choice=ch)


def nvfp4_requantize_t_at(codes, scales, alpha, rows, cols, col0, amax, flags=0, seed=0):
    """nvfp4_requantize_t of columns col0 .. col0 + cols - 1 of a larger X
    (their codes [rows][cols/2] and scales [rows][cols/16]): output rows
    col0 .. of the whole transpose, given the whole output's amax; SR draws
    with the whole output's element indices."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    ct = np.zeros((cols, rows // 2), np.uint8)
    st = np.zeros((cols, rows // 16), np.uint8)
    ch = np.zeros((cols, rows // 16), np.uint8)
    a = np.zeros(1, np.float32)
    amax_arr = np.array([amax], np.float32)
    rc = lib().orc_nvfp4_requantize_t_at(
        _p(codes, C.c_uint8), _p(scales, C.c_uint8), C.c_float(alpha), rows, cols, int(col0),
        flags, C.c_uint64(seed & (2**64 - 1)), _p(amax_arr, C.c_float), _p(a, C.c_float),
        _p(ct, C.c_uint8), _p(st, C.c_uint8), _p(ch, C.c_uint8))
    if rc != 0:
        raise ValueError("oracle nvfp4_requantize_t_at rejected the arguments (%d)" % rc)
    return dict(codes=ct, scales=st, alpha=np.float32(a[0]), choice=ch)


def mxfp4_quantize(x_bf16, flags=ROWWISE | COLWISE, debug=False):
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    out = {}
    cr = sr = cc = sc = tr = tc = None
    if flags & ROWWISE:
        cr = np.zeros((rows, cols // 2), np.uint8)
        sr = np.zeros((rows, cols // 32), np.uint8)
        if debug:
            tr = np.zeros((rows, cols), np.float32)
    if flags & COLWISE:
        cc = np.zeros((cols, rows // 2), np.uint8)
        sc = np.zeros((cols, rows // 32), np.uint8)
        if debug:
            tc = np.zeros((cols, rows), np.float32)
    rc = lib().orc_mxfp4_quantize(_p(x, C.c_uint16), rows, cols, flags,
                                  _p(cr, C.c_uint8), _p(sr, C.c_uint8),
                                  _p(cc, C.c_uint8), _p(sc, C.c_uint8),
                                  _p(tr, C.c_float), _p(tc, C.c_float))
    if rc != 0:
        raise ValueError("oracle mxfp4_quantize rejected the arguments (%d)" % rc)
    if flags & ROWWISE:
        out.update(codes_r=cr, scales_r=sr)
    if flags & COLWISE:
        out.update(codes_c=cc, scales_c=sc)
    if debug:
        out.update(t_r=tr, t_c=tc)
    return out


SIM_NVFP4, SIM_SCALE_HP, SIM_VALUE_HP, SIM_THRESHOLD = 0, 1, 2, 3


def nvfp4_simulate(x_bf16, mode=SIM_NVFP4, thr=0.0):
    """RTN6 quantize-then-dequantize of x with one error source switched off
    (the simulated quantization of the 4/6 paper's Fig. 2); fp32 [rows][cols]."""
    x = np.ascontiguousarray(x_bf16, dtype=np.uint16)
    rows, cols = x.shape
    out = np.zeros((rows, cols), np.float32)
    rc = lib().orc_nvfp4_simulate(_p(x, C.c_uint16), rows, cols, mode, C.c_float(thr),
                                  _p(out, C.c_float))
    if rc != 0:
        raise ValueError("orc_nvfp4_simulate failed: %d" % rc)
    return out


def dequantize(fmt, codes, scales, alpha, rows, cols, flags=0):
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint8)
    out = np.zeros((rows, cols), np.float32)
    rc = lib().orc_dequantize(fmt, _p(codes, C.c_uint8), _p(scales, C.c_uint8),
                              C.c_float(alpha), rows, cols, flags, _p(out, C.c_float))
    if rc != 0:
        raise ValueError("oracle dequantize rejected the arguments (%d)" % rc)
    return out


def mxfp4_gemm(a_codes, a_scales, bt_codes, bt_scales, M, N, K):
    """C = A B for MXFP4 operands, the consumer of the quantized tensors
    (NVIDIA NVFP4 article sec. 1 and 5: MXFP4 values with a power-of-two
    scale per 32; the block-scaled matrix product is the next step of the
    path).  A is [M][K] row-wise (codes [M][K/2], scales [M][K/32]); B is
    given as its transpose [N][K] in the same layout (the column-wise output
    of the MXFP4 quantizer).  The dequantized values are exact in fp32; the
    product is a float64 matmul.  Returns float64 [M][N]."""
    A = dequantize(1, a_codes, a_scales, 0.0, M, K).astype(np.float64)
    BT = dequantize(1, bt_codes, bt_scales, 0.0, N, K).astype(np.float64)
    return A @ BT.T


def unpack_codes(packed):
    """[r][n/2] bytes -> [r][n] 4-bit codes (low nibble = even element)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out
