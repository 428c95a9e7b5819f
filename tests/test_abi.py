"""C-ABI checks that need no GPU: the library loads, exports every function
include/fp4q.h declares, and rejects bad arguments before any HIP call
(so these calls never touch a device; fake pointers are never dereferenced)."""
import os
import re

import pytest

import block_scaled_fp4_reduce_amd as fp4

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "fp4q.h")

OK, E_NULL, E_SHAPE, E_ALIGN, E_FLAGS, E_WS = 0, -1, -2, -3, -4, -5
P = 0x10000          # a 16-byte-aligned fake device address: never used
Q = 0x10008          # 8-byte aligned only
F4 = 0x20004         # 4-byte aligned float pointer


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fp4.LIB_PATH):
        from block_scaled_fp4_reduce_amd import build
        build.build()
    return fp4.lib()


def declared_functions():
    text = open(HDR).read()
    return sorted(set(re.findall(r"^\s*(?:int|size_t|const char\*)\s+(\w+)\s*\(", text, re.M)))


def test_exports_every_declared_function(L):
    names = declared_functions()
    assert set(names) == set(fp4.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_status_strings_and_version(L):
    assert L.fp4_abi_version() == 2
    for code in fp4.STATUS:
        assert L.fp4_status_str(code)
    assert L.fp4_status_str(E_SHAPE) != L.fp4_status_str(E_FLAGS)


def test_workspace_bytes(L):
    assert L.fp4_workspace_bytes(8192, 4096, 1) >= 4
    assert L.fp4_workspace_bytes(16384, 8192, fp4.HAD32 | fp4.ROWWISE) == 0


def nvq(L, x=P, rows=32, cols=64, flags=0, amax=None, alpha=F4, codes=P, scales=P, choice=None,
        ct=None, st=None, ws=P, wsb=1 << 20):
    return L.nvfp4_quantize(x, rows, cols, flags, 0, amax, alpha, codes, scales, choice, ct, st,
                            ws, wsb, None)


def test_nvfp4_rejects(L):
    assert nvq(L, x=None) == E_NULL
    assert nvq(L, codes=None) == E_NULL
    assert nvq(L, alpha=None) == E_NULL
    assert nvq(L, ws=None) == E_NULL                       # amax computed -> needs workspace
    assert nvq(L, cols=40) == E_SHAPE                      # not a multiple of 16
    assert nvq(L, rows=-1) == E_SHAPE
    assert nvq(L, rows=1 << 21, cols=1 << 20) == E_SHAPE   # 2^41 elements
    assert nvq(L, rows=24, flags=fp4.BLOCK2D) == E_SHAPE   # 2D needs rows % 16
    assert nvq(L, flags=fp4.SR | fp4.FOUR_OVER_SIX) == E_FLAGS
    assert nvq(L, flags=fp4.BLOCK2D | fp4.SR) == E_FLAGS
    assert nvq(L, flags=fp4.BLOCK2D | fp4.RHT16) == E_FLAGS
    assert nvq(L, flags=fp4.HAD32) == E_FLAGS
    assert nvq(L, flags=fp4.COLWISE) == E_FLAGS            # transposed output needs 2D
    assert nvq(L, flags=1 << 9) == E_FLAGS
    assert nvq(L, flags=fp4.MSEDEN) == E_FLAGS                 # MS-EDEN needs RHT16
    for f in (fp4.SR, fp4.FOUR_OVER_SIX, fp4.BLOCK2D):
        assert nvq(L, flags=fp4.MSEDEN | fp4.RHT16 | f) == E_FLAGS
    assert nvq(L, x=P + 2) == E_ALIGN
    assert nvq(L, codes=Q) == E_ALIGN
    assert nvq(L, alpha=F4 + 1) == E_ALIGN
    assert nvq(L, wsb=16) == E_WS
    # 2D with transposed output but missing buffers
    assert nvq(L, flags=fp4.BLOCK2D | fp4.COLWISE) == E_NULL


def test_amax_rejects(L):
    assert L.fp4_tensor_amax(P, 32, 64, 0, 0, None, P, 4096, None) == E_NULL
    assert L.fp4_tensor_amax(P, 32, 64, 0, 0, F4, None, 4096, None) == E_NULL
    assert L.fp4_tensor_amax(P, 32, 60, 0, 0, F4, P, 4096, None) == E_SHAPE
    assert L.fp4_tensor_amax(P, 32, 64, fp4.HAD32, 0, F4, P, 4096, None) == E_FLAGS
    assert L.fp4_tensor_amax(P + 4, 32, 64, 0, 0, F4, P, 4096, None) == E_ALIGN
    assert L.fp4_tensor_amax(P, 32, 64, 0, 0, F4, P, 8, None) == E_WS


def rq(L, codes=P, scales=P, alpha=F4, rows=32, cols=64, flags=0, amax=None, alpha_out=F4, ct=P,
       st=P, choice=None, ws=P, wsb=1 << 20):
    return L.nvfp4_requantize_t(codes, scales, alpha, rows, cols, flags, 0, amax, alpha_out, ct, st,
                                choice, ws, wsb, None)


def test_requant_rejects(L):
    assert rq(L, codes=None) == E_NULL
    assert rq(L, scales=None) == E_NULL
    assert rq(L, alpha=None) == E_NULL
    assert rq(L, alpha_out=None) == E_NULL
    assert rq(L, ct=None) == E_NULL
    assert rq(L, st=None) == E_NULL
    assert rq(L, ws=None) == E_NULL                         # amax computed -> needs workspace
    assert rq(L, rows=24) == E_SHAPE                        # rows % 16
    assert rq(L, cols=40) == E_SHAPE                        # cols % 16
    assert rq(L, rows=-16) == E_SHAPE
    assert rq(L, rows=1 << 21, cols=1 << 20) == E_SHAPE     # 2^41 elements
    for f in (fp4.BLOCK2D, fp4.COLWISE, fp4.ROWWISE, fp4.HAD32, fp4.SR | fp4.FOUR_OVER_SIX, 1 << 9):
        assert rq(L, flags=f) == E_FLAGS, f
    assert rq(L, codes=Q) == E_ALIGN
    assert rq(L, ct=Q) == E_ALIGN
    assert rq(L, alpha=F4 + 1) == E_ALIGN
    assert rq(L, amax=F4 + 2) == E_ALIGN
    assert rq(L, wsb=16) == E_WS


def test_rows_rejects(L):
    def rows(x=P, r=32, c=64, flags=0, alpha=F4, codes=P, scales=P):
        return L.nvfp4_quantize_rows(x, r, c, flags, 0, alpha, codes, scales, None, None)
    assert rows(x=None) == E_NULL
    assert rows(alpha=None) == E_NULL
    assert rows(codes=None) == E_NULL
    assert rows(scales=None) == E_NULL
    assert rows(c=40) == E_SHAPE
    assert rows(r=-1) == E_SHAPE
    for f in (fp4.BLOCK2D, fp4.COLWISE, fp4.HAD32, fp4.SR | fp4.FOUR_OVER_SIX, 1 << 9):
        assert rows(flags=f) == E_FLAGS, f
    assert rows(x=P + 2) == E_ALIGN
    assert rows(codes=Q) == E_ALIGN
    assert rows(alpha=F4 + 1) == E_ALIGN
    assert L.nvfp4_quantize_rows(None, 0, 64, 0, 0, None, None, None, None, None) == OK


def test_gemm_rejects(L):
    def gm(a=P, sa=F4, b=P, sb=F4, M=128, N=128, K=256, c=F4):
        return L.mxfp4_gemm(a, sa, b, sb, M, N, K, c, None)
    assert gm(a=None) == E_NULL
    assert gm(sb=None) == E_NULL
    assert gm(c=None) == E_NULL
    assert gm(K=192) == E_SHAPE                  # K % 128
    assert gm(M=-1) == E_SHAPE
    assert gm(a=Q) == E_ALIGN
    assert gm(sa=F4 + 1) == E_ALIGN
    assert gm(M=0, a=None, sa=None, c=None) == OK  # empty product


def test_mx_rejects(L):
    f = fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE
    assert L.mxfp4_quantize(None, 64, 64, f, P, P, P, P, None) == E_NULL
    assert L.mxfp4_quantize(P, 64, 64, f, P, P, None, P, None) == E_NULL
    assert L.mxfp4_quantize(P, 64, 48, f, P, P, P, P, None) == E_SHAPE     # cols % 32
    assert L.mxfp4_quantize(P, 48, 64, f, P, P, P, P, None) == E_SHAPE     # rows % 32 (col-wise)
    assert L.mxfp4_quantize(P, 64, 64, fp4.HAD32, P, P, P, P, None) == E_FLAGS  # no orientation
    assert L.mxfp4_quantize(P, 64, 64, f | fp4.SR, P, P, P, P, None) == E_FLAGS
    assert L.mxfp4_quantize(P, 64, 64, f, Q, P, P, P, None) == E_ALIGN


def test_dequant_rejects(L):
    assert L.fp4_dequantize(2, P, P, F4, 16, 32, 0, P, None) == E_FLAGS
    assert L.fp4_dequantize(0, P, P, None, 16, 32, 0, P, None) == E_NULL
    assert L.fp4_dequantize(0, P, P, F4, 16, 40, 0, P, None) == E_SHAPE
    assert L.fp4_dequantize(0, P, P, F4, 24, 32, fp4.BLOCK2D, P, None) == E_SHAPE
    assert L.fp4_dequantize(1, P, P, None, 16, 48, 0, P, None) == E_SHAPE
    assert L.fp4_dequantize(1, P, P, None, 16, 64, fp4.BLOCK2D, P, None) == E_FLAGS
    assert L.fp4_dequantize(0, P, P, F4, 16, 32, 0, Q, None) == E_ALIGN


def test_empty_tensors_need_no_buffers(L):
    # zero-sized MX and dequant calls succeed without launching anything
    assert L.mxfp4_quantize(None, 0, 64, fp4.ROWWISE, None, None, None, None, None) == OK
    assert L.fp4_dequantize(1, None, None, None, 0, 64, 0, None, None) == OK


def test_noalloc_rejects_before_any_hip_call(L):
    def nq(x=P, rows=32, cols=64, flags=0, amax=None, alpha=F4, codes=P, scales=P):
        return L.nvfp4_quantize_noalloc(x, rows, cols, flags, 0, amax, alpha, codes, scales, None,
                                        None, None, None)
    assert nq(x=None) == E_NULL
    assert nq(alpha=None) == E_NULL
    assert nq(cols=40) == E_SHAPE
    assert nq(flags=fp4.SR | fp4.FOUR_OVER_SIX) == E_FLAGS
    assert nq(codes=Q) == E_ALIGN
    assert nq(amax=F4, x=None) == E_NULL          # with an amax it is nvfp4_quantize's check
