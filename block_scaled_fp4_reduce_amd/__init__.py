"""Block-scaled FP4 quantization (NVFP4 with Four Over Six, RHT16 + SR, 16x16
tiles; MXFP4 with a 32-point Hadamard) for AMD MI355X.

Thin ctypes binding over ``libfp4q.so`` (see ``include/fp4q.h``).  Every
step of the quantization runs in the library's HIP kernels; this module only
allocates torch device buffers, checks dtypes and forwards pointers and the
current stream.  There is no fallback: without the built library, or without
a GPU, the calls raise.

Two layers:
  * ``lib()`` -- the raw C functions (``nvfp4_quantize`` etc.) taking
    integers for device pointers and the stream, returning an int status.
  * tensor helpers with the same names taking/returning torch tensors.
"""
from __future__ import annotations

import ctypes as C
import os

FOUR_OVER_SIX = 1 << 0
SR = 1 << 1
RHT16 = 1 << 2
BLOCK2D = 1 << 3
HAD32 = 1 << 4
ROWWISE = 1 << 5
COLWISE = 1 << 6
MSEDEN = 1 << 7
RTN6 = 0

FORMAT_NVFP4 = 0
FORMAT_MXFP4 = 1

STATUS = {0: "FP4_OK", -1: "FP4_E_NULL", -2: "FP4_E_SHAPE", -3: "FP4_E_ALIGN",
          -4: "FP4_E_FLAGS", -5: "FP4_E_WORKSPACE", -6: "FP4_E_HIP"}

EXPORTS = ("fp4_workspace_bytes", "fp4_tensor_amax", "nvfp4_quantize", "nvfp4_quantize_noalloc",
           "nvfp4_quantize_rows",
           "nvfp4_requantize_t", "mxfp4_quantize", "mxfp4_gemm", "fp4_dequantize",
           "fp4_status_str", "fp4_abi_version")

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp4q.so")
_lib = None


class Fp4Error(RuntimeError):
    def __init__(self, fn, status):
        super().__init__("%s failed: %s (%d): %s" % (
            fn, STATUS.get(status, "?"), status, lib().fp4_status_str(status).decode()))
        self.status = status


def lib():
    """Load libfp4q.so (built in-tree by ``__graft_entry__.build()``)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libfp4q.so is not built: run __graft_entry__.build() "
                               "(python -m block_scaled_fp4_reduce_amd.build)")
        L = C.CDLL(LIB_PATH)
        vp, i64, u32, u64, sz = C.c_void_p, C.c_int64, C.c_uint32, C.c_uint64, C.c_size_t
        L.fp4_workspace_bytes.restype = sz
        L.fp4_workspace_bytes.argtypes = [i64, i64, u32]
        L.fp4_tensor_amax.restype = C.c_int
        L.fp4_tensor_amax.argtypes = [vp, i64, i64, u32, u64, vp, vp, sz, vp]
        L.nvfp4_quantize.restype = C.c_int
        L.nvfp4_quantize.argtypes = [vp, i64, i64, u32, u64, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
        L.nvfp4_quantize_noalloc.restype = C.c_int
        L.nvfp4_quantize_noalloc.argtypes = [vp, i64, i64, u32, u64, vp, vp, vp, vp, vp, vp, vp, vp]
        L.nvfp4_quantize_rows.restype = C.c_int
        L.nvfp4_quantize_rows.argtypes = [vp, i64, i64, u32, u64, vp, vp, vp, vp, vp]
        L.nvfp4_requantize_t.restype = C.c_int
        L.nvfp4_requantize_t.argtypes = [vp, vp, vp, i64, i64, u32, u64, vp, vp, vp, vp, vp, vp, sz,
                                         vp]
        L.mxfp4_quantize.restype = C.c_int
        L.mxfp4_quantize.argtypes = [vp, i64, i64, u32, vp, vp, vp, vp, vp]
        L.mxfp4_gemm.restype = C.c_int
        L.mxfp4_gemm.argtypes = [vp, vp, vp, vp, i64, i64, i64, vp, vp]
        L.fp4_dequantize.restype = C.c_int
        L.fp4_dequantize.argtypes = [C.c_int, vp, vp, vp, i64, i64, u32, vp, vp]
        L.fp4_status_str.restype = C.c_char_p
        L.fp4_status_str.argtypes = [C.c_int]
        L.fp4_abi_version.restype = C.c_int
        L.fp4_abi_version.argtypes = []
        _lib = L
    return _lib


# ------------------------------------------------------------------ helpers
def _torch():
    import torch
    return torch


def _check(fn, rc):
    if rc != 0:
        raise Fp4Error(fn, rc)


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    torch = _torch()
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _as_bits(x):
    torch = _torch()
    if x.dtype == torch.bfloat16:
        x = x.view(torch.int16)
    if x.dtype not in (torch.int16, torch.uint16):
        raise TypeError("expected a bfloat16 (or 16-bit bit-pattern) tensor, got %s" % x.dtype)
    if x.dim() != 2 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("expected a contiguous 2-D tensor on the GPU")
    return x


def fp4_workspace_bytes(rows, cols, flags=0):
    return int(lib().fp4_workspace_bytes(rows, cols, flags))


def _workspace(rows, cols, flags, device, ws=None):
    torch = _torch()
    need = fp4_workspace_bytes(rows, cols, flags)
    if ws is None:
        ws = torch.empty(max(need, 4), dtype=torch.uint8, device=device)
    return ws


# ------------------------------------------------------------------ tensor API
def fp4_tensor_amax(x, flags=0, seed=0, out=None, ws=None, stream=None):
    """Largest magnitude of x (after RHT16 when asked); a 1-element float tensor."""
    torch = _torch()
    xb = _as_bits(x)
    rows, cols = xb.shape
    out = torch.empty(1, dtype=torch.float32, device=x.device) if out is None else out
    ws = _workspace(rows, cols, flags, x.device, ws)
    _check("fp4_tensor_amax", lib().fp4_tensor_amax(
        xb.data_ptr(), rows, cols, flags, seed & (2**64 - 1), out.data_ptr(), ws.data_ptr(),
        ws.numel(), _stream(stream)))
    return out


def nvfp4_quantize(x, flags=0, seed=0, amax=None, want_choice=False, ws=None, stream=None,
                   out=None):
    """NVFP4 quantization.  Returns a dict with ``codes`` [rows][cols/2] uint8,
    ``scales`` (E4M3 bytes), ``alpha`` (1 float), optional ``choice`` and, for
    BLOCK2D|COLWISE, ``codes_t``/``scales_t``.  ``out`` may supply these
    buffers (same keys) to avoid allocation."""
    torch = _torch()
    xb = _as_bits(x)
    rows, cols = xb.shape
    dev = x.device
    two_d = bool(flags & BLOCK2D)
    want_t = two_d and bool(flags & COLWISE)
    srows = rows // 16 if two_d else rows
    o = dict(out or {})
    u8 = torch.uint8
    if "codes" not in o:
        o["codes"] = torch.empty((rows, cols // 2), dtype=u8, device=dev)
    if "scales" not in o:
        o["scales"] = torch.empty((srows, cols // 16), dtype=u8, device=dev)
    if "alpha" not in o:
        o["alpha"] = torch.empty(1, dtype=torch.float32, device=dev)
    if want_choice and "choice" not in o:
        o["choice"] = torch.empty((srows, cols // 16), dtype=u8, device=dev)
    if want_t:
        o.setdefault("codes_t", torch.empty((cols, rows // 2), dtype=u8, device=dev))
        o.setdefault("scales_t", torch.empty((cols // 16, rows // 16), dtype=u8, device=dev))
    if amax is None:
        ws = _workspace(rows, cols, flags, dev, ws)
    _check("nvfp4_quantize", lib().nvfp4_quantize(
        xb.data_ptr(), rows, cols, flags, seed & (2**64 - 1), _ptr(amax), o["alpha"].data_ptr(),
        o["codes"].data_ptr(), o["scales"].data_ptr(), _ptr(o.get("choice")),
        _ptr(o.get("codes_t")), _ptr(o.get("scales_t")), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))
    return o


def nvfp4_quantize_noalloc(x, flags=0, seed=0, amax=None, out=None, stream=None):
    """nvfp4_quantize without a workspace: the library keeps the amax pass's
    partial maxima in its own fixed device array.  ``out`` must hold every
    output buffer (``codes``, ``scales``, ``alpha``, optional ``choice``,
    ``codes_t``/``scales_t`` for BLOCK2D|COLWISE): this call allocates
    nothing.  Calls overlapping on one device race (see include/fp4q.h)."""
    xb = _as_bits(x)
    rows, cols = xb.shape
    o = out
    _check("nvfp4_quantize_noalloc", lib().nvfp4_quantize_noalloc(
        xb.data_ptr(), rows, cols, flags, seed & (2**64 - 1), _ptr(amax), o["alpha"].data_ptr(),
        o["codes"].data_ptr(), o["scales"].data_ptr(), _ptr(o.get("choice")),
        _ptr(o.get("codes_t")), _ptr(o.get("scales_t")), _stream(stream)))
    return o


def nvfp4_quantize_rows(x, flags=0, seed=0, want_choice=False, stream=None, out=None):
    """NVFP4 with one FP32 scale per row, in one read of x.  Returns a dict
    with ``codes`` [rows][cols/2], ``scales`` [rows][cols/16], ``alpha``
    [rows] (float32) and, when asked, ``choice``."""
    torch = _torch()
    xb = _as_bits(x)
    rows, cols = xb.shape
    dev = x.device
    o = dict(out or {})
    u8 = torch.uint8
    o.setdefault("codes", torch.empty((rows, cols // 2), dtype=u8, device=dev))
    o.setdefault("scales", torch.empty((rows, cols // 16), dtype=u8, device=dev))
    o.setdefault("alpha", torch.empty(max(rows, 1), dtype=torch.float32, device=dev))
    if want_choice:
        o.setdefault("choice", torch.empty((rows, cols // 16), dtype=u8, device=dev))
    _check("nvfp4_quantize_rows", lib().nvfp4_quantize_rows(
        xb.data_ptr(), rows, cols, flags, seed & (2**64 - 1), o["alpha"].data_ptr(),
        o["codes"].data_ptr(), o["scales"].data_ptr(), _ptr(o.get("choice")), _stream(stream)))
    return o


def nvfp4_requantize_t(codes, scales, alpha, flags=0, seed=0, amax=None, want_choice=False,
                       ws=None, stream=None, out=None):
    """NVFP4 of dequantize(X)^T for a 1D NVFP4 tensor X given as ``codes``
    [rows][cols/2], ``scales`` [rows][cols/16] and ``alpha`` (1 float).
    Returns a dict with ``codes`` [cols][rows/2], ``scales`` [cols][rows/16],
    ``alpha`` and, when asked, ``choice``; ``out`` may supply these buffers.
    ``amax`` (1 float) skips the amax pass."""
    torch = _torch()
    for t in (codes, scales, alpha):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("expected contiguous GPU tensors")
    if codes.dtype != torch.uint8 or scales.dtype != torch.uint8 or alpha.dtype != torch.float32:
        raise TypeError("expected uint8 codes/scales and a float32 alpha")
    rows, cols = codes.shape[0], codes.shape[1] * 2
    if tuple(scales.shape) != (rows, cols // 16):
        raise ValueError("scales must be [rows][cols/16]")
    dev = codes.device
    o = dict(out or {})
    u8 = torch.uint8
    o.setdefault("codes", torch.empty((cols, rows // 2), dtype=u8, device=dev))
    o.setdefault("scales", torch.empty((cols, rows // 16), dtype=u8, device=dev))
    o.setdefault("alpha", torch.empty(1, dtype=torch.float32, device=dev))
    if want_choice:
        o.setdefault("choice", torch.empty((cols, rows // 16), dtype=u8, device=dev))
    if amax is None:
        ws = _workspace(rows, cols, flags, dev, ws)
    _check("nvfp4_requantize_t", lib().nvfp4_requantize_t(
        codes.data_ptr(), scales.data_ptr(), alpha.data_ptr(), rows, cols, flags,
        seed & (2**64 - 1), _ptr(amax), o["alpha"].data_ptr(), o["codes"].data_ptr(),
        o["scales"].data_ptr(), _ptr(o.get("choice")), _ptr(ws),
        0 if ws is None else ws.numel(), _stream(stream)))
    return o


def mxfp4_quantize(x, flags=HAD32 | ROWWISE | COLWISE, stream=None, out=None):
    """MXFP4 quantization; returns ``codes_r``/``scales_r`` and/or
    ``codes_c``/``scales_c`` (column-wise = row-wise of the transpose)."""
    torch = _torch()
    xb = _as_bits(x)
    rows, cols = xb.shape
    dev = x.device
    o = dict(out or {})
    u8 = torch.uint8
    if flags & ROWWISE:
        o.setdefault("codes_r", torch.empty((rows, cols // 2), dtype=u8, device=dev))
        o.setdefault("scales_r", torch.empty((rows, cols // 32), dtype=u8, device=dev))
    if flags & COLWISE:
        o.setdefault("codes_c", torch.empty((cols, rows // 2), dtype=u8, device=dev))
        o.setdefault("scales_c", torch.empty((cols, rows // 32), dtype=u8, device=dev))
    _check("mxfp4_quantize", lib().mxfp4_quantize(
        xb.data_ptr(), rows, cols, flags, _ptr(o.get("codes_r")), _ptr(o.get("scales_r")),
        _ptr(o.get("codes_c")), _ptr(o.get("scales_c")), _stream(stream)))
    return o


def mxfp4_gemm(a_codes, a_scales, bt_codes, bt_scales, out=None, stream=None):
    """C = A B (fp32 [M][N]) from row-wise MXFP4 A (codes [M][K/2], scales
    [M][K/32]) and B^T in the same layout (codes [N][K/2], scales [N][K/32])."""
    torch = _torch()
    M, N, K = a_codes.shape[0], bt_codes.shape[0], a_codes.shape[1] * 2
    if bt_codes.shape[1] * 2 != K:
        raise ValueError("A and B^T disagree on K")
    for t in (a_codes, a_scales, bt_codes, bt_scales):
        if t.dtype != torch.uint8 or not t.is_cuda or not t.is_contiguous():
            raise ValueError("expected contiguous uint8 GPU tensors")
    out = torch.empty((M, N), dtype=torch.float32, device=a_codes.device) if out is None else out
    _check("mxfp4_gemm", lib().mxfp4_gemm(
        a_codes.data_ptr(), a_scales.data_ptr(), bt_codes.data_ptr(), bt_scales.data_ptr(), M, N, K,
        out.data_ptr(), _stream(stream)))
    return out


def fp4_dequantize(fmt, codes, scales, alpha, rows, cols, flags=0, out=None, stream=None):
    """Decode to fp32 [rows][cols]."""
    torch = _torch()
    out = torch.empty((rows, cols), dtype=torch.float32, device=codes.device) if out is None else out
    _check("fp4_dequantize", lib().fp4_dequantize(
        fmt, codes.data_ptr(), scales.data_ptr(), _ptr(alpha), rows, cols, flags,
        out.data_ptr(), _stream(stream)))
    return out
