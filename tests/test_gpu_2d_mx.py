"""GPU parity of the 16x16-tile NVFP4 path and of MXFP4 (row- and
column-wise, with and without the 32-point Hadamard) against the CPU oracle.
Without rotation both sides run the same fp32 operations, so every code and
scale must match bit for bit.  With the 32-point Hadamard the GPU sums on
the matrix cores in another fp32 order than the oracle's butterfly, so codes
and scales may differ only next to a rounding boundary or a power of two
(see rotated_tolerance.py), at most 1e-5 of the elements, with the same
dequantized error."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from rotated_tolerance import check_mx_outputs

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_reduce_amd as fp4  # noqa: E402


def dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).cuda()


def host(t):
    return t.cpu().numpy()


def same(g, w, what):
    g = host(g)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    assert bad.size == 0, "%s differs at %d places, first %s: gpu %s oracle %s" % (
        what, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


# ------------------------------------------------------------ NVFP4 2D
@pytest.mark.parametrize("flags", [fp4.BLOCK2D, fp4.BLOCK2D | fp4.FOUR_OVER_SIX,
                                   fp4.BLOCK2D | fp4.COLWISE,
                                   fp4.BLOCK2D | fp4.FOUR_OVER_SIX | fp4.COLWISE])
@pytest.mark.parametrize("shape", [(16, 16), (80, 400), (272, 1040), (64, 4096)])
def test_2d_parity(shape, flags):
    x = S.gen("c3", *shape)
    print("2d case", shape, flags, flush=True)
    got = fp4.nvfp4_quantize(dev(x), flags, want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize(x, flags)
    same(got["codes"], want["codes"], "codes")
    same(got["scales"], want["scales"], "scales")
    assert host(got["alpha"])[0] == want["alpha"]
    if flags & fp4.FOUR_OVER_SIX:
        same(got["choice"], want["choice"], "choice")
    if flags & fp4.COLWISE:
        same(got["codes_t"], want["codes_t"], "codes_t")
        same(got["scales_t"], want["scales_t"], "scales_t")


def test_2d_special_values_and_dequant():
    x = S.special_values_tensor(64, 96, seed=11)
    f = fp4.BLOCK2D | fp4.FOUR_OVER_SIX | fp4.COLWISE
    got = fp4.nvfp4_quantize(dev(x), f)
    want = O.nvfp4_quantize(x, f)
    same(got["codes"], want["codes"], "codes")
    same(got["codes_t"], want["codes_t"], "codes_t")
    d = fp4.fp4_dequantize(fp4.FORMAT_NVFP4, got["codes"], got["scales"], got["alpha"], 64, 96,
                           fp4.BLOCK2D)
    same(d, O.dequantize(0, want["codes"], want["scales"], want["alpha"], 64, 96, O.BLOCK2D),
         "dequant")


def test_2d_c3_full():
    x = S.gen("c3")
    f = fp4.BLOCK2D | fp4.FOUR_OVER_SIX | fp4.COLWISE
    got = fp4.nvfp4_quantize(dev(x), f, want_choice=True)
    want = O.nvfp4_quantize(x, f)
    for k in ("codes", "scales", "choice", "codes_t", "scales_t"):
        same(got[k], want[k], k)


# ------------------------------------------------------------ MXFP4
MX_FLAGS = [fp4.ROWWISE, fp4.COLWISE, fp4.ROWWISE | fp4.COLWISE,
            fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE, fp4.HAD32 | fp4.COLWISE,
            fp4.HAD32 | fp4.ROWWISE]


@pytest.mark.parametrize("flags", MX_FLAGS)
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (160, 4128), (320, 256)])
def test_mx_parity(shape, flags):
    x = S.gen("c5", *shape)
    print("mx case", shape, flags, flush=True)
    got = fp4.mxfp4_quantize(dev(x), flags)
    torch.cuda.synchronize()
    want = O.mxfp4_quantize(x, flags, debug=bool(flags & O.HAD32))
    mx_compare(x, flags, got, want, "mx %s" % (shape,))


def mx_compare(x, flags, got, want, what):
    if flags & fp4.HAD32:
        # the rotated-path rule (rotated_tolerance.py) needs the oracle's
        # pre-rounding values: `want` must come from mxfp4_quantize(debug=True)
        print(what, check_mx_outputs(x, flags, got, want, host, what), flush=True)
    else:
        for k in want:
            same(got[k], want[k], k)


@pytest.mark.parametrize("flags", [fp4.ROWWISE, fp4.HAD32 | fp4.ROWWISE])
@pytest.mark.parametrize("shape", [(1, 32), (45, 96), (200, 4128)])
def test_mx_rowwise_ragged_rows(shape, flags):
    """Row-wise output alone needs no row multiple: partial row blocks."""
    x = S.gen("c5", *shape)
    got = fp4.mxfp4_quantize(dev(x), flags)
    torch.cuda.synchronize()
    want = O.mxfp4_quantize(x, flags, debug=bool(flags & O.HAD32))
    mx_compare(x, flags, got, want, "ragged %s" % (shape,))


def test_mx_special_values_subnormal_groups():
    x = S.special_values_tensor(64, 128, seed=5)
    x[:32, :32] = np.arange(1, 0x20 + 1, dtype=np.uint16)[None, :]    # subnormal-only group
    x[32:64, 96:128] = 0x0001                                          # smallest subnormal
    for flags in (fp4.ROWWISE | fp4.COLWISE, fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE):
        got = fp4.mxfp4_quantize(dev(x), flags)
        want = O.mxfp4_quantize(x, flags, debug=bool(flags & O.HAD32))
        mx_compare(x, flags, got, want, "special")


def test_mx_dequant_both_orientations():
    x = S.gen("c5", 64, 96)
    f = fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE
    got = fp4.mxfp4_quantize(dev(x), f)
    want = O.mxfp4_quantize(x, f, debug=True)
    dr = fp4.fp4_dequantize(fp4.FORMAT_MXFP4, got["codes_r"], got["scales_r"], None, 64, 96)
    dc = fp4.fp4_dequantize(fp4.FORMAT_MXFP4, got["codes_c"], got["scales_c"], None, 96, 64)
    # the decode is exact: compare it with the oracle's decode of the GPU's own codes
    same(dr, O.dequantize(1, host(got["codes_r"]), host(got["scales_r"]), 0.0, 64, 96), "dequant rows")
    same(dc, O.dequantize(1, host(got["codes_c"]), host(got["scales_c"]), 0.0, 96, 64), "dequant cols")
    mx_compare(x, f, got, want, "dequant case")


def test_mx_c5_full():
    x = S.gen("c5")
    f = fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE
    got = fp4.mxfp4_quantize(dev(x), f)
    torch.cuda.synchronize()
    want = O.mxfp4_quantize(x, f, debug=True)
    mx_compare(x, f, got, want, "c5 full")
