"""GPU parity of the requantization for the transposed operand
(NVFP4 of dequantize(X)^T) against the CPU oracle, bit for bit.

The fp32 dequantized values are identical on both sides (one fp32 product
q * (alpha * Delta)), the 16-point rotation runs the same fp32 butterfly and
SR uses the same Philox counter, so codes, scales, the 4/6 choice and the
output tensor scale must match exactly for every mode.  Inputs are 1D NVFP4
tensors made by the oracle from the seeded workloads, and arbitrary random
code/scale bytes; shapes span several 256 x 256 tiles, ragged edges in both
dimensions, and the full activation shape.
"""
import numpy as np
import pytest

import oracle as O
import synthetic as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_reduce_amd as fp4  # noqa: E402

SEED = 0x0123456789ABCDEF
FLAG_SETS = [0, fp4.FOUR_OVER_SIX, fp4.SR, fp4.RHT16, fp4.RHT16 | fp4.SR,
             fp4.RHT16 | fp4.FOUR_OVER_SIX]


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def f32(v):
    return torch.tensor([np.float32(v)], dtype=torch.float32, device="cuda")


def run_case(codes, scales, alpha, flags, seed=SEED, ctx=""):
    rows, cols = codes.shape[0], codes.shape[1] * 2
    print("requant case", ctx, (rows, cols), "flags", flags, "alpha", float(alpha), flush=True)
    got = fp4.nvfp4_requantize_t(u8(codes), u8(scales), f32(alpha), flags, seed=seed,
                                 want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_requantize_t(codes, scales, np.float32(alpha), rows, cols, flags, seed=seed)
    keys = ["codes", "scales"] + (["choice"] if flags & fp4.FOUR_OVER_SIX else [])
    for k in keys:
        g, w = got[k].cpu().numpy(), want[k]
        assert g.shape == w.shape, (ctx, k, g.shape, w.shape)
        bad = np.argwhere(g != w)
        assert bad.size == 0, "%s flags=%d: %s differs at %d places, first %s: gpu %s oracle %s" % (
            ctx, flags, k, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])
    assert got["alpha"].cpu().numpy()[0] == want["alpha"], ctx
    return got, want


def quantized(workload, rows, cols, flags=fp4.FOUR_OVER_SIX):
    """A 1D NVFP4 tensor as the oracle quantizes a seeded workload."""
    q = O.nvfp4_quantize(S.gen(workload, rows, cols), flags, seed=SEED)
    return q["codes"], q["scales"], q["alpha"]


@pytest.mark.parametrize("flags", FLAG_SETS)
@pytest.mark.parametrize("shape", [(16, 16), (256, 256), (272, 528), (784, 1040)])
def test_requant_random_bytes(shape, flags):
    codes, scales = S.random_nvfp4(*shape, seed=11)
    run_case(codes, scales, 0.0137, flags, ctx="random")


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
@pytest.mark.parametrize("ntiles", [1023, 1025, 2049])
def test_requant_launch_edges(ntiles, flags):
    """Tile counts around the 1024 workgroups the requantization launches on
    256 CUs (four per CU, two resident): a 16-row input has one 16x256 tile
    per 256 columns, so every workgroup takes one tile, one takes a second,
    or all take two or three (the persistent tile loop and its XCD order)."""
    codes, scales = S.random_nvfp4(16, 256 * ntiles - 240, seed=13)
    run_case(codes, scales, 0.0137, flags, ctx="launch-edge")


@pytest.mark.parametrize("flags", FLAG_SETS)
def test_requant_of_quantized_activation(flags):
    codes, scales, alpha = quantized("c2", 528, 1296)
    run_case(codes, scales, alpha, flags, ctx="c2-activation")


@pytest.mark.parametrize("flags", [fp4.RHT16 | fp4.SR, fp4.FOUR_OVER_SIX])
def test_requant_of_quantized_gradient(flags):
    codes, scales, alpha = quantized("c4", 400, 2064, fp4.RHT16 | fp4.SR)
    run_case(codes, scales, alpha, flags, ctx="c4-gradient")


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_requant_amax_given(flags):
    """With the amax given, the result is the oracle's fp32 quantizer on the
    dequantized transpose with that amax (here 1.5x the unrotated maximum)."""
    codes, scales, alpha = quantized("c2", 272, 784)
    rows, cols = 272, 784
    xt = np.ascontiguousarray(O.dequantize(0, codes, scales, alpha, rows, cols).T)
    amax = np.float32(1.5) * np.abs(xt).max()
    print("requant amax given", flags, float(amax), flush=True)
    got = fp4.nvfp4_requantize_t(u8(codes), u8(scales), f32(alpha), flags, seed=SEED,
                                 amax=f32(amax), want_choice=True)
    torch.cuda.synchronize()
    want = O.nvfp4_quantize_f32(xt, flags, seed=SEED, amax=amax)
    for k in ["codes", "scales"] + (["choice"] if flags & fp4.FOUR_OVER_SIX else []):
        assert np.array_equal(got[k].cpu().numpy(), want[k]), k
    assert got["alpha"].cpu().numpy()[0] == want["alpha"]


def test_requant_edge_cases():
    # thin tensors: one block row / one block column
    for shape in ((16, 4096 + 16), (4096 + 16, 16), (16, 32)):
        codes, scales = S.random_nvfp4(*shape, seed=5)
        run_case(codes, scales, 0.5, fp4.FOUR_OVER_SIX, ctx="thin")
    # all-zero scales: alpha_out 0 and every code +-0
    codes, scales = S.random_nvfp4(64, 64, seed=6)
    run_case(codes, np.zeros_like(scales), 1.0, fp4.FOUR_OVER_SIX, ctx="zero-scales")
    # zero tensor scale
    run_case(codes, scales, 0.0, 0, ctx="zero-alpha")
    # the largest input scale with a large alpha: the rotation's sums of 16
    # values stay finite
    run_case(codes, np.full_like(scales, 126), 1.0e33, fp4.RHT16 | fp4.SR, ctx="large")
    # small magnitudes, still above the domain's 2^-64 floor for the amax
    run_case(codes, scales, 1.0e-21, fp4.FOUR_OVER_SIX, ctx="small")


def test_requant_empty():
    for rows, cols in ((0, 64), (64, 0)):
        got = fp4.nvfp4_requantize_t(torch.zeros((rows, cols // 2), dtype=torch.uint8, device="cuda"),
                                     torch.zeros((rows, cols // 16), dtype=torch.uint8, device="cuda"),
                                     f32(1.0), fp4.FOUR_OVER_SIX)
        torch.cuda.synchronize()
        assert got["alpha"].cpu().numpy()[0] == 0.0


def test_requant_rejects_bad_arguments():
    codes, scales = S.random_nvfp4(32, 48, seed=1)
    c, s, a = u8(codes), u8(scales), f32(1.0)
    for flags in (fp4.BLOCK2D, fp4.COLWISE, fp4.HAD32, fp4.SR | fp4.FOUR_OVER_SIX):
        with pytest.raises(fp4.Fp4Error):
            fp4.nvfp4_requantize_t(c, s, a, flags)
    # rows not a multiple of 16
    codes, scales = S.random_nvfp4(24, 48, seed=1)
    with pytest.raises(fp4.Fp4Error):
        fp4.nvfp4_requantize_t(u8(codes), u8(scales), a, 0)


def test_requant_full_activation():
    """The full 8192 x 4096 activation, 4/6 quantized, requantized with RHT16 + SR
    (the weight-gradient operand of the backward pass) and with 4/6."""
    codes, scales, alpha = quantized("c2", *S.WORKLOADS["c2"])
    for flags in (fp4.RHT16 | fp4.SR, fp4.FOUR_OVER_SIX):
        run_case(codes, scales, alpha, flags, ctx="c2-full")


def test_requant_deterministic_and_seeded():
    codes, scales = S.random_nvfp4(512, 512, seed=9)
    c, s, a = u8(codes), u8(scales), f32(0.25)
    x = fp4.nvfp4_requantize_t(c, s, a, fp4.RHT16 | fp4.SR, seed=SEED)
    y = fp4.nvfp4_requantize_t(c, s, a, fp4.RHT16 | fp4.SR, seed=SEED)
    z = fp4.nvfp4_requantize_t(c, s, a, fp4.RHT16 | fp4.SR, seed=SEED + 1)
    torch.cuda.synchronize()
    assert torch.equal(x["codes"], y["codes"]) and torch.equal(x["scales"], y["scales"])
    assert not torch.equal(x["codes"], z["codes"])
