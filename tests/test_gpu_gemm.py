"""GPU check of the MXFP4 matrix product against the oracle's float64
product of the dequantized operands.

The products of E2M1 values and power-of-two scales are exact; the matrix
cores add them in fp32 in their own order, so every entry must lie within
the fp32 summation bound K * 2^-23 * (|A| |B|)_mn of the exact result
(written below).  Shapes span several 128 x 128 tiles, ragged M and N,
single rows and columns; operands are random code and scale bytes, and the
MXFP4 quantizer's own row-wise and column-wise outputs (with and without the
32-point Hadamard, whose rotations along K cancel in the product)."""
import numpy as np
import pytest

import oracle as O
import synthetic as S

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import block_scaled_fp4_reduce_amd as fp4  # noqa: E402


def u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def random_mx(rows, cols, rng, lo=115, hi=140):
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(lo, hi, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def check(ac, asc, bc, bsc, ctx):
    M, N, K = ac.shape[0], bc.shape[0], ac.shape[1] * 2
    print("gemm case", ctx, (M, N, K), flush=True)
    got = fp4.mxfp4_gemm(u8(ac), u8(asc), u8(bc), u8(bsc))
    torch.cuda.synchronize()
    got = got.cpu().numpy().astype(np.float64)
    want = O.mxfp4_gemm(ac, asc, bc, bsc, M, N, K)
    A = np.abs(O.dequantize(1, ac, asc, 0.0, M, K).astype(np.float64))
    B = np.abs(O.dequantize(1, bc, bsc, 0.0, N, K).astype(np.float64))
    bound = K * 2.0 ** -23 * (A @ B.T) + 1e-30
    err = np.abs(got - want)
    worst = np.unravel_index(np.argmax(err / bound), err.shape)
    assert np.all(err <= bound), "%s: %d entries out of bound, worst %s gpu %r exact %r bound %r" % (
        ctx, int((err > bound).sum()), worst, got[worst], want[worst], bound[worst])
    return got, want


@pytest.mark.parametrize("shape", [(128, 128, 128), (256, 384, 512), (200, 136, 256),
                                   (1, 1, 128), (33, 65, 384), (130, 3, 1024)])
def test_gemm_random_operands(shape):
    M, N, K = shape
    rng = np.random.default_rng(M * 7 + N * 3 + K)
    ac, asc = random_mx(M, K, rng)
    bc, bsc = random_mx(N, K, rng)
    check(ac, asc, bc, bsc, "random")


def test_gemm_unit_scales_exact():
    """All scales 1: the exact results are multiples of 1/4 below 2^24 /
    4, so the fp32 sums must be exact."""
    rng = np.random.default_rng(11)
    M, N, K = 256, 256, 1024
    ac, _ = random_mx(M, K, rng)
    bc, _ = random_mx(N, K, rng)
    ones = lambda r: np.full((r, K // 32), 127, np.uint8)
    got, want = check(ac, ones(M), bc, ones(N), "unit scales")
    assert np.array_equal(got, want)


@pytest.mark.parametrize("flags", [fp4.ROWWISE | fp4.COLWISE, fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE])
def test_gemm_of_quantizer_outputs(flags):
    """A = row-wise MXFP4 of X [M][K]; B^T = column-wise MXFP4 of W [K][N],
    both made by the oracle from seeded c5-like tensors."""
    M, K, N = 192, 512, 160
    qa = O.mxfp4_quantize(S.gen("c5", M, K), flags)
    qb = O.mxfp4_quantize(S.gen("c5", K, N, seed=77), flags)
    check(qa["codes_r"], qa["scales_r"], qb["codes_c"], qb["scales_c"], "quantized")


# Multi-tile grids in the launch configuration of the large products: the
# super-tile order of the tile scheduler is on once the 256 x 256 tiles form
# at least 8 groups of 4 x 8 tiles (M = 2048, N = 8192: 8 x 32 tiles); the
# ragged case has a partial last row and column of tiles, the deep-K cases
# 64 steps of K (and 48 with the super-tile order).
@pytest.mark.parametrize("shape", [(2048, 8192, 1024), (2100, 8320, 512), (512, 512, 8192),
                                   (2304, 8448, 6144)])
def test_gemm_multitile(shape):
    M, N, K = shape
    rng = np.random.default_rng(M + 5 * N + 11 * K)
    ac, asc = random_mx(M, K, rng)
    bc, bsc = random_mx(N, K, rng)
    check(ac, asc, bc, bsc, "multi-tile")


def test_gemm_full_size_sampled():
    """The benchmarked 16384 x 8192 x 8192 product, every output column, on
    rows sampled from each 256-row tile (C[i, :] depends only on A's row i
    and all of B, so the oracle computes just those rows)."""
    M, N, K = 16384, 8192, 8192
    rng = np.random.default_rng(16384)
    ac, asc = random_mx(M, K, rng)
    bc, bsc = random_mx(N, K, rng)
    print("gemm case full size sampled", (M, N, K), flush=True)
    got = fp4.mxfp4_gemm(u8(ac), u8(asc), u8(bc), u8(bsc))
    torch.cuda.synchronize()
    tiles = np.arange(0, M, 256)
    rows = np.unique(np.concatenate([tiles + (tiles * 37) % 256, tiles + 255 - (tiles * 11) % 256,
                                     [0, M - 1]]))
    got = got[torch.from_numpy(rows).cuda()].cpu().numpy().astype(np.float64)
    A = O.dequantize(1, ac[rows], asc[rows], 0.0, len(rows), K).astype(np.float64)
    B = O.dequantize(1, bc, bsc, 0.0, N, K).astype(np.float64)
    want = A @ B.T
    bound = K * 2.0 ** -23 * (np.abs(A) @ np.abs(B).T) + 1e-30
    err = np.abs(got - want)
    assert np.all(err <= bound), "full size: %d sampled entries out of bound" % int((err > bound).sum())


def test_gemm_edges():
    rng = np.random.default_rng(3)
    ac, asc = random_mx(64, 128, rng)
    empty = fp4.mxfp4_gemm(u8(ac[:0]), u8(asc[:0]), u8(ac), u8(asc))
    assert empty.shape == (0, 64)
    z = fp4.mxfp4_gemm(u8(np.zeros((5, 0), np.uint8)), u8(np.zeros((5, 0), np.uint8)),
                       u8(np.zeros((7, 0), np.uint8)), u8(np.zeros((7, 0), np.uint8)))
    torch.cuda.synchronize()
    assert z.shape == (5, 7) and torch.count_nonzero(z).item() == 0
    with pytest.raises(fp4.Fp4Error):                          # K % 128
        fp4.mxfp4_gemm(u8(ac[:, :32]), u8(asc[:, :2]), u8(ac[:, :32]), u8(asc[:, :2]))
