"""GPU parity past 2^32 elements: sampled bands of one 131104 x 32768 bf16
tensor (and of a GEMM with 2^32 outputs) against the CPU oracle.

The interface takes tensors of up to 2^40 elements.  This one holds
4 296 015 872 (8.6 GB), so it passes 2^31 and 2^32 elements, and an index
product kept in 32 bits anywhere would wrap inside it.  Its rows repeat one
seeded 4099-row block of the activation-like generator (a period that does
not divide the wrap distances of 65536 and 131072 rows, so a wrapped access
reads other values), which keeps the input cheap to make; the random draws
(SR by element index, MS-EDEN by block index, requantization SR by output
element index) still differ everywhere.  Each path is checked on three
bands, the start, across 2^31 elements and across 2^32 elements to the end,
against the oracle run on the band alone with the whole tensor's amax and
the band's place in it (the oracle's *_at entry points, pinned on the CPU
against the whole-tensor oracle).  Tensor amaxes are checked whole: the
oracle's amax of the repeated block is the tensor's."""
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

ROWS, COLS, PERIOD = 131104, 32768, 4099
BANDS = [(0, 64), (65504, 65568), (131040, 131104)]   # rows 65536 and 131072 cross 2^31, 2^32
SEED = 0x9E3779B97F4A7C15


def host(t):
    return t.contiguous().cpu().numpy()


def same(g, w, what):
    g = host(g)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    bad = np.argwhere(g != w)
    assert bad.size == 0, "%s differs at %d places, first %s: gpu %s oracle %s" % (
        what, len(bad), bad[:3].tolist(), g[tuple(bad[0])], w[tuple(bad[0])])


def tile_rows(t, rows):
    """Rows 0..rows-1 of the block t repeated down: a view, contiguous."""
    x = t.repeat(-(-rows // t.shape[0]), 1)[:rows]
    assert x.is_contiguous()
    return x


@pytest.fixture(scope="module")
def big():
    assert ROWS * COLS > 2**32
    base = S.gen("c2", PERIOD, COLS)
    print("large tensor", (ROWS, COLS), "period", PERIOD, flush=True)
    x = tile_rows(torch.from_numpy(base.view(np.int16)).cuda(), ROWS)
    yield base, x
    del x
    torch.cuda.empty_cache()


def band_of(base, r0, r1):
    return np.ascontiguousarray(base[np.arange(r0, r1) % PERIOD])


_AMAX = {}


def oracle_amax(base, rht):
    """The oracle's tensor amax of the repeated block (that of the tensor)."""
    if rht not in _AMAX:
        _AMAX[rht] = np.float32(O.tensor_amax(base, fp4.RHT16 if rht else 0, SEED))
    return _AMAX[rht]


@pytest.mark.parametrize("flags", [0, fp4.RHT16])
def test_large_tensor_amax(big, flags):
    base, x = big
    print("large amax flags", flags, flush=True)
    got = host(fp4.fp4_tensor_amax(x, flags, SEED))[0]
    assert got == oracle_amax(base, bool(flags & fp4.RHT16))


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR, fp4.RHT16 | fp4.MSEDEN])
def test_large_nvfp4(big, flags):
    """The whole path (amax pass, then the quantizer); 4/6 also decoded."""
    base, x = big
    print("large nvfp4 flags", flags, flush=True)
    got = fp4.nvfp4_quantize(x, flags, seed=SEED, want_choice=True)
    torch.cuda.synchronize()
    amax = oracle_amax(base, bool(flags & fp4.RHT16))
    for r0, r1 in BANDS:
        want = O.nvfp4_quantize_at(band_of(base, r0, r1), r0, amax, flags, SEED)
        assert host(got["alpha"])[0] == want["alpha"]
        for k in ("codes", "scales", "choice"):
            same(got[k][r0:r1], want[k], "flags %d rows %d: %s" % (flags, r0, k))
    if flags == fp4.FOUR_OVER_SIX:
        print("large nvfp4 dequantize", flush=True)
        deq = fp4.fp4_dequantize(fp4.FORMAT_NVFP4, got["codes"], got["scales"], got["alpha"],
                                 ROWS, COLS)
        torch.cuda.synchronize()
        a = host(got["alpha"])[0]
        for r0, r1 in BANDS:
            want = O.dequantize(0, host(got["codes"][r0:r1]), host(got["scales"][r0:r1]), a,
                                r1 - r0, COLS)
            same(deq[r0:r1], want, "dequantize rows %d" % r0)
        del deq
    del got
    torch.cuda.empty_cache()


def test_large_2d(big):
    base, x = big
    flags = fp4.BLOCK2D | fp4.FOUR_OVER_SIX | fp4.COLWISE
    print("large 2d flags", flags, flush=True)
    got = fp4.nvfp4_quantize(x, flags, want_choice=True)
    torch.cuda.synchronize()
    amax = oracle_amax(base, False)
    for r0, r1 in BANDS:        # 16-row multiples: whole tiles, no random draws
        want = O.nvfp4_quantize(band_of(base, r0, r1), flags, amax=amax)
        assert host(got["alpha"])[0] == want["alpha"]
        same(got["codes"][r0:r1], want["codes"], "2d codes rows %d" % r0)
        for k in ("scales", "choice"):
            same(got[k][r0 // 16:r1 // 16], want[k], "2d %s rows %d" % (k, r0))
        same(got["codes_t"][:, r0 // 2:r1 // 2], want["codes_t"], "2d codes_t rows %d" % r0)
        same(got["scales_t"][:, r0 // 16:r1 // 16], want["scales_t"], "2d scales_t rows %d" % r0)
    del got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_large_rows(big, flags):
    base, x = big
    print("large rows flags", flags, flush=True)
    got = fp4.nvfp4_quantize_rows(x, flags, seed=SEED, want_choice=True)
    torch.cuda.synchronize()
    for r0, r1 in BANDS:
        want = O.nvfp4_quantize_rows_at(band_of(base, r0, r1), r0, flags, SEED)
        same(got["alpha"][r0:r1], want["alpha"], "rows alpha %d" % r0)
        for k in ("codes", "scales", "choice"):
            same(got[k][r0:r1], want[k], "rows flags %d rows %d: %s" % (flags, r0, k))
    del got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags", [fp4.ROWWISE | fp4.COLWISE,
                                   fp4.HAD32 | fp4.ROWWISE | fp4.COLWISE])
def test_large_mx(big, flags):
    base, x = big
    print("large mx flags", flags, flush=True)
    got = fp4.mxfp4_quantize(x, flags)
    torch.cuda.synchronize()
    for r0, r1 in BANDS:        # 32-row multiples: whole column groups
        b = band_of(base, r0, r1)
        want = O.mxfp4_quantize(b, flags, debug=bool(flags & fp4.HAD32))
        gb = {"codes_r": got["codes_r"][r0:r1], "scales_r": got["scales_r"][r0:r1],
              "codes_c": got["codes_c"][:, r0 // 2:r1 // 2],
              "scales_c": got["scales_c"][:, r0 // 32:r1 // 32]}
        if flags & fp4.HAD32:
            print("band", r0, check_mx_outputs(b, flags, gb, want, host, "large mx %d" % r0),
                  flush=True)
        else:
            for k in gb:
                same(gb[k], want[k], "mx %s rows %d" % (k, r0))
    del got
    torch.cuda.empty_cache()


@pytest.mark.parametrize("flags", [fp4.FOUR_OVER_SIX, fp4.RHT16 | fp4.SR])
def test_large_requant(flags):
    """Requantization of a 1D NVFP4 tensor [ROWS][COLS] for its transpose:
    bands of output rows (input columns) at the start, across 2^31 and
    across 2^32 output elements.  4/6 runs the amax pass (the oracle's amax
    is that of the repeated block's decode); RHT16 + SR takes a given amax."""
    codes_b, scales_b = S.random_nvfp4(PERIOD, COLS, seed=41)
    alpha = np.float32(0.0123)
    print("large requant flags", flags, flush=True)
    codes = tile_rows(torch.from_numpy(codes_b).cuda(), ROWS)
    scales = tile_rows(torch.from_numpy(scales_b).cuda(), ROWS)
    a_dev = torch.tensor([alpha], dtype=torch.float32, device="cuda")
    if flags & fp4.RHT16:
        amax = np.float32(2.0)
        got = fp4.nvfp4_requantize_t(codes, scales, a_dev, flags, SEED, want_choice=True,
                                     amax=torch.tensor([amax], dtype=torch.float32, device="cuda"))
    else:
        amax = np.float32(np.abs(O.dequantize(0, codes_b, scales_b, alpha, PERIOD, COLS)).max())
        got = fp4.nvfp4_requantize_t(codes, scales, a_dev, flags, SEED, want_choice=True)
    torch.cuda.synchronize()
    idx = np.arange(ROWS) % PERIOD
    for c0, c1 in [(0, 32), (16368, 16400), (32736, 32768)]:   # c * ROWS crosses 2^31, 2^32
        cb = np.ascontiguousarray(codes_b[:, c0 // 2:c1 // 2][idx])
        sb = np.ascontiguousarray(scales_b[:, c0 // 16:c1 // 16][idx])
        want = O.nvfp4_requantize_t_at(cb, sb, alpha, ROWS, c1 - c0, c0, amax, flags, SEED)
        assert host(got["alpha"])[0] == want["alpha"]
        for k in ("codes", "scales", "choice"):
            same(got[k][c0:c1], want[k], "requant flags %d cols %d: %s" % (flags, c0, k))
    del got, codes, scales
    torch.cuda.empty_cache()


def test_large_gemm():
    """C = A B with M N = 4 311 744 512 outputs (17 GB of fp32): rows at the
    start, across 2^31 and across 2^32 outputs, and the last tile's, within
    the fp32 summation bound of the exact product."""
    M, N, K = 65792, 65536, 128
    rng = np.random.default_rng(77)
    ac = rng.integers(0, 256, size=(M, K // 2), dtype=np.uint8)
    asc = rng.integers(115, 140, size=(M, K // 32), dtype=np.uint8)
    bc = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    bsc = rng.integers(115, 140, size=(N, K // 32), dtype=np.uint8)
    print("large gemm", (M, N, K), flush=True)
    u8 = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()   # noqa: E731
    got = fp4.mxfp4_gemm(u8(ac), u8(asc), u8(bc), u8(bsc))
    torch.cuda.synchronize()
    rows = np.array([0, 1, 255, 256, 32767, 32768, 65535, 65536, 65537, 65790, 65791])
    sub = got.index_select(0, torch.from_numpy(rows).cuda()).cpu().numpy().astype(np.float64)
    want = O.mxfp4_gemm(ac[rows], asc[rows], bc, bsc, len(rows), N, K)
    A = np.abs(O.dequantize(1, ac[rows], asc[rows], 0.0, len(rows), K).astype(np.float64))
    B = np.abs(O.dequantize(1, bc, bsc, 0.0, N, K).astype(np.float64))
    bound = K * 2.0 ** -23 * (A @ B.T) + 1e-30
    err = np.abs(sub - want)
    assert np.all(err <= bound), "%d entries out of bound" % int((err > bound).sum())
    del got
    torch.cuda.empty_cache()
