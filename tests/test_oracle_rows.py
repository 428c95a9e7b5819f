"""Pins of the oracle's NVFP4 with one FP32 scale per row, CPU only.

Each row must be quantized exactly as the already pinned per-tensor
quantizer quantizes that row on its own (same alpha, codes, scales and 4/6
choice).  Stochastic rounding keeps the element index in the whole tensor
as its counter, so it is pinned on tensors whose rows all share one amax,
where the per-row and per-tensor scales coincide.  alpha_r follows Eq. 1 on
the row's amax."""
import numpy as np
import pytest

import oracle as O
import synthetic as S

SEED = 0x0123456789ABCDEF
DET_FLAGS = [0, O.FOUR_OVER_SIX, O.RHT16, O.RHT16 | O.FOUR_OVER_SIX]


@pytest.mark.parametrize("flags", DET_FLAGS)
@pytest.mark.parametrize("wl,shape", [("c2", (12, 272)), ("c4", (9, 160)), ("c1", (5, 1024))])
def test_each_row_is_the_per_tensor_quantizer_of_that_row(wl, shape, flags):
    x = S.gen(wl, *shape)
    got = O.nvfp4_quantize_rows(x, flags, seed=SEED)
    for r in range(shape[0]):
        want = O.nvfp4_quantize(x[r:r + 1], flags, seed=SEED)
        assert got["alpha"][r] == want["alpha"], r
        for k in ("codes", "scales", "choice"):
            assert np.array_equal(got[k][r], want[k][0]), (r, k)


@pytest.mark.parametrize("flags", [O.SR, O.RHT16 | O.SR, 0, O.FOUR_OVER_SIX | O.RHT16])
def test_rows_with_one_amax_equal_the_per_tensor_quantizer(flags):
    """Identical rows share their amax (rotated or not), so the per-row
    scales equal the tensor scale; SR counters are global in both."""
    row = S.gen("c4", 1, 512)
    x = np.ascontiguousarray(np.repeat(row, 24, axis=0))
    got = O.nvfp4_quantize_rows(x, flags, seed=SEED)
    want = O.nvfp4_quantize(x, flags, seed=SEED)
    assert np.all(got["alpha"] == want["alpha"])
    for k in ("codes", "scales", "choice"):
        assert np.array_equal(got[k], want[k]), k


@pytest.mark.parametrize("flags,C", [(0, 448.0), (O.FOUR_OVER_SIX, 256.0)])
def test_alpha_is_eq1_on_the_row_amax(flags, C):
    x = S.gen("c2", 40, 96)
    got = O.nvfp4_quantize_rows(x, flags)
    amax = np.abs(S.bf16_bits_to_f32(x)).max(axis=1)
    want = (amax / np.float32(6.0 * C)).astype(np.float32)
    assert np.array_equal(got["alpha"], want)
    # rows differ in scale, so a per-tensor alpha would not fit them all
    assert len(np.unique(got["alpha"])) > 1


def test_zero_rows_and_rejections():
    x = S.gen("c2", 6, 64)
    x[2] = 0
    x[4] = 0x8000                                   # -0 everywhere
    got = O.nvfp4_quantize_rows(x, O.FOUR_OVER_SIX)
    assert got["alpha"][2] == 0 and got["alpha"][4] == 0
    assert np.all(got["scales"][[2, 4]] == 0)
    assert np.all(got["codes"][2] == 0) and np.all(got["codes"][4] == 0x88)
    with pytest.raises(ValueError):
        O.nvfp4_quantize_rows(x, O.BLOCK2D)
    with pytest.raises(ValueError):
        O.nvfp4_quantize_rows(S.gen("c2", 2, 24))
    with pytest.raises(ValueError):
        O.nvfp4_quantize_rows(x, O.SR | O.FOUR_OVER_SIX)
