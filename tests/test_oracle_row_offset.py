"""The oracle's band entry points (nvfp4_quantize_at, nvfp4_quantize_rows_at,
nvfp4_requantize_t_at) against the whole-tensor oracle (CPU).

They exist so that sampled row bands of tensors far too large for the oracle
can be checked: a band quantized alone, with the first row's index in the
whole tensor and the whole tensor's amax, must give exactly the whole
tensor's codes, scales and choices for those rows.  The random draws are
keyed by element index (SR, NVIDIA NVFP4 article sec. 7) and block index
(the MS-EDEN scale), so a band at the wrong offset must differ."""
import numpy as np
import pytest

import oracle
import synthetic as S

SEED = 0x5EED5EED12345
BANDS = [(0, 48), (17, 40), (47, 48), (23, 48)]


@pytest.mark.parametrize("flags", [
    0, oracle.FOUR_OVER_SIX, oracle.SR, oracle.RHT16 | oracle.SR,
    oracle.RHT16 | oracle.FOUR_OVER_SIX, oracle.RHT16 | oracle.MSEDEN])
def test_band_equals_whole_tensor(flags):
    x = S.gen("c4", 48, 320)
    amax = oracle.tensor_amax(x, flags, SEED)
    whole = oracle.nvfp4_quantize(x, flags, SEED, amax=amax)
    for r0, r1 in BANDS:
        band = oracle.nvfp4_quantize_at(x[r0:r1], r0, amax, flags, SEED)
        assert band["alpha"] == whole["alpha"]
        for k in ("codes", "scales", "choice"):
            assert np.array_equal(band[k], whole[k][r0:r1]), (flags, r0, k)


@pytest.mark.parametrize("flags", [oracle.SR, oracle.RHT16 | oracle.SR, oracle.RHT16 | oracle.MSEDEN])
def test_band_offset_reaches_the_random_draws(flags):
    x = S.gen("c4", 48, 320)
    amax = oracle.tensor_amax(x, flags, SEED)
    whole = oracle.nvfp4_quantize(x, flags, SEED, amax=amax)
    wrong = oracle.nvfp4_quantize_at(x[17:40], 0, amax, flags, SEED)
    key = "scales" if flags & oracle.MSEDEN else "codes"
    assert not np.array_equal(wrong[key], whole[key][17:40])


def test_band_counter_high_word():
    """Element indices past 2^32: the band's counters carry the high word."""
    x = S.gen("c4", 4, 256)
    amax = oracle.tensor_amax(x)
    lo = oracle.nvfp4_quantize_at(x, 0, amax, oracle.SR, SEED)
    hi = oracle.nvfp4_quantize_at(x, (1 << 32) // 256, amax, oracle.SR, SEED)
    # same values and scales, other random words: scales equal, codes not
    assert np.array_equal(lo["scales"], hi["scales"])
    assert not np.array_equal(lo["codes"], hi["codes"])


@pytest.mark.parametrize("flags", [oracle.FOUR_OVER_SIX, oracle.SR, oracle.RHT16 | oracle.SR])
def test_rows_band_equals_whole_tensor(flags):
    x = S.gen("c2", 48, 256)
    whole = oracle.nvfp4_quantize_rows(x, flags, SEED)
    for r0, r1 in BANDS:
        band = oracle.nvfp4_quantize_rows_at(x[r0:r1], r0, flags, SEED)
        assert np.array_equal(band["alpha"], whole["alpha"][r0:r1])
        for k in ("codes", "scales", "choice"):
            assert np.array_equal(band[k], whole[k][r0:r1]), (flags, r0, k)
    if flags & oracle.SR:
        wrong = oracle.nvfp4_quantize_rows_at(x[17:40], 0, flags, SEED)
        assert not np.array_equal(wrong["codes"], whole["codes"][17:40])


def test_band_rejects_2d_and_missing_amax():
    x = S.gen("c3", 32, 64)
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize_at(x, 16, 1.0, oracle.BLOCK2D)
    with pytest.raises(ValueError):
        oracle.nvfp4_quantize_at(x, -1, 1.0, 0)


@pytest.mark.parametrize("flags", [oracle.FOUR_OVER_SIX, oracle.SR, oracle.RHT16 | oracle.SR,
                                   oracle.RHT16 | oracle.FOUR_OVER_SIX])
def test_requant_column_band_equals_whole(flags):
    rows, cols = 64, 96
    codes, scales = S.random_nvfp4(rows, cols, seed=21)
    alpha = np.float32(0.0123)
    amax = 3.0 if flags & oracle.RHT16 else float(
        np.abs(oracle.dequantize(0, codes, scales, alpha, rows, cols)).max())
    whole = oracle.nvfp4_requantize_t_at(codes, scales, alpha, rows, cols, 0, amax, flags, SEED)
    if not flags & oracle.RHT16:        # the given amax is the true one: the plain call
        plain = oracle.nvfp4_requantize_t(codes, scales, alpha, rows, cols, flags, SEED)
        for k in ("codes", "scales", "choice", "alpha"):
            assert np.array_equal(plain[k], whole[k]), k
    for c0, c1 in [(0, 96), (16, 48), (80, 96)]:
        band = oracle.nvfp4_requantize_t_at(codes[:, c0 // 2:c1 // 2], scales[:, c0 // 16:c1 // 16],
                                            alpha, rows, c1 - c0, c0, amax, flags, SEED)
        assert band["alpha"] == whole["alpha"]
        for k in ("codes", "scales", "choice"):
            assert np.array_equal(band[k], whole[k][c0:c1]), (flags, c0, k)
    if flags & oracle.SR:
        wrong = oracle.nvfp4_requantize_t_at(codes[:, 8:24], scales[:, 1:3], alpha, rows, 32, 0,
                                             amax, flags, SEED)
        assert not np.array_equal(wrong["codes"], whole["codes"][16:48])
