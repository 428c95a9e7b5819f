"""Pins of the oracle's requantization for the transposed operand
(quantize(dequantize(X)^T)), CPU only.

When the dequantized values are exactly representable in bf16 (tensor scale
a power of two: q has at most 2 significant bits and an E4M3 scale at most
4, so q * Delta * 2^k has at most 6), the requantization must equal the
already pinned bf16 quantizer applied to the transposed bf16 tensor -- an
independent path through the bf16 entry point, with its own transposition
done here by numpy."""
import numpy as np
import pytest

import oracle as O
import synthetic as S

SEED = 0x0123456789ABCDEF
FLAGS = [0, O.FOUR_OVER_SIX, O.SR, O.RHT16, O.RHT16 | O.SR]


def random_nvfp4(rows, cols, seed=3):
    return S.random_nvfp4(rows, cols, seed)


@pytest.mark.parametrize("flags", FLAGS)
@pytest.mark.parametrize("shape", [(16, 16), (48, 80), (64, 272)])
def test_requant_equals_bf16_path_on_exact_values(shape, flags):
    rows, cols = shape
    codes, scales = random_nvfp4(rows, cols)
    alpha = np.float32(2.0 ** -5)
    deq = O.dequantize(0, codes, scales, alpha, rows, cols)
    xt = np.ascontiguousarray(deq.T)
    bits = S.f32_to_bf16_bits(xt)
    assert np.array_equal(S.bf16_bits_to_f32(bits), xt)      # bf16-exact by construction
    want = O.nvfp4_quantize(bits, flags, seed=SEED)
    got = O.nvfp4_requantize_t(codes, scales, alpha, rows, cols, flags, seed=SEED)
    for k in ("codes", "scales", "choice"):
        assert np.array_equal(got[k], want[k]), k
    assert got["alpha"] == want["alpha"]


def test_quantize_f32_equals_bf16_path():
    x = S.gen("c2", 32, 256)
    xf = S.bf16_bits_to_f32(x)
    for flags in FLAGS:
        a = O.nvfp4_quantize_f32(xf, flags, seed=SEED)
        b = O.nvfp4_quantize(x, flags, seed=SEED)
        for k in ("codes", "scales", "choice"):
            assert np.array_equal(a[k], b[k]), (flags, k)
        assert a["alpha"] == b["alpha"]


def test_requant_of_a_quantized_activation_round_trips_scales():
    """Requantizing X^T and then X (two transposes) with RTN6 reproduces a
    valid NVFP4 tensor whose dequantized values stay within the format's
    relative error of the first dequantization (max |error| per block is at
    most half a grid step of the block scale)."""
    x = S.gen("c2", 64, 128)
    q = O.nvfp4_quantize(x, O.FOUR_OVER_SIX)
    r = O.nvfp4_requantize_t(q["codes"], q["scales"], q["alpha"], 64, 128, 0)
    d0 = O.dequantize(0, q["codes"], q["scales"], q["alpha"], 64, 128).T
    d1 = O.dequantize(0, r["codes"], r["scales"], r["alpha"], 128, 64)
    s = (r["alpha"] * O.e4m3_decode(r["scales"])).astype(np.float64)     # [128][4]
    step = np.repeat(s, 16, axis=1) * 2.0                                 # largest grid step
    assert np.all(np.abs(d1.astype(np.float64) - d0) <= step / 2 + 1e-30)


def test_requant_rejects_bad_shapes():
    c, s = random_nvfp4(16, 32)
    with pytest.raises(ValueError):
        O.nvfp4_requantize_t(c, s, 1.0, 24, 32)          # rows % 16
    with pytest.raises(ValueError):
        O.nvfp4_requantize_t(c, s, 1.0, 16, 32, O.BLOCK2D)
