"""Pins of the rotated-path acceptance check (CPU only): it accepts the
oracle against itself, and rejects a code or a scale changed where no
fp32 evaluation order of the rotation could have changed it."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from rotated_tolerance import H32, check_rotated_mx


def test_hadamard_matrix():
    assert np.array_equal(H32 @ H32.T, 32 * np.eye(32))
    assert np.array_equal(H32, H32.T)


def _case():
    x = S.gen("c5", 64, 256)
    want = O.mxfp4_quantize(x, O.HAD32 | O.ROWWISE)
    return x, want["codes_r"].copy(), want["scales_r"].copy()


def test_accepts_identical():
    x, c, s = _case()
    assert check_rotated_mx(x, c, s, c, s, "self") == (0, 0)


def test_rejects_code_flip_far_from_boundary():
    x, c, s = _case()
    bad = c.copy()
    bad[3, 5] ^= 0x01               # element 10 of row 3: magnitude index changed by one
    with pytest.raises(AssertionError, match="away from a boundary"):
        check_rotated_mx(x, bad, s, c, s, "flip")


def test_rejects_scale_change_far_from_power_of_two():
    x, c, s = _case()
    bad = s.copy()
    bad[7, 2] += 1
    with pytest.raises(AssertionError, match="power of two"):
        check_rotated_mx(x, c, bad, c, s, "scale")


def test_oracle_rotation_within_the_bound():
    """The oracle's fp32 butterfly stays inside the error bound the check
    grants any fp32 evaluation of the 32-term rotation."""
    from rotated_tolerance import C32, U
    x = S.gen("c5", 64, 512)
    xf = S.bf16_bits_to_f32(x).reshape(-1, 32)
    got = np.stack([O.rotate_had32(v) for v in xf]).astype(np.float64)
    g = xf.astype(np.float64)
    exact = (g @ H32) * C32
    bound = 32 * U * C32 * np.abs(g).sum(-1, keepdims=True) + U * np.abs(exact) + 2.0 ** -149
    assert np.all(np.abs(got - exact) <= bound)
    assert np.abs(got - exact).max() > 0          # the butterfly does round


def test_signed_zero_codes_are_equal():
    x, c, s = _case()
    u = O.unpack_codes(c)
    r, k = np.argwhere((u & 7) == 0)[0]            # a zero code; flip its sign
    bad = c.copy()
    bad[r, k // 2] ^= 0x08 << (4 * (k % 2))
    assert check_rotated_mx(x, bad, s, c, s, "zero sign") == (0, 0)
