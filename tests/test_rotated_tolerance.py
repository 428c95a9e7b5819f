"""Pins of the rotated-path acceptance check (CPU only): it accepts the
oracle against itself, and rejects a code or a scale changed where the
oracle's own pre-rounding value is not within one fp32 ulp of a rounding
boundary (or its group maximum not within one ulp of a power of two)."""
import numpy as np
import pytest

import oracle as O
import synthetic as S
from rotated_tolerance import (H32, check_rotated_mx, within_one_ulp_of_boundary,
                               within_one_ulp_of_pow2)


def test_hadamard_matrix():
    assert np.array_equal(H32 @ H32.T, 32 * np.eye(32))
    assert np.array_equal(H32, H32.T)


def _case():
    x = S.gen("c5", 64, 256)
    want = O.mxfp4_quantize(x, O.HAD32 | O.ROWWISE, debug=True)
    return x, want["codes_r"].copy(), want["scales_r"].copy(), want["t_r"]


def _check(c, s, c0, s0, t, what, x=None):
    return check_rotated_mx(c, s, c0, s0, t, what, x_bits=x)


def test_accepts_identical():
    x, c, s, t = _case()
    st = _check(c, s, c, s, t, "self", x)
    assert (st["codes"], st["scales"], st["zero_sign"]) == (0, 0, 0)
    assert st["rel_mse_gpu"] == st["rel_mse_oracle"] > 0


def test_rejects_code_flip_far_from_boundary():
    x, c, s, t = _case()
    bad = c.copy()
    bad[3, 5] ^= 0x01               # element 10 of row 3: magnitude index changed by one
    with pytest.raises(AssertionError, match="away from a boundary"):
        _check(bad, s, c, s, t, "flip")


def test_rejects_scale_change_far_from_power_of_two():
    x, c, s, t = _case()
    bad = s.copy()
    bad[7, 2] += 1
    with pytest.raises(AssertionError, match="power of two"):
        _check(c, bad, c, s, t, "scale")


def test_accepts_code_flip_at_a_boundary_only_within_one_ulp():
    """Plant a value exactly on a boundary in the oracle's t (and one two
    ulps away): the check allows the neighbouring code for the first only."""
    x, c, s, t = _case()
    t = t.copy()
    u = O.unpack_codes(c)
    t[0, 0] = np.float32(2.5)               # on the 2 | 3 boundary; oracle code: 2.0 (even)
    u[0, 0] = (u[0, 0] & 8) | 4
    t[0, 1] = np.nextafter(np.nextafter(np.float32(2.5), np.float32(9)), np.float32(9))
    u[0, 1] = (u[0, 1] & 8) | 5             # oracle code: 3.0
    c_or = (u[:, 0::2] | (u[:, 1::2] << 4)).astype(np.uint8)
    g = u.copy()
    g[0, 0] = (g[0, 0] & 8) | 5             # the other side of the tie: allowed
    got = (g[:, 0::2] | (g[:, 1::2] << 4)).astype(np.uint8)
    st = check_rotated_mx(got, s, c_or, s, t, "tie", max_frac=1.0, mse_tol=1.0)
    assert st["codes"] == 1
    g[0, 1] = (g[0, 1] & 8) | 4             # two ulps away: not allowed
    got = (g[:, 0::2] | (g[:, 1::2] << 4)).astype(np.uint8)
    with pytest.raises(AssertionError, match="away from a boundary"):
        check_rotated_mx(got, s, c_or, s, t, "two ulps", max_frac=1.0, mse_tol=1.0)


def test_ulp_predicates():
    f = np.float32
    up = lambda v: np.nextafter(f(v), f(np.inf))
    dn = lambda v: np.nextafter(f(v), f(-np.inf))
    assert within_one_ulp_of_boundary(np.array([0.25, up(0.25), dn(0.25), -5.0, up(-5.0),
                                                0.0, -0.0, 1e-45], np.float32)).all()
    assert not within_one_ulp_of_boundary(np.array([up(up(0.25)), 0.3, 6.0, 1e-30, -2.0],
                                                   np.float32)).any()
    assert within_one_ulp_of_pow2(np.array([4.0, up(4.0), dn(8.0), 2.0 ** -130], np.float32)).all()
    assert not within_one_ulp_of_pow2(np.array([up(up(4.0)), 5.0, 0.0, 7.5], np.float32)).any()


def test_signed_zero_code_needs_t_at_zero():
    """A +0/-0 code difference is a sign difference: allowed where the
    oracle's t is within one ulp of 0, rejected where t is a small non-zero
    value (the sign of a real value must not change)."""
    x, c, s, t = _case()
    u = O.unpack_codes(c)
    t = t.copy()
    r, k = np.argwhere(((u & 7) == 0) & (np.abs(t) > 1e-3) & (np.abs(t) < 0.2))[0]
    bad = c.copy()
    bad[r, k // 2] ^= 0x08 << (4 * (k % 2))
    with pytest.raises(AssertionError, match="away from a boundary"):
        _check(bad, s, c, s, t, "zero sign")
    t[r, k] = np.float32(0.0) if not (u[r, k] & 8) else np.float32(-0.0)
    st = check_rotated_mx(bad, s, c, s, t, "zero sign at 0", max_frac=1.0)
    assert st["codes"] == 1 and st["zero_sign"] == 1


def test_oracle_rotation_within_the_diagnostic_bound():
    """The oracle's fp32 butterfly stays inside the float64 bound the
    diagnostic grants any fp32 evaluation of the 32-term rotation."""
    from rotated_tolerance import C32, U
    x = S.gen("c5", 64, 512)
    xf = S.bf16_bits_to_f32(x).reshape(-1, 32)
    got = np.stack([O.rotate_had32(v) for v in xf]).astype(np.float64)
    g = xf.astype(np.float64)
    exact = (g @ H32) * C32
    bound = 32 * U * C32 * np.abs(g).sum(-1, keepdims=True) + U * np.abs(exact) + 2.0 ** -149
    assert np.all(np.abs(got - exact) <= bound)
    assert np.abs(got - exact).max() > 0          # the butterfly does round
