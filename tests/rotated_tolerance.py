"""Acceptance of rotated MXFP4 results (32-point Hadamard), GPU vs oracle.

The rotation is a sum of 32 terms; the oracle evaluates it as a butterfly in
fp32, the GPU on the matrix cores (products exact, fp32 accumulation in the
hardware's order), so the two rotated values may differ in their last bits.
The acceptance rule for rotated paths is:

  * a code may differ only where the oracle's own fp32 pre-rounding value t
    (value times 2^-e, the number the E2M1 rounding sees) lies within one
    fp32 ulp of a rounding boundary: some boundary b with
    nextafter(t, -inf) <= b <= nextafter(t, +inf).  The boundaries are the
    E2M1 midpoints +-{0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5} and 0 (the sign:
    a +0 / -0 code difference is allowed only where t is within one ulp of
    zero);
  * a UE8M0 scale may differ only where the oracle's fp32 group maximum lies
    within one fp32 ulp of a power of two; such groups are then compared by
    their dequantized error only;
  * at most 1e-5 of the elements may differ (codes, plus 32 per changed
    scale), asserted.  A +0 / -0 difference where the oracle's t is zero
    itself is the same value (the sign of an exact zero sum depends only on
    the order of the additions) and is counted apart, not in this budget;
  * the dequantized relative MSE, sum (deq - y)^2 / sum y^2 in float64 over
    the oracle's rotated values y, must agree within 1e-6.

As a diagnostic only, every difference is also measured against the
rotation in float64 (exact for bf16 inputs up to 2^-53 relative), with the
first-order bound any fp32 order of the 31 additions obeys:
    |y_impl - y_exact| <= 32 u c S + u |y_exact| + 2^-149,   u = 2^-24,
S the sum of |x| over the group.
"""
import numpy as np

import synthetic as S

U = 2.0 ** -24
C32 = float(np.frombuffer(np.uint32(0x3E3504F3).tobytes(), np.float32)[0])
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
SIGNED_BOUNDS = np.concatenate([-BOUNDS[::-1], [0.0], BOUNDS]).astype(np.float32)


def hadamard32():
    i = np.arange(32)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 1, -1.0, 1.0)


H32 = hadamard32()


def within_one_ulp_of_boundary(t):
    """True where an E2M1 rounding boundary (or 0) lies within one fp32 ulp
    of the fp32 value t."""
    t = np.asarray(t, np.float32)
    lo = np.nextafter(t, np.float32(-np.inf))
    hi = np.nextafter(t, np.float32(np.inf))
    ok = np.zeros(t.shape, bool)
    for b in SIGNED_BOUNDS:
        ok |= (lo <= b) & (b <= hi)
    return ok


def within_one_ulp_of_pow2(m):
    """True where a power of two lies within one fp32 ulp of m > 0 (fp32)."""
    m = np.asarray(m, np.float32)
    lo = np.nextafter(m, np.float32(0)).astype(np.float64)
    hi = np.nextafter(m, np.float32(np.inf)).astype(np.float64)
    pos = m > 0
    lo = np.where(pos & (lo > 0), lo, 2.0 ** -160)
    hi = np.where(pos, hi, 2.0 ** -160)
    # a power of two lies in [lo, hi] iff floor(log2) differs, or lo is one
    return pos & ((np.floor(np.log2(lo)) != np.floor(np.log2(hi))) |
                  (np.exp2(np.floor(np.log2(lo))) == lo))


def _deq(c, s):
    v = E2M1[c & 7] * np.exp2(s.astype(np.float64) - 127)[..., None]
    return np.where(c & 8, -v, v)


def check_rotated_mx(codes_gpu, scales_gpu, codes_or, scales_or, t_or, what,
                     x_bits=None, max_frac=1e-5, mse_tol=1e-6, row_chunk=512):
    """codes_* [R][C/2] bytes, scales_* [R][C/32] UE8M0, t_or [R][C] the
    oracle's pre-rounding values (its debug output) for groups of 32 along
    the rows.  x_bits (optional) [R][C] bf16 input of those groups, for the
    float64 diagnostic.  Raises AssertionError with the first difference the
    rule does not allow; returns a dict of counts."""
    codes_gpu, codes_or = np.asarray(codes_gpu), np.asarray(codes_or)
    scales_gpu, scales_or = np.asarray(scales_gpu), np.asarray(scales_or)
    t_or = np.asarray(t_or, np.float32)
    R, C = t_or.shape
    G = C // 32
    stats = dict(codes=0, zero_sign=0, scales=0, diag_outside_f64_bound=0)
    se_g = se_o = sy = 0.0
    for r0 in range(0, R, row_chunk):
        r1 = min(R, r0 + row_chunk)
        t = t_or[r0:r1].reshape(r1 - r0, G, 32)
        sg = scales_gpu[r0:r1].astype(np.int64)
        so = scales_or[r0:r1].astype(np.int64)
        # the oracle's rotated values: t = y * 2^-e exactly, so y = t * 2^e
        y = np.ldexp(t.astype(np.float64), (so - 127)[..., None])
        gmax = np.abs(y).max(-1).astype(np.float32)
        sdiff = sg != so
        bad = sdiff & ~within_one_ulp_of_pow2(gmax)
        if np.any(bad):
            i = tuple(np.argwhere(bad)[0])
            raise AssertionError("%s: scale differs away from a power of two at group %s: "
                                 "gpu %d oracle %d group max %r" % (
                                     what, (r0 + i[0], i[1]), sg[i], so[i], gmax[i]))
        stats["scales"] += int(sdiff.sum())
        cg = S_unpack(codes_gpu[r0:r1]).reshape(r1 - r0, G, 32)
        co = S_unpack(codes_or[r0:r1]).reshape(r1 - r0, G, 32)
        mism = (cg != co) & ~sdiff[..., None]
        idx = np.nonzero(mism)
        if idx[0].size:
            tv = t[idx]
            bad = ~within_one_ulp_of_boundary(tv)
            if np.any(bad):
                k = int(np.argmax(bad))
                at = (r0 + int(idx[0][k]), int(idx[1][k]), int(idx[2][k]))
                raise AssertionError("%s: code differs away from a boundary at %s: gpu %d "
                                     "oracle %d oracle t %r" % (
                                         what, at, cg[idx][k], co[idx][k], tv[k]))
            zs = ((cg[idx] & 7) == 0) & ((co[idx] & 7) == 0) & (tv == 0)
            stats["zero_sign"] += int(zs.sum())
            stats["codes"] += int(idx[0].size)
            if x_bits is not None:               # diagnostic: float64 bound
                x = S.bf16_bits_to_f32(np.asarray(x_bits)[r0:r1]).astype(np.float64)
                x = x.reshape(r1 - r0, G, 32)
                ye = (x @ H32) * C32
                delta = 32 * U * C32 * np.abs(x).sum(-1, keepdims=True) + U * np.abs(ye) \
                    + 2.0 ** -149
                e = (so[idx[:2]] - 127).astype(np.float64)
                te = np.abs(ye[idx]) * np.exp2(-e)
                dt = 2 * delta[idx] * np.exp2(-e)
                far = np.abs(te[:, None] - BOUNDS).min(-1) > dt
                stats["diag_outside_f64_bound"] += int(far.sum())
        se_g += float(((_deq(cg, sg) - y) ** 2).sum())
        se_o += float(((_deq(co, so) - y) ** 2).sum())
        sy += float((y ** 2).sum())
    total = R * C
    changed = stats["codes"] - stats["zero_sign"] + 32 * stats["scales"]
    assert changed <= max_frac * total, "%s: %d elements differ (%d codes, %d scales) of %d" % (
        what, changed, stats["codes"], stats["scales"], total)
    stats["rel_mse_gpu"] = se_g / sy if sy > 0 else 0.0
    stats["rel_mse_oracle"] = se_o / sy if sy > 0 else 0.0
    assert abs(stats["rel_mse_gpu"] - stats["rel_mse_oracle"]) <= mse_tol, (
        "%s: relative MSE gpu %r oracle %r" % (what, stats["rel_mse_gpu"],
                                               stats["rel_mse_oracle"]))
    return stats


def S_unpack(packed):
    """[r][n/2] bytes -> [r][n] 4-bit codes (low nibble = even element)."""
    p = np.asarray(packed, np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def check_mx_outputs(x_bits, flags, got, want, host, what=""):
    """Compare every output of an MXFP4 call with HAD32 (both orientations);
    `want` is the oracle's output with its debug values (t_r / t_c)."""
    import block_scaled_fp4_reduce_amd as fp4
    stats = {}
    if flags & fp4.ROWWISE:
        stats["rows"] = check_rotated_mx(host(got["codes_r"]), host(got["scales_r"]),
                                         want["codes_r"], want["scales_r"], want["t_r"],
                                         what + " rows", x_bits=x_bits)
    if flags & fp4.COLWISE:
        xt = np.ascontiguousarray(np.asarray(x_bits).T)
        stats["cols"] = check_rotated_mx(host(got["codes_c"]), host(got["scales_c"]),
                                         want["codes_c"], want["scales_c"], want["t_c"],
                                         what + " cols", x_bits=xt)
    return stats
