"""Acceptance of rotated MXFP4 results (32-point Hadamard), GPU vs oracle.

The rotation is a sum of 32 terms; the oracle evaluates it as a butterfly in
fp32, the GPU on the matrix cores (products exact, fp32 accumulation in the
hardware's order).  Both are within a few units in the last place of the
exact sum, so a code may differ only where the exact pre-rounding value lies
next to a rounding boundary (codes +0 and -0 count as equal: they decode to
the same value), and a block scale only where the exact block maximum lies
next to a power of two.  This module checks exactly that,
against the rotation computed in float64 (exact for these inputs up to
2^-53 relative), plus the two global limits: mismatching elements at most
1e-5 of the total, and the dequantized relative MSE of the two results
within 1e-6 of each other.

Error bound used for each rotated value y = fl(fl(sum) * c):
    |y_impl - y_exact| <= 32 u c S + u |y_exact| + 2^-149,   u = 2^-24,
where S is the sum of |x| over the group: any order of 31 fp32 additions of
partial sums bounded by S errs by at most 31 u S (first-order), the
multiply by c adds one rounding, and the last term covers subnormals.
The bound holds for the oracle and the GPU alike, so a disagreement is
only allowed where the exact value is within twice the bound of a boundary.
"""
import numpy as np

import oracle as O
import synthetic as S

U = 2.0 ** -24
C32 = float(np.frombuffer(np.uint32(0x3E3504F3).tobytes(), np.float32)[0])
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
BOUNDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])


def hadamard32():
    i = np.arange(32)
    pc = np.vectorize(lambda v: bin(v).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 1, -1.0, 1.0)


H32 = hadamard32()


def check_rotated_mx(x_bits, codes_gpu, scales_gpu, codes_or, scales_or, what,
                     max_frac=1e-5, mse_tol=1e-6, row_chunk=512):
    """x_bits: [R][C] bf16 bit patterns whose rows hold the 32-value groups
    (pass the transpose for column-wise output).  codes_* [R][C/2] bytes,
    scales_* [R][C/32] UE8M0.  Raises AssertionError with the first
    unexplained difference; returns (mismatched elements, changed scales)."""
    x_bits = np.asarray(x_bits)
    R, C = x_bits.shape
    G = C // 32
    codes_gpu, codes_or = np.asarray(codes_gpu), np.asarray(codes_or)
    scales_gpu, scales_or = np.asarray(scales_gpu), np.asarray(scales_or)
    n_mism = n_scale = 0
    se_g = se_o = sy = 0.0
    for r0 in range(0, R, row_chunk):
        r1 = min(R, r0 + row_chunk)
        x = S.bf16_bits_to_f32(x_bits[r0:r1]).astype(np.float64).reshape(r1 - r0, G, 32)
        y = (x @ H32) * C32                                   # exact rotation (float64)
        delta = 32 * U * C32 * np.abs(x).sum(-1, keepdims=True) + U * np.abs(y) + 2.0 ** -149
        amax = np.abs(y).max(-1)
        dmax = delta.max(-1)
        sg = scales_gpu[r0:r1].astype(np.int64)
        so = scales_or[r0:r1].astype(np.int64)
        # a scale may change only if [amax - 2 dmax, amax + 2 dmax] holds a power of two
        lo = np.maximum(amax - 2 * dmax, 2.0 ** -160)
        hi = amax + 2 * dmax
        straddle = np.floor(np.log2(lo)) != np.floor(np.log2(hi))
        sdiff = sg != so
        if np.any(sdiff & ~straddle):
            i = np.argwhere(sdiff & ~straddle)[0]
            raise AssertionError("%s: scale differs away from a power of two at group %s: "
                                 "gpu %d oracle %d amax %r" % (what, (r0 + i[0], i[1]),
                                                               sg[tuple(i)], so[tuple(i)],
                                                               amax[tuple(i)]))
        n_scale += int(sdiff.sum())
        cg = O.unpack_codes(codes_gpu[r0:r1]).reshape(r1 - r0, G, 32)
        co = O.unpack_codes(codes_or[r0:r1]).reshape(r1 - r0, G, 32)
        # +0 and -0 decode to the same value: a sign-of-zero difference (sums of
        # signed zeros depend on the order) is not a difference of results
        mism = (cg != co) & ~(((cg & 7) == 0) & ((co & 7) == 0)) & ~sdiff[..., None]
        idx = np.nonzero(mism)
        if idx[0].size:
            e = (so[idx[:2]] - 127).astype(np.float64)
            t = np.abs(y[idx]) * np.exp2(-e)                   # exact |pre-rounding value|
            dt = 2 * delta[idx] * np.exp2(-e)
            bad = ~(np.abs(t[:, None] - BOUNDS).min(-1) <= dt)
            if np.any(bad):
                k = int(np.argmax(bad))
                at = (r0 + int(idx[0][k]), int(idx[1][k]), int(idx[2][k]))
                raise AssertionError("%s: code differs away from a boundary at %s: gpu %d "
                                     "oracle %d t %r (bound %r)" % (
                                         what, at, cg[idx][k], co[idx][k], t[k], dt[k]))
        n_mism += int(idx[0].size)
        # dequantized error against the exact rotation, in double
        def deq(c, s):
            v = E2M1[c & 7] * np.exp2(s.astype(np.float64) - 127)[..., None]
            return np.where(c & 8, -v, v)
        se_g += float(((deq(cg, sg) - y) ** 2).sum())
        se_o += float(((deq(co, so) - y) ** 2).sum())
        sy += float((y ** 2).sum())
    total = R * C
    changed = n_mism + 32 * n_scale
    assert changed <= max_frac * total, "%s: %d elements differ (%d codes, %d scales) of %d" % (
        what, changed, n_mism, n_scale, total)
    if sy > 0:
        rg, ro = se_g / sy, se_o / sy
        assert abs(rg - ro) <= mse_tol, "%s: relative MSE gpu %r oracle %r" % (what, rg, ro)
    return n_mism, n_scale


def check_mx_outputs(x_bits, flags, got, want, host, what=""):
    """Compare every output of an MXFP4 call with HAD32 (both orientations)."""
    import block_scaled_fp4_reduce_amd as fp4
    stats = {}
    if flags & fp4.ROWWISE:
        stats["rows"] = check_rotated_mx(x_bits, host(got["codes_r"]), host(got["scales_r"]),
                                         want["codes_r"], want["scales_r"], what + " rows")
    if flags & fp4.COLWISE:
        xt = np.ascontiguousarray(np.asarray(x_bits).T)
        stats["cols"] = check_rotated_mx(xt, host(got["codes_c"]), host(got["scales_c"]),
                                         want["codes_c"], want["scales_c"], what + " cols")
    return stats
