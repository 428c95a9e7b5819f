"""Pins of the oracle's MXFP4 matrix product (C = A B from row-wise MXFP4
A [M][K] and B^T [N][K]), CPU only: a brute-force triple loop over the
decoded values on tiny shapes, and exact integer results when every scale
is 1 (products of E2M1 values are multiples of 1/4)."""
import numpy as np

import oracle as O

E2M1 = np.array([0, .5, 1, 1.5, 2, 3, 4, 6, -0., -.5, -1, -1.5, -2, -3, -4, -6])


def random_mx(rows, cols, rng, scale_lo=120, scale_hi=134):
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(scale_lo, scale_hi, size=(rows, cols // 32), dtype=np.uint8)
    return codes, scales


def test_brute_force_triple_loop():
    rng = np.random.default_rng(4)
    M, N, K = 3, 5, 64
    ac, asc = random_mx(M, K, rng)
    bc, bsc = random_mx(N, K, rng)
    got = O.mxfp4_gemm(ac, asc, bc, bsc, M, N, K)
    qa, qb = O.unpack_codes(ac), O.unpack_codes(bc)
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                va = E2M1[qa[m, k]] * 2.0 ** (int(asc[m, k // 32]) - 127)
                vb = E2M1[qb[n, k]] * 2.0 ** (int(bsc[n, k // 32]) - 127)
                acc += va * vb
            assert abs(got[m, n] - acc) <= 1e-12 * max(1.0, abs(acc)), (m, n)


def test_unit_scales_give_exact_quarter_integers():
    rng = np.random.default_rng(5)
    M, N, K = 40, 24, 256
    ac, _ = random_mx(M, K, rng)
    bc, _ = random_mx(N, K, rng)
    ones_a = np.full((M, K // 32), 127, np.uint8)
    ones_b = np.full((N, K // 32), 127, np.uint8)
    got = O.mxfp4_gemm(ac, ones_a, bc, ones_b, M, N, K)
    ia = (2 * E2M1[O.unpack_codes(ac)]).astype(np.int64)      # 2x E2M1 values are integers
    ib = (2 * E2M1[O.unpack_codes(bc)]).astype(np.int64)
    assert np.array_equal(got * 4, (ia @ ib.T).astype(np.float64))
