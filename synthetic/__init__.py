"""Seeded synthetic bf16 inputs for the block-scaled FP4 quantizers.

This module holds only input generation: no part of the quantization
method.  Both the CPU oracle and the HIP library are fed the same bytes.

Workloads (shapes and value distributions of LLM tensors, with the tensor
roles the pages assign to each quantizer variant):

  c1  256 x 1024       N(0,1); floor(0.001*N) distinct seeded positions x50
  c2  8192 x 4096      Student-t(nu=4) x per-column lognormal(0,1)   (activations)
  c3  14336 x 4096     N(0, 0.02)                                    (weights)
  c4  8192 x 14336     Laplace(0, 1e-3); floor(0.0005*N) positions x100 (gradients)
  c5  16384 x 8192     N(0,1) x per-row lognormal(0, 0.5)

Recipe: numpy ``Generator(PCG64(seed))`` with data seed ``1000 + k`` for
workload ``ck``; values are drawn in float64 (float32 for plain normals),
then rounded to bf16 with round-to-nearest-even on the float32 bit pattern.
Outlier positions are drawn without replacement.  Any shape can be asked
for, so the same recipe yields small parity cases with a ragged tail.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    "c1": (256, 1024),
    "c2": (8192, 4096),
    "c3": (14336, 4096),
    "c4": (8192, 14336),
    "c5": (16384, 8192),
}


def f32_to_bf16_bits(x) -> np.ndarray:
    """float -> bf16 bit patterns (uint16), round to nearest even."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16).reshape(f.shape)


def bf16_bits_to_f32(b) -> np.ndarray:
    b = np.asarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def _scatter_outliers(v: np.ndarray, rng, frac: float, factor: float) -> np.ndarray:
    flat = v.reshape(-1)
    k = int(np.floor(frac * flat.size))
    if k:
        pos = rng.choice(flat.size, size=k, replace=False)
        flat[pos] *= factor
    return v


def gen(workload: str, rows: int | None = None, cols: int | None = None,
        seed: int | None = None) -> np.ndarray:
    """bf16 bits [rows][cols] for a named workload (default: its full shape)."""
    k = int(workload[1:])
    r0, c0 = WORKLOADS[workload]
    rows = r0 if rows is None else rows
    cols = c0 if cols is None else cols
    rng = _rng(1000 + k if seed is None else seed)
    n = rows * cols
    if workload == "c1":
        v = rng.standard_normal(n, dtype=np.float32).reshape(rows, cols)
        v = _scatter_outliers(v, rng, 0.001, 50.0)
    elif workload == "c2":
        colscale = np.exp(rng.standard_normal(cols))            # lognormal(0,1)
        z = rng.standard_normal((rows, cols))
        u1 = rng.random((rows, cols))
        u2 = rng.random((rows, cols))
        chi2 = -2.0 * np.log((1.0 - u1) * (1.0 - u2))            # chi-square, 4 dof
        chi2 = np.maximum(chi2, 1e-300)
        v = (z / np.sqrt(chi2 / 4.0)) * colscale[None, :]
    elif workload == "c3":
        v = (0.02 * rng.standard_normal(n, dtype=np.float32)).reshape(rows, cols)
    elif workload == "c4":
        u = rng.random(n) - 0.5
        w = np.maximum(-2.0 * np.abs(u), -1.0 + 2.0**-53)
        v = (-1e-3 * np.sign(u) * np.log1p(w)).reshape(rows, cols)
        v = _scatter_outliers(v, rng, 0.0005, 100.0)
    elif workload == "c5":
        rowscale = np.exp(0.5 * rng.standard_normal(rows))       # lognormal(0,0.5)
        v = rng.standard_normal((rows, cols), dtype=np.float32) * rowscale[:, None].astype(np.float32)
    else:
        raise KeyError(workload)
    return f32_to_bf16_bits(v)


def special_values_tensor(rows: int, cols: int, seed: int = 7) -> np.ndarray:
    """A tensor mixing the edge cases a quantizer meets: zeros, -0, bf16
    subnormals, all-equal blocks, large and tiny magnitudes side by side,
    and random normals.  Values are grouped per 16-wide block so that whole
    blocks exercise one case each."""
    rng = _rng(seed)
    v = rng.standard_normal((rows, cols)).astype(np.float32)
    bits = f32_to_bf16_bits(v)
    nb = cols // 16
    kinds = rng.integers(0, 8, size=(rows, nb))
    for r in range(rows):
        for b in range(nb):
            sl = slice(16 * b, 16 * b + 16)
            kd = kinds[r, b]
            if kd == 0:
                bits[r, sl] = 0x0000                                   # +0 block
            elif kd == 1:
                bits[r, sl] = 0x8000                                   # -0 block
            elif kd == 2:
                bits[r, sl] = rng.integers(1, 0x80, 16) | (rng.integers(0, 2, 16) << 15)  # subnormals
            elif kd == 3:
                bits[r, sl] = bits[r, 16 * b]                          # all equal
            elif kd == 4:
                bits[r, sl] = f32_to_bf16_bits(v[r, sl] * 1e-6)        # tiny block
            elif kd == 5:
                w = v[r, sl].copy()
                w[rng.integers(0, 16)] *= 1000.0                        # one outlier
                bits[r, sl] = f32_to_bf16_bits(w)
            # kinds 6, 7: plain normals
    return bits


def random_nvfp4(rows: int, cols: int, seed: int = 3, zero_frac: float = 0.02):
    """Bytes of an arbitrary 1D NVFP4 tensor [rows][cols]: uniform random
    packed codes (every nibble, both signs) and E4M3 scale codes 1..126
    (normal and subnormal, never the NaN code), with a fraction of blocks
    given scale code 0.  Returns (codes [rows][cols/2], scales [rows][cols/16])."""
    rng = _rng(seed)
    codes = rng.integers(0, 256, size=(rows, cols // 2), dtype=np.uint8)
    scales = rng.integers(1, 127, size=(rows, cols // 16), dtype=np.uint8)
    scales[rng.random(scales.shape) < zero_frac] = 0
    return codes, scales
