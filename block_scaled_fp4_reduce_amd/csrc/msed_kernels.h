// msed_kernels.h -- MS-EDEN NVFP4 quantization (Quartet II / MS-EDEN
// article, sec. 1): the 16-value block is rotated (RHT16), its FP4 values
// are rounded to nearest, and the randomness sits only in the E4M3 block
// scale.  The unbiasing factor is EDEN's (Vargaftik et al. 2022): values
// are rounded against the unrounded block scale Delta_pre = amax_b * k6,
// the scale is multiplied by S = sum t^2 / sum t q (which keeps the
// dequantized block's projection on the rotated input equal to its squared
// norm) and rounded stochastically onto the E4M3 grid, one Philox draw per
// block.  C = 256, as for Four Over Six, so S > 1 has room below 448.
//
// Mapping onto the chip: the per-tensor quantizer's structure (one block
// per lane, 256 blocks per workgroup step, persistent workgroups, next
// step's loads in flight); per block two IEEE divisions (1/s and N/D) and
// one Philox call replace the 4/6 search, so the kernel costs about what
// plain rounding to nearest does.
#pragma once

#include "device_common.h"
#include "nvfp4_kernels.h"

namespace fp4q {

// Stochastic rounding of a block scale d (E4M3 units) onto the E4M3 grid:
// between neighbours lo <= d < hi up iff u < (d - lo) / (hi - lo); both the
// subtraction and the division by the power-of-two spacing are exact.
// Returns the E4M3 code; d >= 448 gives 448, d <= 0 gives 0.
__device__ __forceinline__ uint32_t e4m3_sr(float d, float u) {
  if (!(d > 0.0f)) return 0u;
  if (d >= 448.0f) return 0x7Eu;
  int E = (int)((__float_as_uint(d) >> 23) & 0xFFu) - 127;   // floor(log2 d) for normal d
  E = E < -6 ? -6 : E;                                        // subnormal E4M3 share 2^-6's step
  const float inv_q = __builtin_ldexpf(1.0f, 3 - E);          // 1 / spacing
  const float nf = __builtin_floorf(d * inv_q);               // lo = nf * spacing
  const float p = d * inv_q - nf;                             // (d - lo) / spacing, exact
  const int n = (int)nf + (u < p ? 1 : 0);
  const int code = ((E + 7) << 3) + n - 8;                    // n = 16 carries into the exponent
  return (uint32_t)(code > 0x7E ? 0x7E : code);
}

// One MS-EDEN block from its raw bf16 (v0, v1); stores through the chunk's
// output resources at byte offsets 8*lane / lane / lane.
template <bool RHT>
__device__ __forceinline__ void msed_block(uint4 v0, uint4 v1, int64_t b, float alpha, float k6,
                                           uint32_t signs, uint32_t seed_lo, uint32_t seed_hi,
                                           __amdgpu_buffer_rsrc_t rc, __amdgpu_buffer_rsrc_t rs,
                                           __amdgpu_buffer_rsrc_t rh, bool want_choice) {
  float y[16];
  unpack8(v0, y);
  unpack8(v1, y + 8);
  if constexpr (RHT) {
#pragma unroll
    for (int k = 0; k < 16; k++)
      y[k] = __uint_as_float(__float_as_uint(y[k]) ^ (((signs >> k) & 1u) << 31));
    fwht<16>(y);
#pragma unroll
    for (int k = 0; k < 16; k++) y[k] = y[k] * 0.25f;
  }
  const float dpre = block_amax16(y) * k6;
  const float s = alpha * dpre;
  const float r = s == 0.0f ? 0.0f : 1.0f / s;
  float t[16];
#pragma unroll
  for (int k = 0; k < 16; k++) t[k] = y[k] * r;
  uint32_t w0 = __builtin_nondeterministic_value(0u), w1 = __builtin_nondeterministic_value(0u);
  w0 = cvt_fp4x2<0>(w0, t[0], t[1], 1.0f);
  w0 = cvt_fp4x2<1>(w0, t[2], t[3], 1.0f);
  w0 = cvt_fp4x2<2>(w0, t[4], t[5], 1.0f);
  w0 = cvt_fp4x2<3>(w0, t[6], t[7], 1.0f);
  w1 = cvt_fp4x2<0>(w1, t[8], t[9], 1.0f);
  w1 = cvt_fp4x2<1>(w1, t[10], t[11], 1.0f);
  w1 = cvt_fp4x2<2>(w1, t[12], t[13], 1.0f);
  w1 = cvt_fp4x2<3>(w1, t[14], t[15], 1.0f);
  // N = sum t^2, D = sum t q: two fma chains each (elements 0..7, 8..15), added
  float n_lo = 0.0f, n_hi = 0.0f, d_lo = 0.0f, d_hi = 0.0f;
  static_for<4>([&](auto jc) {
    constexpr int j = decltype(jc)::value;
    const float2_t qa = fp4x2_to_f32<j>(w0, 1.0f), qb = fp4x2_to_f32<j>(w1, 1.0f);
    n_lo = __builtin_fmaf(t[2 * j], t[2 * j], n_lo);
    d_lo = __builtin_fmaf(t[2 * j], qa.x, d_lo);
    n_lo = __builtin_fmaf(t[2 * j + 1], t[2 * j + 1], n_lo);
    d_lo = __builtin_fmaf(t[2 * j + 1], qa.y, d_lo);
    n_hi = __builtin_fmaf(t[8 + 2 * j], t[8 + 2 * j], n_hi);
    d_hi = __builtin_fmaf(t[8 + 2 * j], qb.x, d_hi);
    n_hi = __builtin_fmaf(t[9 + 2 * j], t[9 + 2 * j], n_hi);
    d_hi = __builtin_fmaf(t[9 + 2 * j], qb.y, d_hi);
  });
  const float N = n_lo + n_hi, D = d_lo + d_hi;
  const float S = D > 0.0f ? N / D : 1.0f;
  const uint32_t w = philox_w0((uint32_t)b, (uint32_t)((uint64_t)b >> 32), 1u, 0u, seed_lo, seed_hi);
  const uint32_t scale = e4m3_sr(S * dpre, (float)(w >> 8) * 0x1p-24f);
  const int lane = threadIdx.x;
  i32x2_t cw;
  cw.x = (int)w0;
  cw.y = (int)w1;
  __builtin_amdgcn_raw_buffer_store_b64(cw, rc, 8 * lane, 0, kStoreNT);
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)scale, rs, lane, 0, kStoreNT);
  if (want_choice) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)0, rh, lane, 0, kStoreNT);
}

// The per-tensor quantizer's loop with the MS-EDEN block (see
// nvfp4_1d_kernel: 256 blocks per chunk, persistent workgroups, the next
// chunk's loads issued before the current chunk is processed).
template <bool RHT>
__global__ __launch_bounds__(kThreads) void nvfp4_msed_kernel(
    const uint4* __restrict__ x, int64_t nblocks, const uint32_t* __restrict__ amax_bits,
    int namax, float* __restrict__ alpha_out, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ choice, uint32_t seed_lo,
    uint32_t seed_hi) {
  __shared__ uint32_t red[kThreads / 64];
  const int nchunks = (int)((nblocks + kThreads - 1) / kThreads);
  const int tail = (int)(nblocks - (int64_t)(nchunks - 1) * kThreads);
  const int G = gridDim.x;
  const int lane = threadIdx.x;
  const bool want_choice = choice != nullptr;
  auto nblk = [&](int cc) {
    return (cc >= 0 && cc < nchunks - 1) ? kThreads : (cc == nchunks - 1 && cc >= 0 ? tail : 0);
  };
  // Chunk order, as in the 1D quantizer: the rotated amax pass reads the
  // tensor in 32 KiB pieces (its 1024 threads one block each), piece a on
  // XCD a % 8 in rising order, so with a grid that is a multiple of 8, XCD
  // x takes the 8 KiB chunks of the pieces it read, highest first, and part
  // of them is still in its L2.  Only right after that pass (namax > 1):
  // with the amax given, nothing is in cache and the plain order is faster
  // (8192x14336: 59.3 against 58.2 us; full step 88.7 -> 87.1 us).
  constexpr int R = kAmaxThreads * 32 / (kThreads * 32);
  static_assert(R >= 1 && (R & (R - 1)) == 0, "rotated amax piece: a power-of-two number of chunks");
  const bool remap_on = (G & 7) == 0 && namax > 1;
  const int top = nchunks > 0 ? (nchunks - 1) / (8 * R) : -1;
  const int nvirt = remap_on ? 8 * R * (top + 1) : nchunks;
  const int k0 = (int)blockIdx.x >> 3, x0 = (int)blockIdx.x & 7, kstep = G >> 3;
  auto chunk_of = [&](int v, int i) {
    if (!remap_on) return v;
    if (v >= nvirt) return nchunks;                     // past the end: nothing
    const int k = kstep * i + k0;
    return 8 * R * (top - k / R) + R * x0 + k % R;
  };
  auto in_rsrc = [&](int v, int i) {
    const int cc = chunk_of(v, i);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(x + 2 * (int64_t)cc * kThreads), 0,
                                             nblk(cc) * 32, 0x00020000);
  };
  int c = blockIdx.x, it = 0;                           // c = blockIdx.x + it G
  uint4 a0, a1, b0, b1;
  {
    const __amdgpu_buffer_rsrc_t r = in_rsrc(c, 0);
    a0 = buffer_load16(r, 32 * lane);
    a1 = buffer_load16(r, 32 * lane + 16);
  }
  uint32_t m = 0;
  for (int i = lane; i < namax; i += kThreads) {
    const uint32_t a = amax_bits[i];
    m = m > a ? m : a;
  }
  m = block_max_u32(m, red);
  const TensorScale ts = tensor_scale(__uint_as_float(m), true);   // C = 256
  if (blockIdx.x == 0 && lane == 0) *alpha_out = ts.alpha;
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;

  auto process = [&](int v, int i, uint4 v0, uint4 v1) __attribute__((always_inline)) {
    const int cc = chunk_of(v, i);
    const int n = nblk(cc);
    const int64_t bb = (int64_t)cc * kThreads;
    msed_block<RHT>(v0, v1, bb + lane, ts.alpha, ts.k6, signs, seed_lo, seed_hi,
                    __builtin_amdgcn_make_buffer_rsrc(codes + bb, 0, n * 8, 0x00020000),
                    __builtin_amdgcn_make_buffer_rsrc(scales + bb, 0, n, 0x00020000),
                    __builtin_amdgcn_make_buffer_rsrc(want_choice ? choice + bb : scales, 0,
                                                      want_choice ? n : 0, 0x00020000),
                    want_choice);
  };

  // Two chunks per trip, the next one's loads in flight; the first trip is
  // peeled off the loop so that the loop is entered with the same loads and
  // stores in flight as at its back edge, and each wait covers only the
  // chunk about to be computed (as in the 1D quantizer).
  auto trip = [&]() __attribute__((always_inline)) -> bool {
    const int cb = c + G;
    {
      const __amdgpu_buffer_rsrc_t r = in_rsrc(cb, it + 1);
      b0 = buffer_load16(r, 32 * lane);
      b1 = buffer_load16(r, 32 * lane + 16);
    }
    process(c, it, a0, a1);
    if (cb >= nvirt) return false;
    const int ca = cb + G;
    {
      const __amdgpu_buffer_rsrc_t r = in_rsrc(ca, it + 2);
      a0 = buffer_load16(r, 32 * lane);
      a1 = buffer_load16(r, 32 * lane + 16);
    }
    process(cb, it + 1, b0, b1);
    c = ca;
    it += 2;
    return true;
  };
  if (c < nvirt && trip()) {
    while (c < nvirt) {
      if (!trip()) break;
    }
  }
}

}  // namespace fp4q
