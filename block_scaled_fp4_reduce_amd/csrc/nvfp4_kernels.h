// nvfp4_kernels.h -- NVFP4 tensor amax and 1D block quantizer for gfx950.
//
// Method: "Four Over Six" (sec. 2.1, Eq. 1-3; sec. 1, Fig. 1 and the
// worked example) and the NVIDIA NVFP4 pretraining article (sec. 2: random
// Hadamard, stochastic rounding; sec. 6: global and local encode scales).
//
// Mapping onto the chip: one lane owns one 16-value block (32 bytes of
// bf16 read as two 16-byte loads), so the per-block scale work is done once
// per block and never shuffled; a wave covers 64 consecutive blocks, i.e.
// 2 KiB of input, 512 B of codes and 64 scale bytes, each stored with one
// coalesced instruction.  The tensor scale comes from the amax pass as a
// small array of per-workgroup partial maxima that every workgroup reduces
// itself while its own input loads are in flight.
#pragma once

#include "device_common.h"

namespace fp4q {

// ------------------------------------------------------------------ amax
// Per-workgroup partial maxima of |x| (or of |RHT16(x)|), as fp32 bit
// patterns: non-negative floats order like their bit patterns, so the max
// is an exact, order-free integer max.
#ifndef FP4Q_AMAX_GROUPS
#define FP4Q_AMAX_GROUPS 256
#endif
#ifndef FP4Q_AMAX_THREADS
#define FP4Q_AMAX_THREADS 1024
#endif
#ifndef FP4Q_AMAX_UNROLL
#define FP4Q_AMAX_UNROLL 4
#endif
#ifndef FP4Q_AMAX_THREADS_1D
#define FP4Q_AMAX_THREADS_1D 512
#endif
#ifndef FP4Q_AMAX_GROUPS_1D
#define FP4Q_AMAX_GROUPS_1D 512
#endif
#ifndef FP4Q_BPT
#define FP4Q_BPT 1
#endif
#ifndef FP4Q_WG_PER_CU
#define FP4Q_WG_PER_CU 12
#endif
#ifndef FP4Q_HW_E4M3
#define FP4Q_HW_E4M3 1
#endif
constexpr int kAmaxMaxGroups = FP4Q_AMAX_GROUPS;
constexpr int kAmaxUnroll = FP4Q_AMAX_UNROLL;
constexpr int kAmaxThreads = FP4Q_AMAX_THREADS;
// The amax pass ahead of the 1D quantizer takes smaller workgroups: 512
// threads on 32 KiB chunks, up to 512 of them (full 8192x4096 4/6 step
// 25.8 -> 25.3 us); the 2D quantizer's step is faster after the larger ones
// (62.8 against 63.7 us), so it and the rotated pass keep those.
constexpr int kAmaxThreads1d = FP4Q_AMAX_THREADS_1D;
constexpr int kAmaxMaxGroups1d = FP4Q_AMAX_GROUPS_1D;
constexpr int kAmaxMaxGroupsAll = kAmaxMaxGroups > kAmaxMaxGroups1d ? kAmaxMaxGroups : kAmaxMaxGroups1d;
constexpr int kBpt = FP4Q_BPT;              // 16-value blocks per lane per chunk (1D quantizer)
// Workgroups launched per CU by the 1D quantizer with SR and by MS-EDEN.
// Their Philox work needs about 100 VGPRs, so four waves per SIMD are
// resident; launching three times as many workgroups as fit (the others
// start as the first ones finish) evens out the end of the grid, where a
// fixed split leaves the CUs that hold the youngest workgroups busy last
// (8192x14336 RHT16 + SR: 175 -> 170 us; MS-EDEN: 61 -> 59 us).
constexpr int kWgPerCu = FP4Q_WG_PER_CU;
// Without SR the 1D quantizer needs at most 64 VGPRs, so six 4-wave
// workgroups fit per CU (six waves per SIMD), which covers its loads better
// than four (8192x4096 4/6: quantize 17.3 -> 16.4 us).
#ifndef FP4Q_WG_PER_CU_NOSR
#define FP4Q_WG_PER_CU_NOSR 6
#endif
constexpr int kWgPerCuNoSr = FP4Q_WG_PER_CU_NOSR;

template <bool RHT, int THREADS>
__global__ __launch_bounds__(THREADS) void amax_partial_kernel(
    const uint4* __restrict__ x, int64_t ngroups16, uint32_t* __restrict__ partials,
    uint32_t seed_lo, uint32_t seed_hi) {
  __shared__ uint32_t red[THREADS / 64];
  uint32_t m = 0;
  if constexpr (!RHT) {
    // Magnitude bits of two bf16 per dword; packed 16-bit integer max.
    // Workgroups walk chunks of THREADS * kAmaxUnroll 16-byte vectors
    // with a stride of the grid; a buffer resource per chunk makes loads
    // past the end read 0, so every load is issued unconditionally and the
    // next chunk is in flight while this one is reduced.
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    constexpr int64_t CH = (int64_t)THREADS * kAmaxUnroll;
    const int64_t nvec = ngroups16 * 2;            // 8 bf16 per uint4
    const int64_t nch = (nvec + CH - 1) / CH;
    auto rsrc = [&](int64_t c) {
      const int64_t left = c < nch ? nvec - c * CH : 0;
      return buffer_rsrc(x + (c < nch ? c : 0) * CH, (left < CH ? left : CH) * 16);
    };
    struct Chunk {
      uint4 v[kAmaxUnroll];
    };
    auto load = [&](int64_t c, Chunk& k) {
      const __amdgpu_buffer_rsrc_t r = rsrc(c);
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; u++)
        k.v[u] = buffer_load16(r, (u * THREADS + (int)threadIdx.x) * 16);
    };
    u16x2 mm = {0, 0};
    Chunk cur, nxt;
    int64_t c = blockIdx.x;
    load(c, cur);
    for (; c < nch; c += gridDim.x) {
      load(c + gridDim.x, nxt);
#pragma unroll
      for (int u = 0; u < kAmaxUnroll; u++) {
        const uint32_t w[4] = {cur.v[u].x, cur.v[u].y, cur.v[u].z, cur.v[u].w};
#pragma unroll
        for (int k = 0; k < 4; k++) {
          const uint32_t a = w[k] & 0x7FFF7FFFu;
          mm = __builtin_elementwise_max(mm, __builtin_bit_cast(u16x2, a));
        }
      }
      cur = nxt;
    }
    const uint32_t lo = mm.x, hi = mm.y;
    m = (lo > hi ? lo : hi) << 16;
  } else {
    const uint32_t signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;
    const int64_t stride = (int64_t)gridDim.x * THREADS;
    const int64_t g = (int64_t)blockIdx.x * THREADS + threadIdx.x;
    float fm = 0.0f;
    for (int64_t i = g; i < ngroups16; i += stride) {
      const uint4 v0 = x[2 * i], v1 = x[2 * i + 1];
      float y[16];
      unpack8(v0, y);
      unpack8(v1, y + 8);
#pragma unroll
      for (int k = 0; k < 16; k++)
        y[k] = __uint_as_float(__float_as_uint(y[k]) ^ (((signs >> k) & 1u) << 31));
      fwht<16>(y);
#pragma unroll
      for (int k = 0; k < 16; k++) fm = fmaxf(fm, fabsf(y[k] * 0.25f));
    }
    m = __float_as_uint(fm);
  }
  m = block_max_u32<THREADS>(m, red);
  if (threadIdx.x == 0) partials[blockIdx.x] = m;
}

// One workgroup: reduce the partials and store the amax as a float.
__global__ __launch_bounds__(kThreads) void amax_finalize_kernel(
    const uint32_t* __restrict__ partials, int n, float* __restrict__ amax_out) {
  __shared__ uint32_t red[kThreads / 64];
  uint32_t m = 0;
  for (int i = threadIdx.x; i < n; i += kThreads) m = m > partials[i] ? m : partials[i];
  m = block_max_u32(m, red);
  if (threadIdx.x == 0) *amax_out = __uint_as_float(m);
}

// ------------------------------------------------------------------ quantizer
// Tensor-level constants derived from the tensor amax.
struct TensorScale {
  float alpha;   // decode scale, Eq. 1: amax / (6 * C)
  float k6, k4;  // encode factors (6*C/M) / amax: the block scale before
                 // E4M3 rounding is amax_b * k_M (Eq. 2 via the global
                 // encode scale of the NVIDIA article, sec. 6)
};

__device__ __forceinline__ TensorScale tensor_scale(float amax, bool four_six) {
  const float C = four_six ? 256.0f : 448.0f;
  TensorScale t;
  t.alpha = amax / (6.0f * C);
  t.k6 = amax == 0.0f ? 0.0f : C / amax;
  t.k4 = amax == 0.0f ? 0.0f : (1.5f * C) / amax;
  return t;
}

// Scale table in LDS: for every E4M3 code, (s, r) = (alpha*Delta, 1/(alpha*Delta))
// with r = 0 when s = 0.  Replaces two per-block divisions by one lookup.
__device__ __forceinline__ void build_scale_table(float2* tab, float alpha) {
  if (threadIdx.x < 128) {
    const uint32_t code = threadIdx.x < 127 ? threadIdx.x : 126u;
    const float s = alpha * e4m3_value(code);
    tab[threadIdx.x] = make_float2(s, s == 0.0f ? 0.0f : 1.0f / s);
  }
}

// The same table over all 256 byte values, for lookups by the raw byte the
// FP8 conversion writes: bytes with the sign bit set (from NaN input only)
// read the entry of their low seven bits.  Needs 256 threads.
__device__ __forceinline__ void build_scale_table256(float2* tab, float alpha) {
  static_assert(kThreads == 256, "one table entry per thread");
  const uint32_t low = threadIdx.x & 0x7Fu;
  const uint32_t code = low < 127 ? low : 126u;
  const float s = alpha * e4m3_value(code);
  tab[threadIdx.x] = make_float2(s, s == 0.0f ? 0.0f : 1.0f / s);
}

// Error of one dequantized pair against its inputs, accumulated with fma
// into the NEGATED running sum: nacc' = fma(d, -d, nacc) = -(d*d + acc) with
// one rounding, and round-to-nearest-even is symmetric, so nacc stays
// exactly -acc at every step.  (The negated form makes the compiler emit the
// three-address v_fma_f32 with a negated operand instead of the accumulating
// v_fmac_f32, which issues at about half its rate on gfx950.)
template <int BYTE>
__device__ __forceinline__ float nerr_pair(uint32_t packed, float s, float y0, float y1,
                                           float nacc) {
  const float2_t q = fp4x2_to_f32<BYTE>(packed, 1.0f);
  const float d0 = __builtin_fmaf(q.x, s, -y0);
  nacc = __builtin_fmaf(d0, -d0, nacc);
  const float d1 = __builtin_fmaf(q.y, s, -y1);
  return __builtin_fmaf(d1, -d1, nacc);
}

// Nearest-even quantization of 16 values with encode scale r; returns the
// two code dwords and the block's squared error of q*s against y, summed as
// two fma chains (elements 0..7 and 8..15) that are then added.
__device__ __forceinline__ float quant16_rtn(const float* y, float s, float r, uint32_t& w0,
                                             uint32_t& w1) {
  // the four byte-wise conversions per word overwrite every byte of w0/w1
  w0 = cvt_fp4x2<0>(w0, y[0] * r, y[1] * r, 1.0f);
  w0 = cvt_fp4x2<1>(w0, y[2] * r, y[3] * r, 1.0f);
  w0 = cvt_fp4x2<2>(w0, y[4] * r, y[5] * r, 1.0f);
  w0 = cvt_fp4x2<3>(w0, y[6] * r, y[7] * r, 1.0f);
  w1 = cvt_fp4x2<0>(w1, y[8] * r, y[9] * r, 1.0f);
  w1 = cvt_fp4x2<1>(w1, y[10] * r, y[11] * r, 1.0f);
  w1 = cvt_fp4x2<2>(w1, y[12] * r, y[13] * r, 1.0f);
  w1 = cvt_fp4x2<3>(w1, y[14] * r, y[15] * r, 1.0f);
  // the two chains from +0, kept negated (from -0): see nerr_pair
  float nlo = -0.0f, nhi = -0.0f;
  nlo = nerr_pair<0>(w0, s, y[0], y[1], nlo);
  nlo = nerr_pair<1>(w0, s, y[2], y[3], nlo);
  nlo = nerr_pair<2>(w0, s, y[4], y[5], nlo);
  nlo = nerr_pair<3>(w0, s, y[6], y[7], nlo);
  nhi = nerr_pair<0>(w1, s, y[8], y[9], nhi);
  nhi = nerr_pair<1>(w1, s, y[10], y[11], nhi);
  nhi = nerr_pair<2>(w1, s, y[12], y[13], nhi);
  nhi = nerr_pair<3>(w1, s, y[14], y[15], nhi);
  return -(nlo + nhi);                            // = lo + hi exactly
}

// Stochastic rounding of t onto the FP4 grid: between neighbours lo <= |t| < hi
// round up iff u < (|t| - lo)/(hi - lo), u = (philox word 0 >> 8) * 2^-24 for
// counter = element index.  Returns the signed grid value.
__device__ __forceinline__ float sr_value(float t, uint64_t idx, uint32_t k0, uint32_t k1) {
  const uint32_t w = philox_w0((uint32_t)idx, (uint32_t)(idx >> 32), 0u, 0u, k0, k1);
  const float u = (float)(w >> 8) * 0x1p-24f;
  const float a = fabsf(t);
  // grid spacing 0.5 / 1 / 2 on [0, 2) / [2, 4) / [4, 6): with inv = 1/spacing
  // (2, 1 or 0.5), lo = floor(a * inv) / inv and p = (a - lo) * inv are exact
  // (power-of-two scalings of exact values), i.e. the division of the
  // definition done as a multiply
  const float inv = a < 2.0f ? 2.0f : (a < 4.0f ? 1.0f : 0.5f);
  const float step = a < 2.0f ? 0.5f : (a < 4.0f ? 1.0f : 2.0f);
  const float lo = __builtin_floorf(a * inv) * step;
  const float p = (a - lo) * inv;
  float mag = u < p ? lo + step : lo;
  mag = a < 6.0f ? mag : 6.0f;                  // saturate (also NaN-free for Inf)
  return __builtin_copysignf(mag, t);
}

__device__ __forceinline__ float quant16_sr(const float* y, float s, float r, uint64_t idx0,
                                            uint32_t k0, uint32_t k1, uint32_t& w0, uint32_t& w1) {
  float q[16];
#pragma unroll
  for (int i = 0; i < 16; i++) q[i] = sr_value(y[i] * r, idx0 + i, k0, k1);
  // grid values convert exactly; every byte of w0/w1 is overwritten
  w0 = cvt_fp4x2<0>(w0, q[0], q[1], 1.0f);
  w0 = cvt_fp4x2<1>(w0, q[2], q[3], 1.0f);
  w0 = cvt_fp4x2<2>(w0, q[4], q[5], 1.0f);
  w0 = cvt_fp4x2<3>(w0, q[6], q[7], 1.0f);
  w1 = cvt_fp4x2<0>(w1, q[8], q[9], 1.0f);
  w1 = cvt_fp4x2<1>(w1, q[10], q[11], 1.0f);
  w1 = cvt_fp4x2<2>(w1, q[12], q[13], 1.0f);
  w1 = cvt_fp4x2<3>(w1, q[14], q[15], 1.0f);
  (void)s;
  return 0.0f;
}

// E4M3 codes of two non-negative block scales.  The hardware conversion
// (OCP E4M3, nearest-even) is used after a clamp to [0, 448], so values past
// the largest finite E4M3 saturate; the result indexes the 128-entry scale
// table (code 0x7F, unreachable for finite input, maps to a copy of 448).
__device__ __forceinline__ void e4m3_pair(float a, float b, uint32_t& ca, uint32_t& cb) {
#if FP4Q_HW_E4M3
  const float a2 = __builtin_amdgcn_fmed3f(a, 0.0f, 448.0f);
  const float b2 = __builtin_amdgcn_fmed3f(b, 0.0f, 448.0f);
  const uint32_t w = (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, b2, 0, false);
  ca = w & 0x7Fu;
  cb = (w >> 8) & 0x7Fu;
#else
  ca = e4m3_rne(a);
  cb = e4m3_rne(b);
#endif
}

// Both E4M3 codes in one word: byte 0 is the code of a, byte 1 that of b
// (after the same clamp to [0, 448] as e4m3_pair; the upper half is
// arbitrary).  `any` is any live value: the conversion keeps the upper half
// of its destination, so no register needs clearing first.
__device__ __forceinline__ uint32_t e4m3_pair_word(float a, float b, uint32_t any) {
  const float a2 = __builtin_amdgcn_fmed3f(a, 0.0f, 448.0f);
  const float b2 = __builtin_amdgcn_fmed3f(b, 0.0f, 448.0f);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a2, b2, (int)any, false);
}

// One quantized 16-value block: its two code words, E4M3 scale code and
// 4/6 choice (1 where M = 4 won).
struct BlockOut {
  uint32_t w0, w1, scale, pick4;
};

// Quantize the 16-value block y whose first element has index idx in its
// row-major tensor (the SR counter), with the (s, 1/s) table and encode
// factors of its scale.
// The block's largest magnitude, max |y_k| from +0.
__device__ __forceinline__ float block_amax16(const float* y) {
  float amax_b = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++) amax_b = fmaxf(amax_b, fabsf(y[k]));
  return amax_b;
}

// quant_block with the block's amax (block_amax16(y)) already known.
template <bool FOUR_SIX, bool SR>
__device__ __forceinline__ BlockOut quant_block_m(const float* y, float amax_b, const float2* tab,
                                                  float k6, float k4, int64_t idx,
                                                  uint32_t seed_lo, uint32_t seed_hi) {
  uint32_t e6, e4;
  e4m3_pair(amax_b * k6, amax_b * k4, e6, e4);
  const float2 sr6 = tab[e6];
  BlockOut o;
  o.w0 = __builtin_nondeterministic_value(0u);
  o.w1 = __builtin_nondeterministic_value(0u);
  o.scale = e6;
  o.pick4 = 0;
  if constexpr (SR) {
    quant16_sr(y, sr6.x, sr6.y, (uint64_t)idx, seed_lo, seed_hi, o.w0, o.w1);
  } else {
    const float err6 = quant16_rtn(y, sr6.x, sr6.y, o.w0, o.w1);
    if constexpr (FOUR_SIX) {
      const float2 sr4 = tab[e4];
      uint32_t u0 = __builtin_nondeterministic_value(0u), u1 = __builtin_nondeterministic_value(0u);
      const float err4 = quant16_rtn(y, sr4.x, sr4.y, u0, u1);
      o.pick4 = err4 < err6 ? 1u : 0u;    // ties keep M = 6
      o.w0 = o.pick4 ? u0 : o.w0;
      o.w1 = o.pick4 ? u1 : o.w1;
      o.scale = o.pick4 ? e4 : e6;
    }
  }
  return o;
}

template <bool FOUR_SIX, bool SR>
__device__ __forceinline__ BlockOut quant_block(const float* y, const float2* tab, float k6,
                                                float k4, int64_t idx, uint32_t seed_lo,
                                                uint32_t seed_hi) {
  return quant_block_m<FOUR_SIX, SR>(y, block_amax16(y), tab, k6, k4, idx, seed_lo, seed_hi);
}

// quant_block, stored for a 1D block layout: codes at idx / 2, scale and
// choice at idx / 16.
template <bool FOUR_SIX, bool SR>
__device__ __forceinline__ void quant_block_at(const float* y, const float2* tab, float k6,
                                               float k4, int64_t idx, uint32_t seed_lo,
                                               uint32_t seed_hi, uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               uint8_t* __restrict__ choice) {
  const BlockOut o = quant_block<FOUR_SIX, SR>(y, tab, k6, k4, idx, seed_lo, seed_hi);
  *(uint2*)(codes + idx / 2) = make_uint2(o.w0, o.w1);
  scales[idx / 16] = (uint8_t)o.scale;
  if (choice) choice[idx / 16] = (uint8_t)o.pick4;
}

// Quantize the lane's 16-value block (raw bf16 in v0, v1) and store codes,
// scale and choice at byte offsets 8*lane / lane / lane of the chunk's
// output resources.
template <bool FOUR_SIX, bool SR, bool RHT>
__device__ __forceinline__ void nvfp4_block(uint4 v0, uint4 v1, int64_t b, const float2* tab,
                                            float k6, float k4, uint32_t signs, uint32_t seed_lo,
                                            uint32_t seed_hi, __amdgpu_buffer_rsrc_t rc,
                                            __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rh,
                                            bool want_choice) {
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
  float amax_b = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; k++) amax_b = fmaxf(amax_b, fabsf(y[k]));

  // scale bytes straight from the conversion word: byte 0 (M = 6) and
  // byte 1 (M = 4) index the 256-entry table as byte offsets
  const uint32_t ew = e4m3_pair_word(amax_b * k6, amax_b * k4, v1.w);
  const char* tb = (const char*)tab;
  const float2 sr6 = *(const float2*)(tb + ((ew & 0xFFu) << 3));
  // every byte of the code words is written by the conversions, so they
  // start from whatever the input registers hold (no clearing instruction)
  uint32_t w0 = v0.x, w1 = v0.y;
  uint32_t scale = ew, pick4 = 0;             // the store keeps the low byte
  if constexpr (SR) {
    quant16_sr(y, sr6.x, sr6.y, (uint64_t)b * 16, seed_lo, seed_hi, w0, w1);
  } else {
    const float err6 = quant16_rtn(y, sr6.x, sr6.y, w0, w1);
    if constexpr (FOUR_SIX) {
      const float2 sr4 = *(const float2*)(tb + (((ew >> 8) & 0xFFu) << 3));
      uint32_t u0 = v0.z, u1 = v0.w;
      const float err4 = quant16_rtn(y, sr4.x, sr4.y, u0, u1);
      pick4 = err4 < err6 ? 1u : 0u;      // ties keep M = 6
      w0 = pick4 ? u0 : w0;
      w1 = pick4 ? u1 : w1;
      scale = pick4 ? ew >> 8 : ew;
    }
  }
  const int lane = threadIdx.x;
  i32x2_t cw;
  cw.x = (int)w0;
  cw.y = (int)w1;
  __builtin_amdgcn_raw_buffer_store_b64(cw, rc, 8 * lane, 0, kStoreNT);
  __builtin_amdgcn_raw_buffer_store_b8((unsigned char)scale, rs, lane, 0, kStoreNT);
  if (want_choice)
    __builtin_amdgcn_raw_buffer_store_b8((unsigned char)pick4, rh, lane, 0, kStoreNT);
}

// 1D NVFP4: one lane per 16-value block of the flattened tensor (blocks never
// straddle rows because cols % 16 == 0).  Persistent workgroups walk chunks
// of kThreads blocks with a stride of the grid, with two register buffers:
// chunk i+1 is loaded while chunk i is computed, so memory and VALU work
// overlap and the tensor-scale prologue runs once per workgroup.  All global
// accesses go through per-chunk buffer resources (uniform base in SGPRs,
// 32-bit lane offsets, hardware bounds on the last chunk).
//   amax_bits/namax: values whose max is the tensor amax (fp32 bit patterns):
//   the amax pass partials, or the caller's amax_in (namax = 1).
template <bool FOUR_SIX, bool SR, bool RHT>
__global__ __launch_bounds__(kThreads) void nvfp4_1d_kernel(
    const uint4* __restrict__ x, int64_t nblocks, const uint32_t* __restrict__ amax_bits,
    int namax, float* __restrict__ alpha_out, uint2* __restrict__ codes,
    uint8_t* __restrict__ scales, uint8_t* __restrict__ choice, uint32_t seed_lo,
    uint32_t seed_hi) {
  __shared__ float2 tab[256];
  __shared__ float kshared[2];
  __shared__ uint32_t red[kThreads / 64];
  // chunk indices fit in 32 bits (rows*cols < 2^40 -> < 2^28 chunks), which
  // keeps the per-chunk bookkeeping on the scalar unit
  const int nchunks = (int)((nblocks + kThreads - 1) / kThreads);
  const int tail = (int)(nblocks - (int64_t)(nchunks - 1) * kThreads);   // blocks in the last chunk
  const int G = gridDim.x;
  const int lane = threadIdx.x;
  const bool want_choice = choice != nullptr;
  // blocks in chunk cc: none outside [0, nchunks) (signed compares: with an
  // empty tensor nchunks - 1 is -1)
  auto nblk = [&](int cc) {
    return (cc >= 0 && cc < nchunks - 1) ? kThreads : (cc == nchunks - 1 && cc >= 0 ? tail : 0);
  };
  // Chunk order.  The amax pass leaves the last quarter or so of what each
  // XCD read in that XCD's L2 (it takes chunks of R = 4 of these 8 KiB
  // chunks, chunk a on XCD a % 8 when its grid is a multiple of 8, in rising
  // order).  With a grid that is a multiple of 8, workgroups here take
  // virtual chunk indices v = w + i G and map them so that XCD x gets
  // exactly the 8 KiB chunks q with (q / R) % 8 == x, highest first:
  // k = (G/8) i + w/8 counts XCD x's chunks, q = 8R (top - k/R) + R x + k % R.
  // The virtual range is padded to a multiple of 8R; indices past the end
  // map to chunks >= nchunks, which read and write nothing.  Not used with
  // RHT16 (its amax pass walks the tensor in another order, and the kernel
  // is ALU-bound).
  constexpr int R = kAmaxThreads1d * kAmaxUnroll * 16 / (kThreads * 32);
  static_assert(R >= 1 && (R & (R - 1)) == 0, "amax chunk: a power-of-two number of 8 KiB chunks");
  const bool remap_on = !RHT && (G & 7) == 0;
  const int top = nchunks > 0 ? (nchunks - 1) / (8 * R) : -1;
  const int nvirt = remap_on ? 8 * R * (top + 1) : nchunks;
  // v = blockIdx.x + i G is this workgroup's i-th virtual chunk
  const int k0 = (int)blockIdx.x >> 3, x0 = (int)blockIdx.x & 7, kstep = G >> 3;
  auto chunk_of = [&](int v, int i) {
    if (!remap_on) return v;
    if (v >= nvirt) return nchunks;                     // prefetch past the end: nothing
    const int k = kstep * i + k0;
    return 8 * R * (top - k / R) + R * x0 + k % R;
  };
  auto in_rsrc = [&](int v, int i) {
    const int cc = chunk_of(v, i);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint4*>(x + 2 * (int64_t)cc * kThreads), 0,
                                             nblk(cc) * 32, 0x00020000);
  };

  // Loads are unconditional: a chunk past the end gets a zero-size resource
  // and reads zeros without touching memory, so no branch separates a
  // prefetch from its consumer.
  int c = blockIdx.x;
  uint4 a0, a1, b0, b1;
  {                                        // in flight during the prologue
    const __amdgpu_buffer_rsrc_t r = in_rsrc(c, 0);
    a0 = buffer_load16(r, 32 * lane);
    a1 = buffer_load16(r, 32 * lane + 16);
  }

  uint32_t m = 0;
  if ((namax & 3) == 0 && (((uintptr_t)amax_bits) & 15) == 0) {
    for (int i = lane; 4 * i < namax; i += kThreads) {   // 16-byte loads of the partials
      const uint4 a = ((const uint4*)amax_bits)[i];
      m = max(m, max(max(a.x, a.y), max(a.z, a.w)));
    }
  } else {
    for (int i = lane; i < namax; i += kThreads) {
      const uint32_t a = amax_bits[i];
      m = m > a ? m : a;
    }
  }
  m = block_max_u32(m, red);
  {                                        // every lane: one table entry
    const TensorScale ts = tensor_scale(__uint_as_float(m), FOUR_SIX);
    build_scale_table256(tab, ts.alpha);
    if (lane == 0) {
      kshared[0] = ts.k6;
      kshared[1] = ts.k4;
      if (blockIdx.x == 0) *alpha_out = ts.alpha;
    }
  }
  __syncthreads();
  const float k6 = kshared[0], k4 = kshared[1];
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;

  auto process = [&](int v, int i, uint4 v0, uint4 v1) __attribute__((always_inline)) {
    const int cc = chunk_of(v, i);
    const int n = nblk(cc);
    const int64_t b0 = (int64_t)cc * kThreads;
    nvfp4_block<FOUR_SIX, SR, RHT>(
        v0, v1, b0 + lane, tab, k6, k4, signs, seed_lo, seed_hi,
        __builtin_amdgcn_make_buffer_rsrc(codes + b0, 0, n * 8, 0x00020000),
        __builtin_amdgcn_make_buffer_rsrc(scales + b0, 0, n, 0x00020000),
        __builtin_amdgcn_make_buffer_rsrc(want_choice ? choice + b0 : scales, 0, want_choice ? n : 0,
                                          0x00020000),
        want_choice);
  };

  // Two chunks per trip, the next one's loads in flight.  The first trip is
  // peeled off the loop so that the loop is entered with the same loads and
  // stores in flight as at its back edge: the compiler then waits only for
  // the chunk about to be computed, not for the previous chunk's stores.
  int it = 0;                              // c = blockIdx.x + it G
  // (forced inline: out of line, the registers it shares would live in scratch)
  auto trip = [&]() __attribute__((always_inline)) -> bool {   // false: no chunk left after it
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

// ------------------------------------------------------------------ dequantize
// NVFP4: out = q * (alpha * Delta); one lane per 16 values.
__global__ __launch_bounds__(kThreads) void nvfp4_dequant_kernel(
    const uint2* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ alpha, int64_t nblocks, int64_t bcols, bool two_d,
    float4* __restrict__ out) {
  const int64_t b = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (b >= nblocks) return;
  const int64_t row = b / bcols, bc = b - row * bcols;
  const int64_t sidx = two_d ? (row / 16) * bcols + bc : b;
  const float s = alpha[0] * e4m3_value(scales[sidx] & 0x7Fu);
  const uint2 c = codes[b];
  float q[16];
  float2_t t;
  t = fp4x2_to_f32<0>(c.x, 1.0f); q[0] = t.x; q[1] = t.y;
  t = fp4x2_to_f32<1>(c.x, 1.0f); q[2] = t.x; q[3] = t.y;
  t = fp4x2_to_f32<2>(c.x, 1.0f); q[4] = t.x; q[5] = t.y;
  t = fp4x2_to_f32<3>(c.x, 1.0f); q[6] = t.x; q[7] = t.y;
  t = fp4x2_to_f32<0>(c.y, 1.0f); q[8] = t.x; q[9] = t.y;
  t = fp4x2_to_f32<1>(c.y, 1.0f); q[10] = t.x; q[11] = t.y;
  t = fp4x2_to_f32<2>(c.y, 1.0f); q[12] = t.x; q[13] = t.y;
  t = fp4x2_to_f32<3>(c.y, 1.0f); q[14] = t.x; q[15] = t.y;
#pragma unroll
  for (int k = 0; k < 4; k++)
    out[4 * b + k] = make_float4(q[4 * k] * s, q[4 * k + 1] * s, q[4 * k + 2] * s, q[4 * k + 3] * s);
}

// MXFP4: out = q * 2^(code - 127); one lane per 32 values.
__global__ __launch_bounds__(kThreads) void mxfp4_dequant_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales, int64_t ngroups,
    float4* __restrict__ out) {
  const int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (g >= ngroups) return;
  const uint32_t sc = scales[g];
  // 2^(sc-127) as a float; sc = 0 is the subnormal 2^-127
  const float s = sc ? __uint_as_float(sc << 23) : __uint_as_float(0x00400000u);
  const uint4 c = codes[g];
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int k = 0; k < 4; k++) {
    const float2_t a = fp4x2_to_f32<0>(w[k], 1.0f), b2 = fp4x2_to_f32<1>(w[k], 1.0f);
    const float2_t c2 = fp4x2_to_f32<2>(w[k], 1.0f), d = fp4x2_to_f32<3>(w[k], 1.0f);
    out[8 * g + 2 * k] = make_float4(a.x * s, a.y * s, b2.x * s, b2.y * s);
    out[8 * g + 2 * k + 1] = make_float4(c2.x * s, c2.y * s, d.x * s, d.y * s);
  }
}

}  // namespace fp4q
