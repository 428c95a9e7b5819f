// rows_kernels.h -- NVFP4 with one FP32 scale per row: quantization in one
// read of the input.
//
// The NVIDIA NVFP4 article (sec. 9) names the extra pass over memory for
// the tensor's global scale as a cost and proposes finer-grained global
// scales, per row or per block.  Here every row r takes its own
// alpha_r = amax_r / (6 C) ("Four Over Six" Eq. 1 on the row; amax after
// RHT16 when asked) and is otherwise quantized exactly as the per-tensor
// quantizer quantizes it (Eq. 2-3, the 4/6 choice, SR with the element index
// in the whole tensor as Philox counter).
//
// Mapping onto the chip.  Short rows (up to 128 blocks): one wave owns one
// row at a time (persistent waves, rows strided over the grid); its lanes
// load the row's 16-value blocks, reduce the row maximum across the wave
// (DPP), build the row's (s, 1/s) table of every E4M3 code in the wave's
// slice of LDS, and quantize the blocks still held in registers while the
// next row's loads are in flight -- no barrier at all.  Longer rows: one
// workgroup per row, so that a pipeline stage stays as small as the
// per-tensor quantizer's (one wave per row would put half the tensor in
// flight before any SIMD starts); the row maximum then takes one barrier and
// the table a second.  Rows up to 16384 values stay in registers and are
// read once; longer ones are swept twice, the second sweep re-reading the
// row from cache.
#pragma once

#include "device_common.h"
#include "nvfp4_kernels.h"

namespace fp4q {

constexpr int kRowThreads = 256;
constexpr int kRowWaves = kRowThreads / 64;
#ifndef FP4Q_ROW_WG_PER_CU
#define FP4Q_ROW_WG_PER_CU 6
#endif
constexpr int kRowWgPerCu = FP4Q_ROW_WG_PER_CU;   // cap on resident workgroups per CU
// Workgroups launched per resident one by the workgroup-per-row kernel: the
// later ones start as the first ones finish and take the rows that a fixed
// share would leave to the youngest resident workgroups, which the hardware
// serves last (8192x4096 4/6: 19.5 -> 17.7 us).
constexpr int kRowWgLaunch = 3;

// The 16 values of a block from its two 16-byte halves, rotated by RHT16
// when asked.
template <bool RHT>
__device__ __forceinline__ void row_block_values(const uint4& v0, const uint4& v1, uint32_t signs,
                                                 float* y) {
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
}

// A wave's NB blocks per lane of one row (or row chunk); separate
// compile-time-indexed members, so they stay in registers.
template <int NB>
struct RowRegs {
  uint4 v[NB][2];
};

// Load chunk c of a row into R; blocks past the row's end (or every block,
// when the row is past the tensor: nbytes = 0) read as zeros through the
// resource bounds, so the loads are never conditional.
template <int NB>
__device__ __forceinline__ void row_load(RowRegs<NB>& R, const uint16_t* xr, int64_t nblk,
                                         int64_t c, bool live, int lane) {
  constexpr int kChunk = 64 * NB;
  const int64_t b0 = c * kChunk;
  const int64_t nb = !live ? 0 : (nblk - b0 < kChunk ? nblk - b0 : kChunk);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(xr + b0 * 16), 0, (int)(nb * 32), 0x00020000);
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    R.v[i][0] = buffer_load16(r, 32 * (lane + 64 * i));
    R.v[i][1] = buffer_load16(r, 32 * (lane + 64 * i) + 16);
  });
}

template <bool RHT, int NB>
__device__ __forceinline__ float row_chunk_max(const RowRegs<NB>& R, uint32_t signs, float m) {
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    float y[16];
    row_block_values<RHT>(R.v[i][0], R.v[i][1], signs, y);
#pragma unroll
    for (int k = 0; k < 16; k++) m = fmaxf(m, fabsf(y[k]));
  });
  return m;
}

// The row's constants from its amax, and its (s, 1/s) table for every E4M3
// code (code 127 copies 126) in the wave's LDS slice, two entries per lane.
template <bool FOUR_SIX>
__device__ __forceinline__ TensorScale row_constants(float m, float2* tab, int lane) {
  const TensorScale ts = tensor_scale(wave_max_nonneg(m), FOUR_SIX);
  wave_lds_sync();                                        // the last row's reads are done
#pragma unroll
  for (int e = lane; e < 128; e += 64) {
    const float s = ts.alpha * e4m3_value(e < 127 ? (uint32_t)e : 126u);
    tab[e] = make_float2(s, s == 0.0f ? 0.0f : 1.0f / s);
  }
  wave_lds_sync();
  return ts;
}

// Quantize chunk c of row `row` (indices fixed at compile time, so R stays
// in registers even where the SR block code is too long to unroll a loop).
// Stores go through buffer resources over the row's outputs (scalar base,
// 32-bit lane offsets), which costs the texture addresser less than 64-bit
// per-lane addresses.
template <bool FOUR_SIX, bool SR, bool RHT, int NB>
__device__ __forceinline__ void row_chunk_quant(const RowRegs<NB>& R, int64_t row, int64_t cols,
                                                int64_t nblk, int64_t c, const float2* tab,
                                                const TensorScale& ts, uint32_t signs,
                                                uint32_t seed_lo, uint32_t seed_hi, int lane,
                                                uint8_t* codes, uint8_t* scales, uint8_t* choice) {
  const int64_t b0 = c * (64 * NB);
  const int nb = (int)(nblk - b0 < 64 * NB ? nblk - b0 : 64 * NB);
  const int64_t blk0 = row * nblk + b0;                  // first block of the chunk
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(codes + 8 * blk0, 0, 8 * nb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(scales + blk0, 0, nb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      choice ? choice + blk0 : scales, 0, choice ? nb : 0, 0x00020000);
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int j = 64 * i + lane;                          // block within the chunk
    if (j < nb) {
      float y[16];
      row_block_values<RHT>(R.v[i][0], R.v[i][1], signs, y);
      const BlockOut o = quant_block<FOUR_SIX, SR>(y, tab, ts.k6, ts.k4, (blk0 + j) * 16,
                                                    seed_lo, seed_hi);
      i32x2_t cw;
      cw.x = (int)o.w0;
      cw.y = (int)o.w1;
      __builtin_amdgcn_raw_buffer_store_b64(cw, rc, 8 * j, 0, kStoreNT);
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)o.scale, rs, j, 0, kStoreNT);
      if (choice) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)o.pick4, rh, j, 0, kStoreNT);
    }
  });
}

// Rows of at most 64 * NB blocks, one wave each: a row is read once and the
// next row's loads are in flight while it is quantized (two register sets
// in turn).
template <bool FOUR_SIX, bool SR, bool RHT, int NB>
__global__ __launch_bounds__(kRowThreads) void nvfp4_rows_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, float* __restrict__ alpha_rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ choice,
    uint32_t seed_lo, uint32_t seed_hi) {
  __shared__ float2 tabs[kRowWaves][128];
  // the wave index through readfirstlane: provably uniform, so row indices
  // and buffer resources live in scalar registers (a per-lane resource would
  // make the compiler loop over lanes around every load)
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  float2* tab = tabs[wave];
  const int64_t nblk = cols / 16;
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;
  const int64_t stride = (int64_t)gridDim.x * kRowWaves;
  int64_t row = (int64_t)blockIdx.x * kRowWaves + wave;

  {
    auto process = [&](const RowRegs<NB>& R, int64_t r) {
      const TensorScale ts = row_constants<FOUR_SIX>(row_chunk_max<RHT>(R, signs, 0.0f), tab, lane);
      if (lane == 0) alpha_rows[r] = ts.alpha;
      row_chunk_quant<FOUR_SIX, SR, RHT>(R, r, cols, nblk, 0, tab, ts, signs, seed_lo, seed_hi,
                                         lane, codes, scales, choice);
    };
    RowRegs<NB> A, B;
    row_load(A, x + row * cols, nblk, 0, row < rows, lane);
    while (row < rows) {
      const int64_t rb = row + stride;
      row_load(B, x + rb * cols, nblk, 0, rb < rows, lane);
      process(A, row);
      if (rb >= rows) break;
      const int64_t ra = rb + stride;
      row_load(A, x + ra * cols, nblk, 0, ra < rows, lane);
      process(B, rb);
      row = ra;
    }
  }
}

// ------------------------------------------------------------------------
// Rows of more than 128 blocks: a whole workgroup per row.  Thread t holds
// blocks t + 256 i (i < NB) of the row, so one row is one stage of a
// pipeline as fine as the per-tensor quantizer's (8 KB per workgroup for a
// 4096-value row); the row maximum goes wave max -> LDS -> one barrier, the
// table is built by 128 threads -> a second barrier.  The next row's loads
// are in flight meanwhile (two register sets in turn).

template <int NB>
__device__ __forceinline__ void wgrow_load(RowRegs<NB>& R, const uint16_t* xr, int64_t nblk,
                                           int64_t c, bool live) {
  constexpr int kChunk = kRowThreads * NB;
  const int64_t b0 = c * kChunk;
  const int64_t nb = !live ? 0 : (nblk - b0 < kChunk ? nblk - b0 : kChunk);
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc((void*)(xr + b0 * 16), 0, (int)(nb * 32), 0x00020000);
  const int t = threadIdx.x;
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    R.v[i][0] = buffer_load16(r, 32 * (t + kRowThreads * i));
    R.v[i][1] = buffer_load16(r, 32 * (t + kRowThreads * i) + 16);
  });
}

// The row's constants from the threads' partial maxima, and its table, in
// one wave (the row's index picks which, so the work rotates over the
// SIMDs), with two division sequences instead of one per table entry:
//  * lanes 0-2 divide alpha = amax / (6 C), k6 = C / amax, k4 = 1.5 C / amax;
//  * an E4M3 value is k 2^j with k in 1..15, k = k_odd 2^t, and for every
//    tensor in the method's domain all the products and reciprocals below
//    are normal fp32 numbers, so scaling by powers of two commutes with
//    rounding: fl(alpha Delta) = fl(alpha k_odd) 2^(t+j) and
//    fl(1 / fl(alpha Delta)) = fl(1 / fl(alpha k_odd)) 2^-(t+j).  Lanes 0-7
//    divide the eight bases (k_odd = 1, 3, ..., 15); every table entry is
//    then two exact ldexp's of a base.
// Thread 0 of that wave passes alpha, k6, k4 on through LDS behind the
// barrier the table needs anyway.
template <bool FOUR_SIX>
__device__ __forceinline__ TensorScale wgrow_constants(float m, int64_t row, float* red,
                                                       float2* tab, float2* bases, float* kc) {
  const float wm = wave_max_nonneg(m);
  const int lane = threadIdx.x & 63;
  if (lane == 0) red[threadIdx.x >> 6] = wm;
  __syncthreads();                                  // partials written; last row's table read
  if ((int)(threadIdx.x >> 6) == (int)(row & (kRowWaves - 1))) {
    const float rm = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    const float C = FOUR_SIX ? 256.0f : 448.0f;
    // one division sequence: lane 0 alpha, lane 1 k6, lane 2 k4
    const float num = lane == 0 ? rm : (lane == 1 ? C : 1.5f * C);
    const float den = lane == 0 ? 6.0f * C : rm;
    float q = num / den;
    q = (lane > 0 && rm == 0.0f) ? 0.0f : q;
    const float alpha = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(q), 0));
    if (lane < 3) kc[lane] = q;
    // the second: the eight bases (alpha k_odd, 1 / that)
    const float base = alpha * (float)(2 * (lane & 7) + 1);
    const float rbase = base == 0.0f ? 0.0f : 1.0f / base;
    if (lane < 8) bases[lane] = make_float2(base, rbase);
    wave_lds_sync();
#pragma unroll
    for (int e = lane; e < 128; e += 64) {
      const uint32_t code = e < 127 ? (uint32_t)e : 126u;   // code 127 copies 126
      const uint32_t ex = code >> 3, mt = code & 7u;
      const uint32_t k = ex ? 8u + mt : mt;                 // Delta = k 2^j
      const int j = ex ? (int)ex - 10 : -9;
      const int t = __builtin_ctz(k | 16u);                 // k = k_odd 2^t (k = 0: t = 4)
      const float2 b = bases[((k >> t) - 1) >> 1 & 7];
      tab[e] = k == 0u ? make_float2(0.0f, 0.0f)
                       : make_float2(__builtin_ldexpf(b.x, t + j), __builtin_ldexpf(b.y, -(t + j)));
    }
  }
  __syncthreads();                                  // table and constants ready
  TensorScale ts;
  ts.alpha = kc[0];
  ts.k6 = kc[1];
  ts.k4 = kc[2];
  return ts;
}

// Values kept between the two steps of a row: with one block per thread
// its 16 (rotated) values, otherwise only each block's maximum (the values
// are unpacked again from the raw registers).
template <int NB>
struct RowKeep {
  float y[NB == 1 ? 16 : 1];
  float amax[NB];
};

template <bool RHT, int NB>
__device__ __forceinline__ float wgrow_chunk_max(const RowRegs<NB>& R, uint32_t signs,
                                                 RowKeep<NB>& K, float m) {
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    float y[16];
    row_block_values<RHT>(R.v[i][0], R.v[i][1], signs, y);
    K.amax[i] = block_amax16(y);
    m = fmaxf(m, K.amax[i]);
    if constexpr (NB == 1) {
#pragma unroll
      for (int k = 0; k < 16; k++) K.y[k] = y[k];
    }
  });
  return m;
}

template <bool FOUR_SIX, bool SR, bool RHT, int NB>
__device__ __forceinline__ void wgrow_chunk_quant(const RowRegs<NB>& R, const RowKeep<NB>& K,
                                                  int64_t row, int64_t nblk, int64_t c,
                                                  const float2* tab, const TensorScale& ts,
                                                  uint32_t signs, uint32_t seed_lo,
                                                  uint32_t seed_hi, uint8_t* codes,
                                                  uint8_t* scales, uint8_t* choice) {
  constexpr int kChunk = kRowThreads * NB;
  const int64_t b0 = c * kChunk;
  const int nb = (int)(nblk - b0 < kChunk ? nblk - b0 : kChunk);
  const int64_t blk0 = row * nblk + b0;
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(codes + 8 * blk0, 0, 8 * nb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(scales + blk0, 0, nb, 0x00020000);
  const __amdgpu_buffer_rsrc_t rh = __builtin_amdgcn_make_buffer_rsrc(
      choice ? choice + blk0 : scales, 0, choice ? nb : 0, 0x00020000);
  static_for<NB>([&](auto ic) {
    constexpr int i = decltype(ic)::value;
    const int j = threadIdx.x + kRowThreads * i;
    if (j < nb) {
      float y[16];
      if constexpr (NB == 1) {
#pragma unroll
        for (int k = 0; k < 16; k++) y[k] = K.y[k];
      } else {
        row_block_values<RHT>(R.v[i][0], R.v[i][1], signs, y);
      }
      const BlockOut o = quant_block_m<FOUR_SIX, SR>(y, K.amax[i], tab, ts.k6, ts.k4,
                                                      (blk0 + j) * 16, seed_lo, seed_hi);
      i32x2_t cw;
      cw.x = (int)o.w0;
      cw.y = (int)o.w1;
      __builtin_amdgcn_raw_buffer_store_b64(cw, rc, 8 * j, 0, kStoreNT);
      __builtin_amdgcn_raw_buffer_store_b8((unsigned char)o.scale, rs, j, 0, kStoreNT);
      if (choice) __builtin_amdgcn_raw_buffer_store_b8((unsigned char)o.pick4, rh, j, 0, kStoreNT);
    }
  });
}

template <bool FOUR_SIX, bool SR, bool RHT, int NB, bool ONE>
__global__ __launch_bounds__(kRowThreads) void nvfp4_rows_wg_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, float* __restrict__ alpha_rows,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ choice,
    uint32_t seed_lo, uint32_t seed_hi) {
  __shared__ float2 tab[128];
  __shared__ float red[kRowWaves];
  __shared__ float kc[3];
  __shared__ float2 bases[8];
  const int64_t nblk = cols / 16;
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;
  const int64_t stride = gridDim.x;
  int64_t row = blockIdx.x;

  if constexpr (ONE) {
    auto process = [&](const RowRegs<NB>& R, int64_t r) {
      RowKeep<NB> K;
      const TensorScale ts = wgrow_constants<FOUR_SIX>(wgrow_chunk_max<RHT>(R, signs, K, 0.0f), r,
                                                       red, tab, bases, kc);
      if (threadIdx.x == 0) alpha_rows[r] = ts.alpha;
      wgrow_chunk_quant<FOUR_SIX, SR, RHT>(R, K, r, nblk, 0, tab, ts, signs, seed_lo, seed_hi,
                                           codes, scales, choice);
    };
    RowRegs<NB> A, B;
    wgrow_load(A, x + row * cols, nblk, 0, row < rows);
    while (row < rows) {
      const int64_t rb = row + stride;
      wgrow_load(B, x + rb * cols, nblk, 0, rb < rows);
      process(A, row);
      if (rb >= rows) break;
      const int64_t ra = rb + stride;
      wgrow_load(A, x + ra * cols, nblk, 0, ra < rows);
      process(B, rb);
      row = ra;
    }
  } else {
    const int64_t nchunk = (nblk + kRowThreads * NB - 1) / (kRowThreads * NB);
    for (; row < rows; row += stride) {
      const uint16_t* xr = x + row * cols;
      RowRegs<NB> R;
      RowKeep<NB> K;
      float m = 0.0f;
      for (int64_t c = 0; c < nchunk; c++) {
        wgrow_load(R, xr, nblk, c, true);
        m = wgrow_chunk_max<RHT>(R, signs, K, m);
      }
      const TensorScale ts = wgrow_constants<FOUR_SIX>(m, row, red, tab, bases, kc);
      if (threadIdx.x == 0) alpha_rows[row] = ts.alpha;
      for (int64_t c = 0; c < nchunk; c++) {
        wgrow_load(R, xr, nblk, c, true);
        // the chunk's block maxima, again (K holds the last chunk's)
        wgrow_chunk_max<RHT>(R, signs, K, 0.0f);
        wgrow_chunk_quant<FOUR_SIX, SR, RHT>(R, K, row, nblk, c, tab, ts, signs, seed_lo,
                                             seed_hi, codes, scales, choice);
      }
    }
  }
}

}  // namespace fp4q
