// requant_kernels.h -- requantization of a 1D NVFP4 tensor for the
// transposed operand: NVFP4 of dequantize(X)^T, with the output's own
// tensor scale and any 1D mode (RTN6, Four Over Six, SR, RHT16).
//
// Method: Quartet II / MS-EDEN article sec. 2 (the backward pass quantizes
// part of the data again); NVIDIA NVFP4 article sec. 7 (the weight gradient
// contracts over the other dimension, so its operand needs blocks along the
// other axis).  Dequantization is q * (alpha * Delta) in fp32 (the decode of
// sec. 6 of that article); the quantization is Eq. 1-3 of "Four Over Six" on
// those fp32 values.
//
// Mapping onto the chip.  An output block is 16 consecutive input rows of
// one input column.  A thread loads one dword (8 codes) from each of 16
// consecutive input rows, plus the 16 matching scale bytes: that is 8 whole
// output blocks, transposed in registers with no LDS.  A workgroup of 512
// threads covers a 256 x 256 input tile -- 16 row segments x 32 groups of
// 8 columns -- so each of its 256 output rows gets one complete 128-byte
// line of codes from one CU (no partial lines shared between L2s), and a
// wave's loads read two 128-byte input row pieces per instruction.
// Tiles are taken in super-tile-major order (8 x 8 super-tiles), and each
// XCD takes one contiguous eighth of that order, its persistent workgroups
// striding through it: the tiles of a super-tile run on one XCD at the same
// time, so the eight tiles side by side that share each 128-byte line of
// input scales, and the eight stacked tiles that share each line of output
// scales, meet in one L2, while every XCD gets the same number of tiles.
// A first pass computes the output's tensor amax (after RHT16 when asked)
// the same way.
#pragma once

#include "device_common.h"
#include "nvfp4_kernels.h"

namespace fp4q {

constexpr int kRqThreads = 512;
constexpr int kRqTileRows = 256;   // 16 segments of 16 input rows
constexpr int kRqTileCols = 256;   // 32 groups of 8 input columns
// Workgroups launched per CU: two fit at once; the other two start as the
// first ones finish and even out the end of the grid (8192x14336 gradient
// requantization: 191 -> 186 us).
constexpr int kRqWgPerCu = 4;
constexpr int kRqSuper = 8;           // tiles per side of an XCD super-tile
constexpr int kRqAmaxGroups = 1024;   // most partial maxima the amax pass writes

// The 16 dequantized values of column pair B of the thread's 8 columns
// (columns 2B and 2B+1) down its 16 rows.
template <int B>
__device__ __forceinline__ void rq_column_pair(const uint32_t* cw, const float* sc, float* ya,
                                               float* yb) {
#pragma unroll
  for (int k = 0; k < 16; k++) {
    const float2_t q = fp4x2_to_f32<B>(cw[k], 1.0f);
    ya[k] = q.x * sc[k];
    yb[k] = q.y * sc[k];
  }
}

template <bool RHT>
__device__ __forceinline__ void rq_rotate(float* y, uint32_t signs) {
  if constexpr (RHT) {
#pragma unroll
    for (int k = 0; k < 16; k++)
      y[k] = __uint_as_float(__float_as_uint(y[k]) ^ (((signs >> k) & 1u) << 31));
    fwht<16>(y);
#pragma unroll
    for (int k = 0; k < 16; k++) y[k] = y[k] * 0.25f;
  }
}

// The j-th tile in super-tile-major order: kRqSuper x kRqSuper super-tiles
// row by row, tiles row-major inside each (the last super-row and
// super-column may be smaller).  Tile counts stay below 2^29.
__device__ __forceinline__ TileOrder rq_tile(uint32_t j, uint32_t TY, uint32_t TX) {
  const uint32_t sy = j / (kRqSuper * TX), r = j - sy * kRqSuper * TX;
  const uint32_t h = min((uint32_t)kRqSuper, TY - kRqSuper * sy);
  const uint32_t sx = r / (kRqSuper * h), within = r - sx * kRqSuper * h;
  const uint32_t w = min((uint32_t)kRqSuper, TX - kRqSuper * sx);
  const uint32_t wy = within / w;
  TileOrder t;
  t.ty = kRqSuper * sy + wy;
  t.tx = kRqSuper * sx + (within - wy * w);
  return t;
}

// This workgroup's tiles: j, j + step, ... below end.  With a grid that is
// a multiple of 8, workgroup b runs on XCD b % 8 and that XCD owns tiles
// [x n / 8, (x + 1) n / 8) of the order above; other grids share one range.
struct RqRange {
  uint32_t j, end, step;
};

__device__ __forceinline__ RqRange rq_range(uint32_t ntiles) {
  const uint32_t nx = gridDim.x % kXcds == 0 ? kXcds : 1;
  const uint32_t x = blockIdx.x % nx, k = blockIdx.x / nx;
  RqRange q;
  q.j = (uint32_t)((uint64_t)ntiles * x / nx) + k;
  q.end = (uint32_t)((uint64_t)ntiles * (x + 1) / nx);
  q.step = gridDim.x / nx;
  return q;
}

// Where a thread's segment of a tile sits, and whether it is inside the
// tensor (rows % 16 == 0 and cols % 16 == 0 make each segment of 16 rows x
// 8 columns wholly inside or wholly outside).
struct RqSeg {
  int64_t r0, c0;   // first input row and column
  bool in;
};

__device__ __forceinline__ RqSeg rq_seg(const TileOrder& to, int64_t rows, int64_t cols) {
  const int t = threadIdx.x, cg = t & 31, s = t >> 5;
  RqSeg g;
  g.r0 = to.ty * kRqTileRows + 16 * s;
  g.c0 = to.tx * kRqTileCols + 8 * cg;
  g.in = g.r0 < rows && g.c0 < cols;
  return g;
}

// Codes (one dword per row) and decode scales alpha * Delta of a segment.
__device__ __forceinline__ void rq_load(const uint8_t* __restrict__ codes,
                                        const uint8_t* __restrict__ scales, float alpha,
                                        int64_t cols, const RqSeg& g, uint32_t* cw, float* sc) {
  const uint8_t* cp = codes + g.r0 * (cols / 2) + g.c0 / 2;
  const uint8_t* sp = scales + g.r0 * (cols / 16) + g.c0 / 16;
  uint32_t sb[16];
#pragma unroll
  for (int k = 0; k < 16; k++) {
    cw[k] = *(const uint32_t*)(cp + k * (cols / 2));
    sb[k] = sp[k * (cols / 16)];
  }
#pragma unroll
  for (int k = 0; k < 16; k++) sc[k] = alpha * e4m3_value(sb[k] & 0x7Fu);
}

// Pass 1: per-workgroup maxima of |output values| as fp32 bit patterns.
template <bool RHT>
__global__ __launch_bounds__(kRqThreads) void rq_amax_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ alpha_in, int64_t rows, int64_t cols, uint32_t TY, uint32_t TX,
    uint32_t* __restrict__ partials, uint32_t seed_lo, uint32_t seed_hi) {
  __shared__ uint32_t red[kRqThreads / 64];
  const float alpha = *alpha_in;
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;
  float m = 0.0f;
  for (RqRange q = rq_range(TY * TX); q.j < q.end; q.j += q.step) {
    const RqSeg g = rq_seg(rq_tile(q.j, TY, TX), rows, cols);
    if (!g.in) continue;
    uint32_t cw[16];
    float sc[16];
    rq_load(codes, scales, alpha, cols, g, cw, sc);
    auto pair = [&](auto bc) {
      constexpr int B = decltype(bc)::value;
      float ya[16], yb[16];
      rq_column_pair<B>(cw, sc, ya, yb);
      rq_rotate<RHT>(ya, signs);
      rq_rotate<RHT>(yb, signs);
#pragma unroll
      for (int k = 0; k < 16; k++) m = fmaxf(m, fmaxf(fabsf(ya[k]), fabsf(yb[k])));
    };
    pair(std::integral_constant<int, 0>{});
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 3>{});
  }
  const uint32_t mb = block_max_u32<kRqThreads>(__float_as_uint(m), red);
  if (threadIdx.x == 0) partials[blockIdx.x] = mb;
}

// Pass 2: quantize with the tensor scale from the partial maxima.
template <bool FOUR_SIX, bool SR, bool RHT>
__global__ __launch_bounds__(kRqThreads) void rq_quant_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const float* __restrict__ alpha_in, int64_t rows, int64_t cols, uint32_t TY, uint32_t TX,
    const uint32_t* __restrict__ partials, int npart,
    float* __restrict__ alpha_out, uint8_t* __restrict__ codes_t,
    uint8_t* __restrict__ scales_t, uint8_t* __restrict__ choice_t, uint32_t seed_lo,
    uint32_t seed_hi) {
  __shared__ float2 tab[128];
  __shared__ uint32_t red[kRqThreads / 64];
  const float alpha = *alpha_in;
  uint32_t m = 0;
  for (int i = threadIdx.x; i < npart; i += kRqThreads) m = max(m, partials[i]);
  m = block_max_u32<kRqThreads>(m, red);
  const TensorScale ts = tensor_scale(__uint_as_float(m), FOUR_SIX);
  if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_out = ts.alpha;
  build_scale_table(tab, ts.alpha);
  uint32_t signs = 0;
  if constexpr (RHT) signs = philox_w0(0u, 0u, 0u, 1u, seed_lo, seed_hi) & 0xFFFFu;
  __syncthreads();

  for (RqRange q = rq_range(TY * TX); q.j < q.end; q.j += q.step) {
    const RqSeg g = rq_seg(rq_tile(q.j, TY, TX), rows, cols);
    if (!g.in) continue;
    uint32_t cw[16];
    float sc[16];
    rq_load(codes, scales, alpha, cols, g, cw, sc);
    // output rows g.c0 + j (input columns), output block starting at g.r0
    auto pair = [&](auto bc) {
      constexpr int B = decltype(bc)::value;
      float ya[16], yb[16];
      rq_column_pair<B>(cw, sc, ya, yb);
      rq_rotate<RHT>(ya, signs);
      rq_rotate<RHT>(yb, signs);
      // element index in the output: output row g.c0 + j, column g.r0
      quant_block_at<FOUR_SIX, SR>(ya, tab, ts.k6, ts.k4, (g.c0 + 2 * B) * rows + g.r0, seed_lo,
                                   seed_hi, codes_t, scales_t, choice_t);
      quant_block_at<FOUR_SIX, SR>(yb, tab, ts.k6, ts.k4, (g.c0 + 2 * B + 1) * rows + g.r0,
                                   seed_lo, seed_hi, codes_t, scales_t, choice_t);
    };
    pair(std::integral_constant<int, 0>{});
    pair(std::integral_constant<int, 1>{});
    pair(std::integral_constant<int, 2>{});
    pair(std::integral_constant<int, 3>{});
  }
}

}  // namespace fp4q
