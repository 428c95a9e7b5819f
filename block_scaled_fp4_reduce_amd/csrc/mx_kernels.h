// mx_kernels.h -- MXFP4 quantization with an optional 32-point Hadamard,
// row-wise and column-wise outputs from one read of the input.
//
// Method: NVIDIA NVFP4 article sec. 1 and sec. 5 (MXFP4: 32 values share a
// power-of-two UE8M0 scale); AMD MI355X MXFP4 pretraining article sec. 2
// (a fixed, deterministic Hadamard rotation before quantizing, for both
// operands of the weight-gradient product, hence both orientations).
//
// Mapping onto the chip.  A workgroup of 16 waves (one per CU, four per
// SIMD; 8 waves run 6 % slower) owns a 256x256 region,
// processed as four 128x128 tiles, each staged through LDS, so every global
// access is a full, coalesced segment (the kernel is bound by the memory
// pipeline, not by arithmetic, once the rotation runs on the matrix cores):
//  1. a tile is read with 16-byte non-temporal loads, 16 lanes per
//     256-byte row piece, and written to LDS (the loads of the next three
//     tiles are already in flight);
//  2. each wave quantizes one 32x32 block row-wise and one column-wise
//     (two each with 8 waves),
//     staging codes and scales of the whole region in LDS;
//  3. after the region's fourth tile, every region row (and column) leaves
//     as one full 128-byte code line (eight lanes of 16 bytes) and 8 scale
//     bytes, so no output line is written in pieces from two places.
// With the rotation, the 32-point transforms are dense 32x32 products (the
// Hadamard matrix H, entries +-1, exact in bf16) on the matrix cores:
// v_mfma_f32_32x32x16_bf16 twice per 32x32 block, products exact and sums
// accumulated in fp32 in the hardware's order (rotated values may differ
// from a butterfly's in the last bits: the accepted tolerance for rotated
// paths).  Without it, each lane reads its values straight from LDS in the
// same layout, and the results are exact.
//
// Instruction layout (lane l, element j = 0..7; verified on the device):
//   A[m][k]: m = l % 32, k = 8*(l/32) + j      B[k][n]: k = 8*(l/32) + j, n = l % 32
//   D[m][n] (16 fp32): n = l % 32, m = 8*(i/4) + 4*(l/32) + i%4, i = 0..15
// Both orientations are D = H * B, so a 32-value group is column n of D and
// lies in lanes n and n + 32 (16 values each):
//   row-wise:    B[k][n] = X[row n][col k]      column-wise: B[k][n] = X[row k][col n]
// Lanes l < 32 ("A") hold group elements {0-3, 8-11, 16-19, 24-27}, lanes
// l >= 32 ("B") {4-7, 12-15, 20-23, 28-31}; one lane swap
// (v_permlane32_swap) shares the group maximum and regroups the codes so
// that lane A holds bytes 0-7 and lane B bytes 8-15 of the group's 16 code
// bytes.  Tiles go to workgroups in XCD-aware order (16x16-tile super-tiles
// per XCD, grid a multiple of 8), so partial segments meet in one L2.
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr bool kHaveMx = true;
#ifndef FP4Q_MX_WG_PER_CU
#define FP4Q_MX_WG_PER_CU 1
#endif
#ifndef FP4Q_MX_WAVES
#define FP4Q_MX_WAVES 16
#endif
constexpr int kMxWaves = FP4Q_MX_WAVES;          // 8 or 16 waves per workgroup
constexpr int kMxThreads = 64 * kMxWaves;
constexpr int kMxBlocksPerWave = 16 / kMxWaves;  // 32x32 blocks per wave and orientation
constexpr int kMxPieces = 2048 / kMxThreads;     // 16-byte input pieces per thread and tile
constexpr int kMxTile = 128;                     // tile rows and columns
constexpr int kMxRegion = 256;                   // a workgroup's region: 2x2 tiles
constexpr int kMxPitch = kMxTile + 8;            // bf16 per LDS row of the input tile
constexpr int kMxCodePitch = 144;                // bytes per LDS row of a code stage (128 + pad)
constexpr int kMxSuper = 8;                      // 8x8 regions per XCD super-tile
constexpr int kMxWgPerCu = FP4Q_MX_WG_PER_CU;    // persistent workgroups per CU (LDS: 110 KiB each)

// fp32 nearest to 1/sqrt(32) (bit pattern 0x3E3504F3): orthonormal H32.
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// H[l % 32][16 h + 8 (l/32) + j] as bf16 +-1 (entries (-1)^popcount(m & k)).
__device__ __forceinline__ bf16x8_t had32_operand(int lane, int h) {
  uint32_t w[4];
#pragma unroll
  for (int p = 0; p < 4; p++) {
    uint32_t v = 0;
#pragma unroll
    for (int q = 0; q < 2; q++) {
      const int k = 16 * h + 8 * (lane >> 5) + 2 * p + q, m = lane & 31;
      v |= (uint32_t)((__builtin_popcount(m & k) & 1) ? 0xBF80u : 0x3F80u) << (16 * q);
    }
    w[p] = v;
  }
  return __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
}

// v_permlane32_swap(X, Y) leaves X' = (X[0..31], Y[0..31]) and
// Y' = (X[32..63], Y[32..63]) across the two half-waves: with X = Y = v,
// every lane then holds its own value and its partner's (lane l ^ 32).

// Quantize one 32-value group held as 16 + 16 values by a lane pair (this
// lane's y[i] is group element 8*(i/4) + 4*(lane/32) + i%4): exponent
// e = floor(log2 amax) - 2 (UE8M0 code e + 127, 0 for zero or subnormal
// maxima), then nearest-even E2M1 of y / 2^e by the hardware conversion with
// the power-of-two scale in its exponent operand.  Returns the 8 code bytes
// this lane stores (lo, hi) and the scale code.
__device__ __forceinline__ void mx_quant_pair(const float* y, uint32_t& lo, uint32_t& hi,
                                              uint32_t& code) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 16; i++) am = fmaxf(am, fabsf(y[i]));
  const auto m2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(am), __float_as_uint(am),
                                                   false, false);
  am = fmaxf(__uint_as_float(m2[0]), __uint_as_float(m2[1]));   // own and partner maximum
  const int ef = (int)(__float_as_uint(am) >> 23);              // biased exponent of amax
  code = (uint32_t)(ef > 2 ? ef - 2 : 0);
  // 2^e with exponent field = code; the conversion reads a zero field as
  // 2^-127 (checked on the device over every |y| < 2^-121), so tiny groups
  // need no special case
  const float scale = __uint_as_float(code << 23);
  uint32_t d01 = __builtin_nondeterministic_value(0u), d23 = __builtin_nondeterministic_value(0u);
  d01 = cvt_fp4x2<0>(d01, y[0], y[1], scale);     // elements 8q + 4 (l/32) + 0..3, q = 0
  d01 = cvt_fp4x2<1>(d01, y[2], y[3], scale);
  d01 = cvt_fp4x2<2>(d01, y[4], y[5], scale);     // q = 1
  d01 = cvt_fp4x2<3>(d01, y[6], y[7], scale);
  d23 = cvt_fp4x2<0>(d23, y[8], y[9], scale);     // q = 2
  d23 = cvt_fp4x2<1>(d23, y[10], y[11], scale);
  d23 = cvt_fp4x2<2>(d23, y[12], y[13], scale);   // q = 3
  d23 = cvt_fp4x2<3>(d23, y[14], y[15], scale);
  // code word q = A.half_q | B.half_q << 16; lane A stores words 0, 1 and
  // lane B words 2, 3.  One swap of (d01, d23) hands lane A (d01_A, d01_B)
  // and lane B (d23_A, d23_B): the A and B halves of the words it stores.
  const auto r = __builtin_amdgcn_permlane32_swap(d01, d23, false, false);
  const uint32_t a = r[0], b = r[1];
  lo = (a & 0xFFFFu) | (b << 16);
  hi = (a >> 16) | (b & 0xFFFF0000u);
}

template <bool HAD, bool ROW, bool COL>
__global__ __launch_bounds__(kMxThreads) void mxfp4_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ codes_r,
    uint8_t* __restrict__ scales_r, uint8_t* __restrict__ codes_c,
    uint8_t* __restrict__ scales_c) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kMxTile * kMxPitch];
  __shared__ __attribute__((aligned(16))) uint8_t rcode[ROW ? kMxRegion * kMxCodePitch : 16];
  __shared__ __attribute__((aligned(16))) uint8_t ccode[COL ? kMxRegion * kMxCodePitch : 16];
  __shared__ __attribute__((aligned(8))) uint8_t rscale[ROW ? kMxRegion * 8 : 8];
  __shared__ __attribute__((aligned(8))) uint8_t cscale[COL ? kMxRegion * 8 : 8];
  const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
  const int n = lane & 31, half = lane >> 5;
  const bool is_a = half == 0;
  const uint32_t RY = (uint32_t)((rows + kMxRegion - 1) / kMxRegion);
  const uint32_t RX = (uint32_t)((cols + kMxRegion - 1) / kMxRegion);
  const uint32_t nslots = (uint32_t)xcd_grid(RY, RX, kMxSuper, kMxSuper);
  const uint32_t G = gridDim.x;
  bf16x8_t h0 = {}, h1 = {};
  if constexpr (HAD) {
    h0 = had32_operand(lane, 0);
    h1 = had32_operand(lane, 1);
  }

  // Work unit j of this workgroup: quadrant j % 4 of region slot
  // blockIdx.x + (j / 4) G.  Quadrant q covers rows 128 (q / 2) and
  // columns 128 (q % 2) of the region.
  struct Unit {
    int64_t R0, C0;      // tile origin (rows, columns); R0 < 0: no tile
    int64_t RR0, CC0;    // region origin
    int q;
  };
  auto unit = [&](uint32_t j) {
    Unit u;
    TileOrder to;
    const uint32_t slot = blockIdx.x + (j >> 2) * G;
    u.q = (int)(j & 3);
    const bool valid = slot < nslots && xcd_tile<kMxSuper, kMxSuper>(slot, RY, RX, to);
    u.RR0 = valid ? to.ty * kMxRegion : -1;
    u.CC0 = valid ? to.tx * kMxRegion : -1;
    u.R0 = u.RR0 + kMxTile * (u.q >> 1);
    u.C0 = u.CC0 + kMxTile * (u.q & 1);
    if (!valid || u.R0 >= rows || u.C0 >= cols) u.R0 = -1;
    return u;
  };

  // Piece p = t + kMxThreads P of a tile: row p / 16 = t / 16 + (kMxThreads
  // / 16) P, columns 8 (t % 16) .. +7.  Pieces outside the tensor read x[0..7] instead
  // (cols % 8 == 0 keeps a piece inside its row); their values are never
  // stored.  Non-temporal: the input is read once, so it should not
  // displace the output lines.
  const int lr = t >> 4, lc = 8 * (t & 15);
  const int64_t ld_off = (int64_t)lr * cols + lc;
  auto load = [&](const Unit& u, Tile4& v) {
    const bool valid = u.R0 >= 0;
    const uint16_t* base = x + (valid ? u.R0 * cols + u.C0 : 0) + ld_off;
    // rows / columns left from the tile origin, capped to 32 bits (uniform)
    const int rem_r = valid ? (int)(rows - u.R0 < kMxTile ? rows - u.R0 : kMxTile) : 0;
    const int rem_c = valid ? (int)(cols - u.C0 < kMxTile ? cols - u.C0 : kMxTile) : 0;
    const bool col_ok = lc < rem_c;
    static_for<kMxPieces>([&](auto pc) {
      constexpr int P = decltype(pc)::value;
      constexpr int dr = kMxThreads / 16 * P;
      const bool ok = col_ok && lr + dr < rem_r;
      v.template at<P>() =
          __builtin_nontemporal_load((const u32x4_t*)(ok ? base + (int64_t)dr * cols : x));
    });
  };

  // The 16 values this lane holds of group (block row br, block col bc) of
  // the tile, in the D layout above: rotated when HAD, else read directly.
  auto row_group = [&](int br, int bc, float* y) {     // row 32 br + n, columns 32 bc + ...
    const uint16_t* base = tile + (32 * br + n) * kMxPitch + 32 * bc;
    if constexpr (HAD) {
      const u32x4_t b0 = *(const u32x4_t*)(base + 8 * half);
      const u32x4_t b1 = *(const u32x4_t*)(base + 16 + 8 * half);
      f32x16_t acc = {};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h0, __builtin_bit_cast(bf16x8_t, b0), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(h1, __builtin_bit_cast(bf16x8_t, b1), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; i++) y[i] = acc[i] * kInvSqrt32;
    } else {
#pragma unroll
      for (int q = 0; q < 4; q++) {
        const u32x2_t w = *(const u32x2_t*)(base + 8 * q + 4 * half);
        y[4 * q + 0] = bf16_lo(w.x);
        y[4 * q + 1] = bf16_hi(w.x);
        y[4 * q + 2] = bf16_lo(w.y);
        y[4 * q + 3] = bf16_hi(w.y);
      }
    }
  };
  auto col_group = [&](int br, int bc, float* y) {     // column 32 bc + n, rows 32 br + ...
    const uint16_t* base = tile + 32 * br * kMxPitch + 32 * bc + n;
    if constexpr (HAD) {
      uint32_t w[8];
#pragma unroll
      for (int p = 0; p < 8; p++) {          // B[k][n], k = 16 (p/4) + 8 half + 2 (p%4) + {0, 1}
        const uint16_t* s = base + (16 * (p >> 2) + 8 * half + 2 * (p & 3)) * kMxPitch;
        w[p] = (uint32_t)s[0] | ((uint32_t)s[kMxPitch] << 16);
      }
      f32x16_t acc = {};
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          h0, __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3])), acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
          h1, __builtin_bit_cast(bf16x8_t, make_uint4(w[4], w[5], w[6], w[7])), acc, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 16; i++) y[i] = acc[i] * kInvSqrt32;
    } else {
#pragma unroll
      for (int i = 0; i < 16; i++)
        y[i] = __uint_as_float(
            (uint32_t)base[(8 * (i >> 2) + 4 * half + (i & 3)) * kMxPitch] << 16);
    }
  };

  // store offsets within a region (per-thread constants): 16-byte code
  // segment g = t % 8 of region row (column) t / 8 (+ kMxThreads / 8 per
  // round), and scale byte t % 8 of the same row (column)
  const int e0 = t >> 3, g = t & 7;
  const int64_t sr_off = (int64_t)e0 * (cols / 2) + 16 * g, ss_off = (int64_t)e0 * (cols / 32) + g;
  const int64_t sc_off = (int64_t)e0 * (rows / 2) + 16 * g, scs_off = (int64_t)e0 * (rows / 32) + g;

  // Tile work: quantize into the region's LDS stage; after the fourth
  // quadrant, write the region's outputs.  `u.R0 < 0` is uniform.
  auto process = [&](Tile4& cur, const Unit& u) {
    if (u.R0 >= 0) {
      static_for<kMxPieces>([&](auto pc) {
        constexpr int P = decltype(pc)::value;
        const int p = t + kMxThreads * P;
        *(u32x4_t*)(tile + (p >> 4) * kMxPitch + 8 * (p & 15)) = cur.template at<P>();
      });
      __syncthreads();
      // wave w: row-wise blocks (bw, bs + s), column-wise blocks (bs + s, bw)
      // with bw = w / (4 / B), bs = B (w % (4 / B)), B = kMxBlocksPerWave
      constexpr int kPerRow = 4 / kMxBlocksPerWave;
      const int bw = wave / kPerRow, bs = kMxBlocksPerWave * (wave % kPerRow);
      const int qy = u.q >> 1, qx = u.q & 1;
      if constexpr (ROW) {
#pragma unroll
        for (int s = 0; s < kMxBlocksPerWave; s++) {
          float y[16];
          row_group(bw, bs + s, y);
          uint32_t lo, hi, code;
          mx_quant_pair(y, lo, hi, code);
          const int r = kMxTile * qy + 32 * bw + n;          // region row
          *(u32x2_t*)(rcode + r * kMxCodePitch + 64 * qx + 16 * (bs + s) + 8 * half) =
              u32x2_t{lo, hi};
          if (is_a) rscale[8 * r + 4 * qx + bs + s] = (uint8_t)code;
        }
      }
      if constexpr (COL) {
#pragma unroll
        for (int s = 0; s < kMxBlocksPerWave; s++) {
          float y[16];
          col_group(bs + s, bw, y);
          uint32_t lo, hi, code;
          mx_quant_pair(y, lo, hi, code);
          const int c = kMxTile * qx + 32 * bw + n;          // region column
          *(u32x2_t*)(ccode + c * kMxCodePitch + 64 * qy + 16 * (bs + s) + 8 * half) =
              u32x2_t{lo, hi};
          if (is_a) cscale[8 * c + 4 * qy + bs + s] = (uint8_t)code;
        }
      }
      __syncthreads();   // the next quadrant overwrites the tile
    }
    if (u.q != 3 || u.RR0 < 0) return;
    // region stores: every row (column) of the region leaves as one 128-byte
    // code line and 8 scale bytes; outside the tensor nothing is stored
    // (cols % 32 == 0 for row-wise and rows % 32 == 0 for column-wise output)
    const int rem_r = (int)(rows - u.RR0 < kMxRegion ? rows - u.RR0 : kMxRegion);
    const int rem_c = (int)(cols - u.CC0 < kMxRegion ? cols - u.CC0 : kMxRegion);
    constexpr int kStep = kMxThreads / 8;                    // region rows per round
#pragma unroll
    for (int i = 0; i < kMxRegion / kStep; i++) {
      const int e = e0 + kStep * i;
      if constexpr (ROW) {
        if (e < rem_r && 32 * g < rem_c) {
          *(u32x4_t*)(codes_r + (u.RR0 + kStep * i) * (cols / 2) + u.CC0 / 2 + sr_off) =
              *(const u32x4_t*)(rcode + e * kMxCodePitch + 16 * g);
          scales_r[(u.RR0 + kStep * i) * (cols / 32) + u.CC0 / 32 + ss_off] = rscale[8 * e + g];
        }
      }
      if constexpr (COL) {
        if (e < rem_c && 32 * g < rem_r) {
          *(u32x4_t*)(codes_c + (u.CC0 + kStep * i) * (rows / 2) + u.RR0 / 2 + sc_off) =
              *(const u32x4_t*)(ccode + e * kMxCodePitch + 16 * g);
          scales_c[(u.CC0 + kStep * i) * (rows / 32) + u.RR0 / 32 + scs_off] = cscale[8 * e + g];
        }
      }
    }
  };

  // Four register sets in turn, each tile's loads issued three tiles ahead
  // (no copy between the sets, so the wait for a tile's loads never
  // includes later loads or the region's stores; two sets, one tile ahead:
  // 3 % slower, six sets: no better).
  Tile4 t0, t1, t2, t3;
  Unit u0 = unit(0), u1 = unit(1), u2 = unit(2), u3;
  load(u0, t0);
  load(u1, t1);
  load(u2, t2);
  for (uint32_t j = 0;; j += 4) {
    if (blockIdx.x + (j >> 2) * G >= nslots) break;
    u3 = unit(j + 3);
    load(u3, t3);
    process(t0, u0);
    if (blockIdx.x + ((j + 1) >> 2) * G >= nslots) break;
    u0 = unit(j + 4);
    load(u0, t0);
    process(t1, u1);
    if (blockIdx.x + ((j + 2) >> 2) * G >= nslots) break;
    u1 = unit(j + 5);
    load(u1, t1);
    process(t2, u2);
    if (blockIdx.x + ((j + 3) >> 2) * G >= nslots) break;
    u2 = unit(j + 6);
    load(u2, t2);
    process(t3, u3);
  }
}

inline hipError_t launch_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, bool had,
                         uint8_t* codes_r, uint8_t* scales_r, uint8_t* codes_c,
                         uint8_t* scales_c, hipStream_t st, int num_cus) {
  const int64_t nslots = xcd_grid((rows + kMxRegion - 1) / kMxRegion,
                                  (cols + kMxRegion - 1) / kMxRegion, kMxSuper, kMxSuper);
  // persistent: a multiple of 8 workgroups (XCD count)
  int64_t grid = (int64_t)num_cus * kMxWgPerCu;
  if (grid > nslots) grid = nslots;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  const bool rw = codes_r != nullptr, cw = codes_c != nullptr;
#define FP4Q_MX(H, R, C)                                                                  \
  launch(mxfp4_kernel<H, R, C>, (unsigned)grid, kMxThreads, st, x, rows, cols, codes_r, \
         scales_r, codes_c, scales_c)
  if (had) {
    if (rw && cw) return FP4Q_MX(true, true, true);
    if (rw) return FP4Q_MX(true, true, false);
    return FP4Q_MX(true, false, true);
  }
  if (rw && cw) return FP4Q_MX(false, true, true);
  if (rw) return FP4Q_MX(false, true, false);
  return FP4Q_MX(false, false, true);
#undef FP4Q_MX
}

}  // namespace fp4q
