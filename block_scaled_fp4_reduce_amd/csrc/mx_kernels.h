// mx_kernels.h -- MXFP4 quantization with an optional 32-point Hadamard,
// row-wise and column-wise outputs from one read of the input.
//
// Method: NVIDIA NVFP4 article sec. 1 and sec. 5 (MXFP4: 32 values share a
// power-of-two UE8M0 scale); AMD MI355X MXFP4 pretraining article sec. 2
// (a fixed, deterministic Hadamard rotation before quantizing, for both
// operands of the weight-gradient product, hence both orientations).
//
// Mapping onto the chip: a workgroup of 4*kMxRows threads owns one
// kMxRows x 128 tile at a time.  Each thread loads one 32-value row group
// (four 16-byte loads), quantizes it row-wise straight from registers, and
// stores it to LDS; after one barrier each thread reads one 32-value column
// group back from LDS (a wave reads 64 adjacent columns of one row per
// instruction: 128 contiguous bytes, no bank conflicts) and quantizes it
// column-wise.  Row pitch in LDS is padded by 16 bytes so the row-group
// stores do not collide on banks.  Workgroups are persistent and load the
// next tile while computing the current one.  Tiles are handed out in
// XCD-aware order (16x16-tile super-tiles per XCD; the grid is a multiple
// of 8 so a workgroup's tiles stay on its XCD), so the scale bytes that
// neighbouring tiles write into one 64-byte segment all land in the same L2
// before the line goes to memory.
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr bool kHaveMx = true;
#ifndef FP4Q_MX_ROWS
#define FP4Q_MX_ROWS 128
#endif
constexpr int kMxTile = 128;                     // tile columns
constexpr int kMxRows = FP4Q_MX_ROWS;            // tile rows (64 or 128)
constexpr int kMxThreads = kMxRows * 4;          // one row group and one column group per thread
constexpr int kMxPitch = kMxTile + 8;            // bf16 per LDS row (16-byte pad)
#ifndef FP4Q_MX_WG_PER_CU
#define FP4Q_MX_WG_PER_CU 2
#endif
constexpr int kMxWgPerCu = FP4Q_MX_WG_PER_CU;    // persistent workgroups per CU

// fp32 nearest to 1/sqrt(32) (bit pattern 0x3E3504F3): orthonormal H32.
constexpr float kInvSqrt32 = 0x1.6a09e6p-3f;

// Quantize 32 values (already rotated if asked) to MXFP4: UE8M0 code of
// floor(log2 amax) - 2 (0 for zero or subnormal maxima), then nearest-even
// E2M1 of y / 2^e, done by the hardware conversion with the power-of-two
// scale in its exponent operand.  Returns the scale code; codes in w[0..3].
__device__ __forceinline__ uint32_t mx_quant32(float* y, uint32_t* w) {
  float amax = 0.0f;
#pragma unroll
  for (int k = 0; k < 32; k++) amax = fmaxf(amax, fabsf(y[k]));
  const int ef = (int)(__float_as_uint(amax) >> 23);           // biased exponent of amax
  const uint32_t code = (uint32_t)(ef > 2 ? ef - 2 : 0);        // e + 127, e >= -127
  float scale = __uint_as_float(code << 23);                    // 2^e (exponent field = code)
  if (code == 0) {
    // e = -127: scale the (tiny) values by 2^127 exactly first and convert
    // with unit scale, so the conversion never sees a zero exponent field
#pragma unroll
    for (int k = 0; k < 32; k++) y[k] = y[k] * 0x1p127f;
    scale = 1.0f;
  }
#pragma unroll
  for (int d = 0; d < 4; d++) {
    uint32_t v = 0;
    v = cvt_fp4x2<0>(v, y[8 * d + 0], y[8 * d + 1], scale);
    v = cvt_fp4x2<1>(v, y[8 * d + 2], y[8 * d + 3], scale);
    v = cvt_fp4x2<2>(v, y[8 * d + 4], y[8 * d + 5], scale);
    v = cvt_fp4x2<3>(v, y[8 * d + 6], y[8 * d + 7], scale);
    w[d] = v;
  }
  return code;
}

template <bool HAD>
__device__ __forceinline__ void mx_rotate(float* y) {
  if constexpr (HAD) {
    fwht<32>(y);
#pragma unroll
    for (int k = 0; k < 32; k++) y[k] = y[k] * kInvSqrt32;
  }
}

constexpr int kMxSuper = 16;

struct Group32 {   // one thread's 32 bf16 values of a tile row (four 16-byte pieces)
  uint4 a, b, c, d;
};   // 16x16 tiles (2048x2048 values) per XCD super-tile

template <bool HAD, bool ROW, bool COL>
__global__ __launch_bounds__(kMxThreads) void mxfp4_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ codes_r,
    uint8_t* __restrict__ scales_r, uint8_t* __restrict__ codes_c,
    uint8_t* __restrict__ scales_c) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kMxRows * kMxPitch];
  const int t = threadIdx.x;
  const int r = t >> 2, g = t & 3;                 // row group of this thread
  const uint32_t TY = (uint32_t)((rows + kMxRows - 1) / kMxRows);
  const uint32_t TX = (uint32_t)((cols + kMxTile - 1) / kMxTile);
  constexpr int SY = kMxSuper * (kMxTile / kMxRows), SX = kMxSuper;
  const uint32_t nslots = (uint32_t)xcd_grid(TY, TX, SY, SX);

  // Decode `slot` and load this thread's row group of its tile.  Every load
  // is issued (addresses clamped into the tensor) so the compiler can keep
  // the next tile's loads in flight; values loaded for positions outside
  // the tensor are never stored (row groups need col < cols, column groups
  // row < rows, and cols % 8 == 0 keeps each 16-byte piece inside a row).
  auto load = [&](uint32_t slot, Group32& v, TileOrder& to) {
    const bool valid = slot < nslots && xcd_tile<SY, SX>(slot, TY, TX, to);
    if (!valid) to.ty = to.tx = -1;
    const int64_t row = valid ? to.ty * kMxRows + r : 0;
    const int64_t rr = row < rows ? row : rows - 1;
    const int64_t c0 = valid ? to.tx * kMxTile + 32 * g : 0;
    const uint16_t* src = x + rr * cols;
    auto piece = [&](int j) {
      const int64_t c = c0 + 8 * j < cols ? c0 + 8 * j : cols - 8;
      return *(const uint4*)(src + c);
    };
    v.a = piece(0);
    v.b = piece(1);
    v.c = piece(2);
    v.d = piece(3);
  };

  Group32 cur, nxt;
  TileOrder tcur, tnxt;
  uint32_t slot = blockIdx.x;
  load(slot, cur, tcur);
  while (slot < nslots) {
    const uint32_t next = slot + gridDim.x;    // grid is a multiple of 8: same XCD
    load(next, nxt, tnxt);                     // in flight while this tile is computed
    const TileOrder to = tcur;
    if (to.ty >= 0) {                          // uniform over the workgroup
      const int64_t R0 = to.ty * kMxRows, C0 = to.tx * kMxTile;
      const int64_t row = R0 + r, c0 = C0 + 32 * g;
      if constexpr (COL) {
        uint4* dst = (uint4*)(tile + r * kMxPitch + 32 * g);
        dst[0] = cur.a;
        dst[1] = cur.b;
        dst[2] = cur.c;
        dst[3] = cur.d;
      }
      if constexpr (ROW) {
        if (row < rows && c0 < cols) {         // cols % 32 == 0: the group is whole
          float y[32];
          unpack8(cur.a, y);
          unpack8(cur.b, y + 8);
          unpack8(cur.c, y + 16);
          unpack8(cur.d, y + 24);
          mx_rotate<HAD>(y);
          uint32_t w[4];
          const uint32_t code = mx_quant32(y, w);
          // lanes 4r..4r+3 store one row's 64 contiguous bytes in one instruction
          *(uint4*)(codes_r + row * (cols / 2) + c0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
          scales_r[row * (cols / 32) + c0 / 32] = (uint8_t)code;
        }
      }
      if constexpr (COL) {
        __syncthreads();
        // column groups: thread t takes tile column t%128, rows 32*(t/128) .. +31;
        // a column's pieces come from the kMxRows/32 groups of this workgroup
        const int c = t & (kMxTile - 1), gc = t >> 7;
        const int64_t col = C0 + c, r0 = R0 + 32 * gc;
        if (col < cols && r0 < rows) {         // rows % 32 == 0: the group is whole
          float y[32];
#pragma unroll
          for (int k = 0; k < 32; k++)
            y[k] = __uint_as_float((uint32_t)tile[(32 * gc + k) * kMxPitch + c] << 16);
          mx_rotate<HAD>(y);
          uint32_t w[4];
          const uint32_t code = mx_quant32(y, w);
          *(uint4*)(codes_c + col * (rows / 2) + r0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
          scales_c[col * (rows / 32) + r0 / 32] = (uint8_t)code;
        }
        __syncthreads();                       // LDS free for the next tile
      }
    }
    cur = nxt;
    tcur = tnxt;
    slot = next;
  }
}

inline void launch_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, bool had,
                         uint8_t* codes_r, uint8_t* scales_r, uint8_t* codes_c,
                         uint8_t* scales_c, hipStream_t st, int num_cus) {
  const int64_t nslots = xcd_grid((rows + kMxRows - 1) / kMxRows, (cols + kMxTile - 1) / kMxTile,
                                  kMxSuper * (kMxTile / kMxRows), kMxSuper);
  // persistent: a multiple of 8 workgroups (XCD count)
  int64_t grid = (int64_t)num_cus * kMxWgPerCu;
  if (grid > nslots) grid = nslots;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  const bool rw = codes_r != nullptr, cw = codes_c != nullptr;
#define FP4Q_MX(H, R, C)                                                                     \
  mxfp4_kernel<H, R, C><<<(unsigned)grid, kMxThreads, 0, st>>>(x, rows, cols, codes_r, scales_r, \
                                                                codes_c, scales_c)
  if (had) {
    if (rw && cw) FP4Q_MX(true, true, true);
    else if (rw) FP4Q_MX(true, true, false);
    else FP4Q_MX(true, false, true);
  } else {
    if (rw && cw) FP4Q_MX(false, true, true);
    else if (rw) FP4Q_MX(false, true, false);
    else FP4Q_MX(false, false, true);
  }
#undef FP4Q_MX
}

}  // namespace fp4q
