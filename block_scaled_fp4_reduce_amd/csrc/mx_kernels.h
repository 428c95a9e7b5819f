// mx_kernels.h -- MXFP4 quantization with an optional 32-point Hadamard,
// row-wise and column-wise outputs from one read of the input.
//
// Method: NVIDIA NVFP4 article sec. 1 and sec. 5 (MXFP4: 32 values share a
// power-of-two UE8M0 scale); AMD MI355X MXFP4 pretraining article sec. 2
// (a fixed, deterministic Hadamard rotation before quantizing, for both
// operands of the weight-gradient product, hence both orientations).
//
// Mapping onto the chip: a 512-thread workgroup owns a 128x128 tile.  Each
// thread loads one 32-value row group (four 16-byte loads), quantizes it
// row-wise straight from registers, and stores it to LDS; after one barrier
// each thread reads one 32-value column group back from LDS (a wave reads 64
// adjacent columns of one row per instruction: 128 contiguous bytes, no bank
// conflicts) and quantizes it column-wise.  Row pitch in LDS is padded by 16
// bytes so the row-group stores do not collide on banks.
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr bool kHaveMx = true;
constexpr int kMxThreads = 512;
constexpr int kMxTile = 128;
constexpr int kMxPitch = kMxTile + 8;    // bf16 per LDS row (16-byte pad)

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

template <bool HAD, bool ROW, bool COL>
__global__ __launch_bounds__(kMxThreads) void mxfp4_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, uint8_t* __restrict__ codes_r,
    uint8_t* __restrict__ scales_r, uint8_t* __restrict__ codes_c,
    uint8_t* __restrict__ scales_c) {
  __shared__ __attribute__((aligned(16))) uint16_t tile[kMxTile * kMxPitch];
  const int t = threadIdx.x;
  const int64_t tiles_x = (cols + kMxTile - 1) / kMxTile;
  const int64_t R0 = (blockIdx.x / tiles_x) * kMxTile;
  const int64_t C0 = (blockIdx.x % tiles_x) * kMxTile;

  // ---- row groups: thread t takes tile row t/4, columns 32*(t%4) .. +31
  {
    const int r = t >> 2, g = t & 3;
    const int64_t row = R0 + r, c0 = C0 + 32 * g;
    uint4 v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const bool ok = row < rows && c0 + 8 * j < cols;
      v[j] = ok ? *(const uint4*)(x + row * cols + c0 + 8 * j) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (COL) {
#pragma unroll
      for (int j = 0; j < 4; j++) *(uint4*)(tile + r * kMxPitch + 32 * g + 8 * j) = v[j];
    }
    if constexpr (ROW) {
      if (row < rows && c0 < cols) {           // cols % 32 == 0: the group is whole
        float y[32];
#pragma unroll
        for (int j = 0; j < 4; j++) unpack8(v[j], y + 8 * j);
        mx_rotate<HAD>(y);
        uint32_t w[4];
        const uint32_t code = mx_quant32(y, w);
        *(uint4*)(codes_r + row * (cols / 2) + c0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
        scales_r[row * (cols / 32) + c0 / 32] = (uint8_t)code;
      }
    }
  }
  if constexpr (COL) {
    __syncthreads();
    // ---- column groups: thread t takes tile column t%128, rows 32*(t/128) .. +31
    const int c = t & (kMxTile - 1), g = t >> 7;
    const int64_t col = C0 + c, r0 = R0 + 32 * g;
    if (col < cols && r0 < rows) {             // rows % 32 == 0: the group is whole
      float y[32];
#pragma unroll
      for (int k = 0; k < 32; k++)
        y[k] = __uint_as_float((uint32_t)tile[(32 * g + k) * kMxPitch + c] << 16);
      mx_rotate<HAD>(y);
      uint32_t w[4];
      const uint32_t code = mx_quant32(y, w);
      *(uint4*)(codes_c + col * (rows / 2) + r0 / 2) = make_uint4(w[0], w[1], w[2], w[3]);
      scales_c[col * (rows / 32) + r0 / 32] = (uint8_t)code;
    }
  }
}

inline void launch_mxfp4(const uint16_t* x, int64_t rows, int64_t cols, bool had,
                         uint8_t* codes_r, uint8_t* scales_r, uint8_t* codes_c,
                         uint8_t* scales_c, hipStream_t st) {
  const int64_t grid = ((rows + kMxTile - 1) / kMxTile) * ((cols + kMxTile - 1) / kMxTile);
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
