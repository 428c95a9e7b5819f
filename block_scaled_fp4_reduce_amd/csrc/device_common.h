// device_common.h -- gfx950 device helpers shared by the quantizer kernels.
//
// Number formats ("Four Over Six", sec. 1 and 2.1; NVIDIA NVFP4 article,
// sec. 1): FP4 E2M1 values +-{0,.5,1,1.5,2,3,4,6}; FP8 E4M3 block scales
// (bias 7, max 448); UE8M0 power-of-two scales for MXFP4.
#pragma once

#include <tuple>
#include <utility>

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

constexpr int kThreads = 256;             // 4 wave64s per workgroup

// Host: launch `kernel` on `st` and return that launch's own status
// (hipLaunchKernel's return value), so a failure left behind by an earlier,
// unrelated HIP call of the caller is neither reported nor consumed.
template <typename... P, typename... A>
inline hipError_t launch(void (*kernel)(P...), unsigned grid, unsigned block, hipStream_t st,
                         A... a) {
  static_assert(sizeof...(P) == sizeof...(A), "argument count");
  std::tuple<P...> args{static_cast<P>(a)...};
  return std::apply(
      [&](auto&... v) {
        void* argv[] = {(void*)&v...};
        return hipLaunchKernel((const void*)kernel, dim3(grid), dim3(block), argv, 0, st);
      },
      args);
}

typedef float float2_t __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------- bf16
// bf16 -> fp32 is exact: the bf16 bits are the upper half of the fp32 bits.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ void unpack8(const uint4& v, float* y) {
  y[0] = bf16_lo(v.x); y[1] = bf16_hi(v.x);
  y[2] = bf16_lo(v.y); y[3] = bf16_hi(v.y);
  y[4] = bf16_lo(v.z); y[5] = bf16_hi(v.z);
  y[6] = bf16_lo(v.w); y[7] = bf16_hi(v.w);
}

// ---------------------------------------------------------------- E4M3
// Nearest-even rounding of x >= 0 to E4M3, saturating at 448 (code 0x7E).
// Normal range: round the fp32 mantissa to 3 bits on the bit pattern and
// rebias the exponent from 127 to 7.  Below 2^-6 the step is 2^-9, so the
// code is x * 512 rounded to an integer.  Negative and NaN inputs give 0.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
  const uint32_t b = __float_as_uint(x);
  uint32_t normal = ((b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20) - (120u << 3);
  normal = normal < 0x7Eu ? normal : 0x7Eu;
  const float sub = fmaxf(__builtin_rintf(x * 512.0f), 0.0f);
  return x >= 0x1p-6f ? normal : (uint32_t)sub;
}

// E4M3 code (0..126) -> value; exact.
__device__ __forceinline__ float e4m3_value(uint32_t code) {
  const uint32_t e = code >> 3, m = code & 7u;
  return e ? __builtin_ldexpf((float)(8u + m), (int)e - 10) : __builtin_ldexpf((float)m, -9);
}

// ---------------------------------------------------------------- E2M1
// Hardware conversions of gfx950.  The scale operand carries an E8M0
// exponent in the fp32 exponent field: 1.0f means "no scaling", and
// __uint_as_float(code << 23) divides (encode) or multiplies (decode) by
// 2^(code - 127) exactly.  Rounding is nearest-even, saturating at 6.
template <int BYTE>
__device__ __forceinline__ uint32_t cvt_fp4x2(uint32_t old, float a, float b, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, scale, BYTE);
}

template <int BYTE>
__device__ __forceinline__ float2_t fp4x2_to_f32(uint32_t packed, float scale) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, scale, BYTE);
}

// ---------------------------------------------------------------- Philox4x32-10
// Salmon, Moraes, Dror, Shaw (SC'11).  Returns output word 0 only; the
// compiler drops the work the last rounds spend on the other words.
// a ^ b ^ k in one VALU instruction: gfx950's three-input bitwise op with
// truth table 0x96 (odd parity of the three bits).  Through the compiler
// builtin, not inline asm, so that no hazard padding follows it.
__device__ __forceinline__ uint32_t xor3_vvs(uint32_t a, uint32_t b, uint32_t k) {
  return __builtin_amdgcn_bitop3_b32(a, b, k, 0x96);
}

__device__ __forceinline__ uint32_t philox_w0(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                             uint32_t k0, uint32_t k1) {
  // the first round in plain C, so known-zero counter words fold away
  {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
    const uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
#pragma unroll
  for (int r = 1; r < 10; r++) {
    const uint64_t p0 = (uint64_t)0xD2511F53u * c0;
    const uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
    const uint32_t n0 = xor3_vvs((uint32_t)(p1 >> 32), c1, k0);
    const uint32_t n2 = xor3_vvs((uint32_t)(p0 >> 32), c3, k1);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return c0;
}

// ---------------------------------------------------------------- Hadamard
// Unnormalised Walsh-Hadamard butterfly (natural order): stage h pairs
// (j, j+h) for j with bit h clear into (sum, difference).  N = 16 or 32.
template <int N>
__device__ __forceinline__ void fwht(float* v) {
#pragma unroll
  for (int h = 1; h < N; h <<= 1) {
#pragma unroll
    for (int j = 0; j < N; j++) {
      if (j & h) continue;
      const float a = v[j], b = v[j + h];
      v[j] = a + b;
      v[j + h] = a - b;
    }
  }
}

// ---------------------------------------------------------------- compile-time loops
// f(integral_constant<int, 0>) ... f(integral_constant<int, N-1>): register
// arrays indexed inside stay in registers whatever the unroller decides.
template <typename F, int... K>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, K...>) {
  (f(std::integral_constant<int, K>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ---------------------------------------------------------------- register tiles
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));   // plain vectors: stay in VGPRs
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

struct Tile4 {      // one thread's (up to) four 16-byte pieces of a tile (separate
  u32x4_t v0, v1, v2, v3;   // members: never an indexed array)
  template <int P>
  __device__ __forceinline__ u32x4_t& at() {
    static_assert(P >= 0 && P < 4, "piece index");
    if constexpr (P == 0) return v0;
    else if constexpr (P == 1) return v1;
    else if constexpr (P == 2) return v2;
    else return v3;
  }
};

// ---------------------------------------------------------------- buffer access
// Buffer resource over [base, base + bytes): loads past the end read 0 and
// stores past the end are dropped, so tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, int64_t bytes) {
  const int n = bytes < 0 ? 0 : (bytes > 0x7FFFFFF0 ? 0x7FFFFFF0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void_t;   // LDS destination of direct loads
typedef int i32x2_t __attribute__((ext_vector_type(2)));

// Cache policy of quantizer output stores: non-temporal (streaming), for
// kernels whose waves write whole contiguous runs of codes and scales.  The
// outputs are written once and never read back by the kernel, so they should
// not displace input lines, and fewer dirty lines are left in L2 when the
// kernel ends.  Segments completed piecewise by several tiles (the 2D
// kernel's transposed codes, MX, requantization) keep ordinary stores:
// streaming partial lines there costs far more than it saves.
constexpr int kStoreNT = 2;

__device__ __forceinline__ uint4 buffer_load16(__amdgpu_buffer_rsrc_t r, int off) {
  const i32x4_t v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4((uint32_t)v.x, (uint32_t)v.y, (uint32_t)v.z, (uint32_t)v.w);
}

// ---------------------------------------------------------------- XCD-aware tile order
// MI355X has 8 XCDs with one L2 each, and consecutive workgroup ids go to
// consecutive XCDs.  Outputs whose 64-byte segments are completed by
// neighbouring tiles (scale bytes, transposed codes) must be finished inside
// one L2, or partial lines reach memory separately.  This maps workgroup ids
// onto a TY x TX tile grid so that each XCD walks whole SY x SX super-tiles,
// row-major inside each.  Returns false for ids with no tile (ragged edges).
#ifndef FP4Q_XCD_ORDER
#define FP4Q_XCD_ORDER 1
#endif
constexpr int kXcds = 8;

struct TileOrder {
  int64_t ty, tx;
};

// Tile counts stay below 2^31 (the host caps tensors at 2^40 elements and
// tiles hold at least 2^10), so the index arithmetic is 32-bit; SY and SX
// are compile-time powers of two.
template <int SY, int SX>
__device__ __forceinline__ bool xcd_tile(uint32_t b, uint32_t TY, uint32_t TX, TileOrder& t) {
  const uint32_t NSY = (TY + SY - 1) / SY, NSX = (TX + SX - 1) / SX, NS = NSY * NSX;
  if (!FP4Q_XCD_ORDER || NS < kXcds) {     // too few super-tiles: plain row-major order
    if (b >= TY * TX) return false;
    const uint32_t ty = b / TX;
    t.ty = ty;
    t.tx = b - ty * TX;
    return true;
  }
  constexpr uint32_t per = (uint32_t)SY * SX;
  const uint32_t xcd = b % kXcds, k = b / kXcds;
  const uint32_t s = (k / per) * kXcds + xcd, within = k % per;
  if (s >= NS) return false;
  const uint32_t sy = s / NSX, sx = s - sy * NSX;
  const uint32_t ty = sy * SY + within / SX, tx = sx * SX + within % SX;
  t.ty = ty;
  t.tx = tx;
  return ty < TY && tx < TX;
}

// Grid size for xcd_tile over a TY x TX tile grid.
__host__ __device__ inline int64_t xcd_grid(int64_t TY, int64_t TX, int SY, int SX) {
  const int64_t NSY = (TY + SY - 1) / SY, NSX = (TX + SX - 1) / SX, NS = NSY * NSX;
  if (!FP4Q_XCD_ORDER || NS < kXcds) return TY * TX;
  return ((NS + kXcds - 1) / kXcds) * kXcds * (int64_t)SY * SX;
}

// Cross-lane reads inside a 16-lane DPP row (no LDS round trip).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i within each 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15-i within each 16

// Max of a non-negative value over the 16 lanes of a DPP row, in every lane
// of the row (the xor-1, xor-2, half-mirror and mirror steps pair the lanes
// as a butterfly would).  Non-negative floats order like their bit
// patterns, so this is an integer max (one DPP max instruction per step).
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_row_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ float tile_max(float v) {
  uint32_t u = __float_as_uint(v);
  u = max(u, dpp_row_u<kDppXor1>(u));
  u = max(u, dpp_row_u<kDppXor2>(u));
  u = max(u, dpp_row_u<kDppHalfMirror>(u));
  return __uint_as_float(max(u, dpp_row_u<kDppMirror>(u)));
}

// Max of a non-negative value over the whole (fully active) wave, as a
// uniform value: DPP max inside each 16-lane row, then the four row results
// through readlane (for non-negative floats the bit patterns order as the
// values do).
__device__ __forceinline__ float wave_max_nonneg(float v) {
  const uint32_t t = __float_as_uint(tile_max(v));
  const uint32_t a = __builtin_amdgcn_readlane(t, 0), b = __builtin_amdgcn_readlane(t, 16);
  const uint32_t c = __builtin_amdgcn_readlane(t, 32), d = __builtin_amdgcn_readlane(t, 48);
  const uint32_t ab = a > b ? a : b, cd = c > d ? c : d;
  return __uint_as_float(ab > cd ? ab : cd);
}

// Order LDS traffic of one wave (its lanes exchange data through LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// ---------------------------------------------------------------- wave/workgroup max
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t m) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    const uint32_t o = (uint32_t)__shfl_xor((int)m, off, 64);
    m = m > o ? m : o;
  }
  return m;
}

// Max over a workgroup of NT threads; every thread gets the result.
template <int NT = kThreads>
__device__ __forceinline__ uint32_t block_max_u32(uint32_t m, uint32_t* red /* [NT/64] */) {
  m = wave_max_u32(m);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) red[wave] = m;
  __syncthreads();
  uint32_t r = red[0];
#pragma unroll
  for (int w = 1; w < NT / 64; w++) r = r > red[w] ? r : red[w];
  return r;
}

}  // namespace fp4q
