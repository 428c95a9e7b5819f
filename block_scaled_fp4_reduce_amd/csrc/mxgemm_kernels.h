// mxgemm_kernels.h -- the consumer of the quantized tensors: C = A B for
// MXFP4 operands on gfx950's block-scaled FP4 matrix cores.
//
// The NVIDIA NVFP4 article (sec. 1 and 5) describes MXFP4 -- E2M1 values
// with one power-of-two (UE8M0) scale per 32 -- as a format the hardware
// multiplies directly; the AMD MI355X MXFP4 article (sec. 2) trains with
// both operands in it.  A is [M][K] in the row-wise layout of the MXFP4
// quantizer, B is given as B^T [N][K] (its column-wise output), so both
// feed the instruction without repacking.
//
// v_mfma_scale_f32_32x32x64_f8f6f4 with FP4 operands (checked on the GPU):
// lane l serves row (A) or column (B) l % 32 and the K half l / 32; its four
// dwords are 32 consecutive codes of that row (even element in the low
// nibble) and its scale register the UE8M0 byte of those 32 values.  The
// 16 accumulators of lane l are D[8 (i / 4) + 4 (l / 32) + i % 4][l % 32].
//
// Workgroup: 512 threads, a 256 x 256 tile of C, each wave 128 x 64 (4 x 2
// instructions per 64 values of K, six 16-byte operand reads for eight
// instructions); K in steps of 128 values, staged in LDS (double buffered,
// rows padded to 80 bytes so the 16-byte operand reads of 8 or 16
// consecutive rows hit distinct banks), global loads issued two steps
// ahead (two register staging sets).  Tiles go out in XCD
// super-tile order (4 x 8 tiles per XCD per round), so the workgroups that
// share A and B K-slabs run on one L2 at the same time.  Rows past M or N
// read as zeros through the buffer-resource bounds; stores past them are
// dropped.
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr int kGemmThreads = 512;                  // 8 waves: 2 (M) x 4 (N)
constexpr int kGemmBM = 256, kGemmBN = 256;        // C tile per workgroup
constexpr int kGemmMI = 4, kGemmNJ = 2;            // 32 x 32 blocks per wave (128 x 64)
constexpr int kGemmBK = 128;                       // K values per step
constexpr int kGemmRowBytes = kGemmBK / 2;         // 64 code bytes per row per step
constexpr int kGemmPitch = kGemmRowBytes + 16;     // LDS row pitch (bytes)
constexpr int kGemmSuperY = 4, kGemmSuperX = 8;    // tiles per XCD super-tile

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One K step of both operands, in registers between its global load and its
// LDS store: two 16-byte pieces of each 16 KB tile per thread, and one scale
// dword (four K blocks of one row): A's for threads below 256, B's above.
struct GemmStage {
  u32x4_t a0, a1, b0, b1;
  uint32_t s;
};

__device__ __forceinline__ void gemm_load(GemmStage& g, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsa,
                                          __amdgpu_buffer_rsrc_t rsb, int64_t K, int ks) {
  const int t = threadIdx.x;
  const int kb = ks * kGemmRowBytes;               // byte offset of the step in a code row
  // piece q = t + 512 i: row q / 4, 16-byte column q % 4
  const int r0 = t >> 2, r1 = (t + kGemmThreads) >> 2, c = 16 * (t & 3);
  const int rowb = (int)(K / 2);
  g.a0 = __builtin_bit_cast(u32x4_t, buffer_load16(ra, r0 * rowb + kb + c));
  g.a1 = __builtin_bit_cast(u32x4_t, buffer_load16(ra, r1 * rowb + kb + c));
  g.b0 = __builtin_bit_cast(u32x4_t, buffer_load16(rb, r0 * rowb + kb + c));
  g.b1 = __builtin_bit_cast(u32x4_t, buffer_load16(rb, r1 * rowb + kb + c));
  const int srow = (int)(K / 32), sb = ks * (kGemmBK / 32);
  // waves 0-3 load A's scales, waves 4-7 B's: the choice is uniform over a
  // wave, said so explicitly, so it is one load through a scalar-selected
  // resource (a per-lane choice of resource would become a loop over its
  // values and blur the compiler's count of loads in flight)
  const int half = __builtin_amdgcn_readfirstlane(t >> 8);
  const __amdgpu_buffer_rsrc_t rs = half ? rsb : rsa;
  g.s = __builtin_amdgcn_raw_buffer_load_b32(rs, (t - 256 * half) * srow + sb, 0, 0);
}

__device__ __forceinline__ void gemm_store(const GemmStage& g, uint8_t* la, uint8_t* lb,
                                           uint32_t* lsa, uint32_t* lsb) {
  const int t = threadIdx.x;
  const int r0 = t >> 2, r1 = (t + kGemmThreads) >> 2, c = 16 * (t & 3);
  *(u32x4_t*)(la + r0 * kGemmPitch + c) = g.a0;
  *(u32x4_t*)(la + r1 * kGemmPitch + c) = g.a1;
  *(u32x4_t*)(lb + r0 * kGemmPitch + c) = g.b0;
  *(u32x4_t*)(lb + r1 * kGemmPitch + c) = g.b1;
  if (t < 256) lsa[t] = g.s;
  else lsb[t - 256] = g.s;
}

__global__ __launch_bounds__(kGemmThreads) void mxfp4_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ bt_codes, const uint8_t* __restrict__ bt_scales, int64_t M,
    int64_t N, int64_t K, float* __restrict__ c_out, uint32_t tiles_m, uint32_t tiles_n) {
  __shared__ __attribute__((aligned(16))) uint8_t lA[2][kGemmBM * kGemmPitch];
  __shared__ __attribute__((aligned(16))) uint8_t lB[2][kGemmBN * kGemmPitch];
  __shared__ uint32_t lsA[2][kGemmBM], lsB[2][kGemmBN];

  TileOrder to;
  if (!xcd_tile<kGemmSuperY, kGemmSuperX>(blockIdx.x, tiles_m, tiles_n, to)) return;  // uniform
  const int64_t m0 = to.ty * kGemmBM, n0 = to.tx * kGemmBN;
  const int64_t mrows = M - m0 < kGemmBM ? M - m0 : kGemmBM;
  const int64_t nrows = N - n0 < kGemmBN ? N - n0 : kGemmBN;
  // resources over this tile's rows of each operand (rows past M / N read 0)
  const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a_codes + m0 * (K / 2)), 0, (int)(mrows * (K / 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(bt_codes + n0 * (K / 2)), 0, (int)(nrows * (K / 2)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(a_scales + m0 * (K / 32)), 0, (int)(mrows * (K / 32)), 0x00020000);
  const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(bt_scales + n0 * (K / 32)), 0, (int)(nrows * (K / 32)), 0x00020000);

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int r = lane & 31, g = lane >> 5;
  f32x16_t acc[kGemmMI][kGemmNJ];
#pragma unroll
  for (int i = 0; i < kGemmMI; i++)
#pragma unroll
    for (int j = 0; j < kGemmNJ; j++) acc[i][j] = f32x16_t{};

  const int nk = (int)(K / kGemmBK);
  // Two register staging sets: step j's global loads are issued two steps
  // ahead (during step j - 2) and stored to LDS at the end of step j - 1,
  // so they have two steps of matrix work to arrive.  The loop is unrolled
  // by two so that each set is named at compile time (a runtime index
  // would put the sets in scratch memory).
  // Loads for steps past the end are issued too (unconditional loads keep
  // the compiler's count of loads in flight exact, so each wait is for the
  // right step): buffer loads are bounds-checked against the operand rows,
  // and those registers are never stored to LDS.
  GemmStage st0, st1;
  gemm_load(st0, ra, rb, rsa, rsb, K, 0);
  gemm_load(st1, ra, rb, rsa, rsb, K, 1);
  gemm_store(st0, lA[0], lB[0], lsA[0], lsB[0]);
  __syncthreads();
  // one K step: prefetch step ks + 2 into `mine` (free: its data went to LDS
  // last step), multiply from LDS buffer `b`, store step ks + 1 (in
  // `other`) to the other buffer
  auto step = [&](int ks, GemmStage& mine, GemmStage& other, int b) {
    gemm_load(mine, ra, rb, rsa, rsb, K, ks + 2);
#pragma unroll
    for (int s = 0; s < 2; s++) {                 // two 64-value halves of the step
      i32x8_t av[kGemmMI], bv[kGemmNJ];
      int sa[kGemmMI], sb[kGemmNJ];
#pragma unroll
      for (int i = 0; i < kGemmMI; i++) {
        const int row = 128 * wm + 32 * i + r;
        const u32x4_t v = *(const u32x4_t*)(lA[b] + row * kGemmPitch + 32 * s + 16 * g);
        av[i] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sa[i] = (int)((lsA[b][row] >> (8 * (2 * s + g))) & 0xFFu);
      }
#pragma unroll
      for (int j = 0; j < kGemmNJ; j++) {
        const int row = 64 * wn + 32 * j + r;
        const u32x4_t v = *(const u32x4_t*)(lB[b] + row * kGemmPitch + 32 * s + 16 * g);
        bv[j] = i32x8_t{(int)v.x, (int)v.y, (int)v.z, (int)v.w, 0, 0, 0, 0};
        sb[j] = (int)((lsB[b][row] >> (8 * (2 * s + g))) & 0xFFu);
      }
#pragma unroll
      for (int i = 0; i < kGemmMI; i++)
#pragma unroll
        for (int j = 0; j < kGemmNJ; j++)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              av[i], bv[j], acc[i][j], 4, 4, 0, sa[i], 0, sb[j]);
    }
    if (ks + 1 < nk) gemm_store(other, lA[b ^ 1], lB[b ^ 1], lsA[b ^ 1], lsB[b ^ 1]);
    __syncthreads();
  };
  for (int ks = 0; ks < nk; ks += 2) {
    step(ks, st0, st1, 0);
    if (ks + 1 < nk) step(ks + 1, st1, st0, 1);
  }

  // C tile: lane holds D[8 (v / 4) + 4 g + v % 4][r] of each 32 x 32 block
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
      c_out + m0 * N, 0, (int)(mrows * N * 4), 0x00020000);
#pragma unroll
  for (int j = 0; j < kGemmNJ; j++) {
    const int64_t col = 64 * wn + 32 * j + r;
    if (col < nrows) {
#pragma unroll
      for (int i = 0; i < kGemmMI; i++)
#pragma unroll
        for (int v = 0; v < 16; v++) {
          const int64_t row = 128 * wm + 32 * i + 8 * (v / 4) + 4 * g + (v % 4);
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][v]), rc,
                                                (int)((row * N + n0 + col) * 4), 0, 0);
        }
    }
  }
}

// C = 0 for an empty sum (K = 0): a plain fill, not a memset, so the call
// can be captured in a HIP graph.
__global__ __launch_bounds__(256) void fill_zero_kernel(float* __restrict__ c, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    c[i] = 0.0f;
}

}  // namespace fp4q
