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
// Workgroup: 256 threads, a 256 x 256 tile of C, each of the 4 waves (one per
// SIMD) 128 x 128 (4 x 4 instructions per 64 values of K, eight 16-byte
// operand reads for sixteen instructions: with 8 waves of 128 x 64 the LDS
// operand reads were as long as the matrix work, and the kernel ran 5 %
// slower); K in steps of 128 values, staged in LDS (double buffered, rows
// padded to 80 bytes so the 16-byte operand reads of 8 or 16 consecutive
// rows hit distinct banks), global loads issued two steps ahead (two
// register staging sets).  Tiles go out in XCD super-tile order (4 x 8
// tiles per XCD per round), so the workgroups that share A and B K-slabs
// run on one L2 at the same time.  Rows past M or N read as zeros through
// the buffer-resource bounds; stores past them are dropped.
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr int kGemmThreads = 256;                  // 4 waves: 2 (M) x 2 (N)
constexpr int kGemmBM = 256, kGemmBN = 256;        // C tile per workgroup
constexpr int kGemmMI = 4, kGemmNJ = 4;            // 32 x 32 blocks per wave (128 x 128)
constexpr int kGemmBK = 128;                       // K values per step
constexpr int kGemmRowBytes = kGemmBK / 2;         // 64 code bytes per row per step
constexpr int kGemmPitch = kGemmRowBytes + 16;     // LDS row pitch (bytes)
constexpr int kGemmSuperY = 4, kGemmSuperX = 8;    // tiles per XCD super-tile

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One K step of both operands, in registers between its global load and its
// LDS store: four 16-byte pieces of each 16 KB tile per thread (piece q =
// t + 256 i: row q / 4, 16-byte column q % 4), and one scale dword (four K
// blocks of row t) of each operand.
struct GemmStage {
  u32x4_t a[4], b[4];
  uint32_t sa, sb;
};

__device__ __forceinline__ void gemm_load(GemmStage& g, __amdgpu_buffer_rsrc_t ra,
                                          __amdgpu_buffer_rsrc_t rb, __amdgpu_buffer_rsrc_t rsa,
                                          __amdgpu_buffer_rsrc_t rsb, int64_t K, int ks) {
  const int t = threadIdx.x;
  const int kb = ks * kGemmRowBytes;
  const int rowb = (int)(K / 2);
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = t + kGemmThreads * i, row = q >> 2, c = 16 * (q & 3);
    g.a[i] = __builtin_bit_cast(u32x4_t, buffer_load16(ra, row * rowb + kb + c));
    g.b[i] = __builtin_bit_cast(u32x4_t, buffer_load16(rb, row * rowb + kb + c));
  }
  const int srow = (int)(K / 32), sb = ks * (kGemmBK / 32);
  g.sa = __builtin_amdgcn_raw_buffer_load_b32(rsa, t * srow + sb, 0, 0);
  g.sb = __builtin_amdgcn_raw_buffer_load_b32(rsb, t * srow + sb, 0, 0);
}

__device__ __forceinline__ void gemm_store(const GemmStage& g, uint8_t* la, uint8_t* lb,
                                           uint32_t* lsa, uint32_t* lsb) {
  const int t = threadIdx.x;
#pragma unroll
  for (int i = 0; i < 4; i++) {
    const int q = t + kGemmThreads * i, row = q >> 2, c = 16 * (q & 3);
    *(u32x4_t*)(la + row * kGemmPitch + c) = g.a[i];
    *(u32x4_t*)(lb + row * kGemmPitch + c) = g.b[i];
  }
  lsa[t] = g.sa;
  lsb[t] = g.sb;
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
  const int wm = wave >> 1, wn = wave & 1;
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
        const int row = 128 * wn + 32 * j + r;
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
    const int64_t col = 128 * wn + 32 * j + r;
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
