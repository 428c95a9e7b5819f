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
// SIMD) 128 x 128: 4 x 4 instructions per 64 values of K, so each operand
// register feeds four instructions.  K goes in stages of 256 values (128
// code bytes of each row: whole 128-byte lines, which the memory system
// serves markedly faster than half lines) through two LDS buffers, filled
// by direct global-to-LDS loads (buffer_load ... lds: no register staging,
// no LDS store instructions).  Within a stage each wave reads the operands
// of the next 64 values while the matrix cores work on the current ones;
// one barrier per stage, which also releases the buffer for the loads of
// the stage after next.  LDS layout of a stage: 128 bytes per operand row,
// unpadded, its eight 16-byte chunks permuted so that the reads of 16
// consecutive rows hit 16 distinct bank groups; the 8 UE8M0 bytes of a row
// per stage as two dwords, placed so that the four rows a lane multiplies
// (32 apart) are two 16-byte reads.  Bytes of K past the end (a last half
// stage, stages past K) and rows past M or N load as zeros: zero codes
// contribute exact zeros.  C goes out with non-temporal stores.  Tiles go
// out in XCD super-tile order (4 x 8 tiles per XCD per round), so the
// workgroups that share A and B K-slabs run on one L2 at the same time.
// Workgroups are persistent, one per CU, so a tile's first loads overlap
// the previous tile's C stores (16384 x 8192 x 8192: 569 -> 559 us).
#pragma once

#include "device_common.h"

namespace fp4q {

constexpr int kGemmThreads = 256;                  // 4 waves: 2 (M) x 2 (N)
constexpr int kGemmBM = 256, kGemmBN = 256;        // C tile per workgroup
constexpr int kGemmMI = 4, kGemmNJ = 4;            // 32 x 32 blocks per wave (128 x 128)
constexpr int kGemmBK = 256;                       // K values per stage
constexpr int kGemmKMultiple = 128;                // K granularity of the interface
constexpr int kGemmRowBytes = kGemmBK / 2;         // 128 code bytes per row per stage
constexpr int kGemmOpBytes = kGemmBM * kGemmRowBytes;         // 32 KiB per operand
constexpr int kGemmScaleDw = kGemmBM * (kGemmBK / 32) / 4;    // 512 scale dwords per operand
constexpr int kGemmSuperY = 4, kGemmSuperX = 8;    // tiles per XCD super-tile
constexpr uint32_t kGemmOob = 0x7FFFFF00u;         // an offset past every buffer: loads 0
constexpr int kCachePolicyNt = 2;                  // buffer-op cache policy: non-temporal

typedef int i32x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

// One LDS stage: both operands' codes and scale dwords.
struct GemmStageLds {
  uint8_t a[kGemmOpBytes];
  uint8_t b[kGemmOpBytes];
  uint32_t sa[kGemmScaleDw];
  uint32_t sb[kGemmScaleDw];
};

// Wait until at most N of this wave's vector-memory operations are
// outstanding and, with LGKM0, all of its LDS operations are done (gfx9
// s_waitcnt: vmcnt in bits 3:0 and 15:14, expcnt in 6:4, lgkmcnt in 11:8).
template <int N, bool LGKM0>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | ((LGKM0 ? 0 : 15) << 8));
}

// Workgroup barrier without a memory fence: the waits before it are
// explicit (a fence would wait for every load in flight, including those of
// the stage after next).  The empty asm statements keep the compiler from
// moving memory accesses across it.
__device__ __forceinline__ void gemm_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Bank-group permutation of the 16-byte chunks of operand row r in LDS:
// chunk c sits at position c ^ gemm_swz(r).  The 64 banks of 4 bytes hold
// two 128-byte rows; an operand read serves 16 lanes (16 consecutive rows,
// one chunk each) per pass, and gemm_swz spreads them over 16 distinct
// 16-byte bank groups (rows of one parity take 8 distinct positions), and
// any 8 consecutive rows over 8 distinct positions.
__device__ __forceinline__ int gemm_swz(int r) { return ((r >> 1) ^ (r << 2)) & 7; }

// Per-thread source offsets of the direct loads (stage 0; stage ks adds
// 128 ks to codes and 8 ks to scales).  Code load i (0..7) of wave w fills
// the stage's 1 KiB piece j = 8 w + i: 16-byte position p = 64 j + lane is
// row p / 8 = 64 w + 8 i + lane / 8, chunk (p % 8) ^ gemm_swz(row); the
// permutation depends on row % 16 only, so load i is load i % 2 moved by
// 8 (i - i % 2) rows.  Scale dwords of a stage: row
// 128 wm + 32 i + r, dword dw (bytes 4 dw .. 4 dw + 3 of its 8) at dword
// 256 wm + 128 (i / 2) + 4 r + 2 (i % 2) + dw, so that a lane's four rows
// are two 16-byte reads and 16 lanes read 256 consecutive bytes.  Scale
// load i (0..1) of wave w fills dwords 64 (2 w + i) + lane: row 128 (w / 2)
// + 32 (2 (w % 2) + lane / 2 % 2) + 16 i + lane / 4, dword lane % 2; load 1
// is load 0 moved by 16 rows.
struct GemmSrc {
  uint32_t code[2];        // loads 0 and 1: row * rowb + 16 * chunk
  uint32_t code_k[2];      // 16 * chunk: byte of the stage within its row
  uint32_t code_row[2];    // loads 0 and 1: the row (within the tile)
  uint32_t scale;          // load 0: row * srow + 4 * dw
  uint32_t scale_k;        // 4 * dw
  uint32_t scale_row;      // load 0: the row
};

__device__ __forceinline__ void gemm_src(GemmSrc& q, int rowb, int srow) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const int row = 64 * wave + 8 * i + (lane >> 3), c = (lane & 7) ^ gemm_swz(row);
    q.code[i] = (uint32_t)(row * rowb + 16 * c);
    q.code_k[i] = (uint32_t)(16 * c);
    q.code_row[i] = (uint32_t)row;
  }
  const int row = 128 * (wave >> 1) + 32 * (2 * (wave & 1) + ((lane >> 1) & 1)) + (lane >> 2);
  const int dw = lane & 1;
  q.scale = (uint32_t)(row * srow + 4 * dw);
  q.scale_k = (uint32_t)(4 * dw);
  q.scale_row = (uint32_t)row;
}

// Issue the 20 direct loads of stage ks into `st` (8 + 8 code loads of 16
// bytes, 2 + 2 scale loads of 4 bytes).  Bytes past K and rows past M (A)
// or N (B) take an offset past the buffer, so they load as zeros; the
// whole offset is per lane (the buffer's range check does not cover a
// scalar offset).
__device__ __forceinline__ void gemm_issue_stage(GemmStageLds& st, const GemmSrc& q,
                                                 __amdgpu_buffer_rsrc_t ra,
                                                 __amdgpu_buffer_rsrc_t rb,
                                                 __amdgpu_buffer_rsrc_t rsa,
                                                 __amdgpu_buffer_rsrc_t rsb, int rowb, int srow,
                                                 uint32_t mrows, uint32_t nrows, int ks) {
  // uniform: the LDS destinations are scalar (M0) addresses
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t kc = (uint32_t)(ks * kGemmRowBytes), kscale = (uint32_t)(ks * (kGemmBK / 32));
#pragma unroll
  for (int i = 0; i < 8; i++) {
    const bool kin = kc + q.code_k[i & 1] < (uint32_t)rowb;
    const uint32_t row = q.code_row[i & 1] + 8 * (i & ~1);
    const uint32_t o = q.code[i & 1] + kc + (uint32_t)(8 * (i & ~1) * rowb);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void_t*)(st.a + 1024 * (8 * wave + i)), 16,
                                             kin && row < mrows ? o : kGemmOob, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, (lds_void_t*)(st.b + 1024 * (8 * wave + i)), 16,
                                             kin && row < nrows ? o : kGemmOob, 0, 0, 0);
  }
  const bool kin = kscale + q.scale_k < (uint32_t)srow;
#pragma unroll
  for (int i = 0; i < 2; i++) {
    const uint32_t row = q.scale_row + 16 * i;
    const uint32_t o = q.scale + kscale + (uint32_t)(16 * i * srow);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsa, (lds_void_t*)(st.sa + 64 * (2 * wave + i)), 4,
                                             kin && row < mrows ? o : kGemmOob, 0, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsb, (lds_void_t*)(st.sb + 64 * (2 * wave + i)), 4,
                                             kin && row < nrows ? o : kGemmOob, 0, 0, 0);
  }
}
constexpr int kGemmLoadsPerStage = 20;

// Operands of one 64-value step of this lane: 4 A and 4 B code registers.
struct GemmOps {
  u32x4_t a[kGemmMI], b[kGemmNJ];
};
// Scale dwords of one stage for this lane's 4 A and 4 B rows: dword 2 i + d
// holds bytes 4 d .. 4 d + 3 of the stage's 8 for row block i.
struct GemmScales {
  u32x4_t a[2], b[2];
};
// The same scales as the instruction takes them: for each of the 4 A and 4
// B rows one word holding the bytes of this lane's K half, byte `sub` for
// step sub (bytes 0, 2, 4, 6 of the row's 8 for lanes 0..31, bytes 1, 3, 5,
// 7 for lanes 32..63), so the instruction's byte select picks it.
struct GemmScaleWords {
  uint32_t a[kGemmMI], b[kGemmNJ];
};

// Read the operands of step `sub` (K values 64 sub .. 64 sub + 63 of the
// stage): lane (r, g) takes chunk 2 sub + g of its rows.
__device__ __forceinline__ void gemm_read_ops(const GemmStageLds& st, int sub, GemmOps& o) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31, g = lane >> 5;
  const int pos = 16 * ((2 * sub + g) ^ gemm_swz(r));
#pragma unroll
  for (int i = 0; i < kGemmMI; i++)
    o.a[i] = *(const u32x4_t*)(st.a + (128 * wm + 32 * i + r) * kGemmRowBytes + pos);
#pragma unroll
  for (int j = 0; j < kGemmNJ; j++)
    o.b[j] = *(const u32x4_t*)(st.b + (128 * wn + 32 * j + r) * kGemmRowBytes + pos);
}

__device__ __forceinline__ void gemm_read_scales(const GemmStageLds& st, GemmScales& s) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1, r = lane & 31;
  s.a[0] = *(const u32x4_t*)(st.sa + 256 * wm + 4 * r);
  s.a[1] = *(const u32x4_t*)(st.sa + 256 * wm + 128 + 4 * r);
  s.b[0] = *(const u32x4_t*)(st.sb + 256 * wn + 4 * r);
  s.b[1] = *(const u32x4_t*)(st.sb + 256 * wn + 128 + 4 * r);
}

__device__ __forceinline__ void gemm_scale_words(const GemmScales& s, GemmScaleWords& w) {
  // v_perm_b32 byte selects over (hi = bytes 4..7, lo = bytes 0..3)
  const uint32_t sel = (threadIdx.x & 32) ? 0x07050301u : 0x06040200u;
#pragma unroll
  for (int i = 0; i < kGemmMI; i++)
    w.a[i] = __builtin_amdgcn_perm(s.a[i >> 1][2 * (i & 1) + 1], s.a[i >> 1][2 * (i & 1)], sel);
#pragma unroll
  for (int j = 0; j < kGemmNJ; j++)
    w.b[j] = __builtin_amdgcn_perm(s.b[j >> 1][2 * (j & 1) + 1], s.b[j >> 1][2 * (j & 1)], sel);
}

// The 16 matrix instructions of step SUB; the scale byte is selected by
// the instruction (op_sel), from the words of gemm_scale_words.
template <int SUB>
__device__ __forceinline__ void gemm_mfma_step(f32x16_t (&acc)[kGemmMI][kGemmNJ],
                                               const GemmOps& o, const GemmScaleWords& w) {
  // FP4 operands fill the low four registers of the instruction's eight; the
  // upper four are not read (left undefined rather than zeroed)
#pragma unroll
  for (int i = 0; i < kGemmMI; i++) {
    const i32x8_t av = __builtin_shufflevector((i32x4_t)o.a[i], (i32x4_t)o.a[i], 0, 1, 2, 3, -1,
                                               -1, -1, -1);
#pragma unroll
    for (int j = 0; j < kGemmNJ; j++) {
      const i32x8_t bv = __builtin_shufflevector((i32x4_t)o.b[j], (i32x4_t)o.b[j], 0, 1, 2, 3, -1,
                                                 -1, -1, -1);
      acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
          av, bv, acc[i][j], 4, 4, SUB, (int)w.a[i], SUB, (int)w.b[j]);
    }
  }
}

// Instruction order hints for the scheduler (masks: 0x008 matrix, 0x100
// LDS read) for steps 0..2 of a stage: each matrix instruction of the first
// half of a step is followed by one LDS read of the next step's operands.
__device__ __forceinline__ void gemm_order_steps012() {
#pragma unroll
  for (int st = 0; st < 3; st++) {
#pragma unroll
    for (int k = 0; k < 8; k++) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 8, 0);
  }
}
__global__ __launch_bounds__(kGemmThreads) void mxfp4_gemm_kernel(
    const uint8_t* __restrict__ a_codes, const uint8_t* __restrict__ a_scales,
    const uint8_t* __restrict__ bt_codes, const uint8_t* __restrict__ bt_scales, int64_t M,
    int64_t N, int64_t K, float* __restrict__ c_out, uint32_t tiles_m, uint32_t tiles_n) {
  __shared__ __attribute__((aligned(16))) GemmStageLds ring[2];   // stage ks in ring[ks % 2]

  // Persistent: workgroup w takes slots w, w + G, w + 2G, ... (G a multiple
  // of 8, so every slot of a workgroup maps to its own XCD).  After the
  // first tile, each wave's LDS reads of the last stage are waited for and
  // the workgroup meets at a barrier before the next tile's loads refill
  // the ring; those loads go out while the previous tile's C stores drain.
  const uint32_t nslots = (uint32_t)xcd_grid(tiles_m, tiles_n, kGemmSuperY, kGemmSuperX);
  for (uint32_t slot = blockIdx.x; slot < nslots; slot += gridDim.x) {
    if (slot != blockIdx.x) {
      __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));   // lgkmcnt(0) only
      gemm_barrier();
    }
    TileOrder to;
    if (!xcd_tile<kGemmSuperY, kGemmSuperX>(slot, tiles_m, tiles_n, to)) continue;  // uniform
    const int64_t m0 = to.ty * kGemmBM, n0 = to.tx * kGemmBN;
    const int64_t mrows = M - m0 < kGemmBM ? M - m0 : kGemmBM;
    const int64_t nrows = N - n0 < kGemmBN ? N - n0 : kGemmBN;
    const int rowb = (int)(K / 2), srow = (int)(K / 32);
    // resources over this tile's rows of each operand (rows past M / N read 0)
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a_codes + m0 * rowb), 0, (int)(mrows * rowb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(bt_codes + n0 * rowb), 0, (int)(nrows * rowb), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(a_scales + m0 * srow), 0, (int)(mrows * srow), 0x00020000);
    const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(bt_scales + n0 * srow), 0, (int)(nrows * srow), 0x00020000);
    GemmSrc q;
    gemm_src(q, rowb, srow);
    const uint32_t mr = (uint32_t)mrows, nr = (uint32_t)nrows;

    f32x16_t acc[kGemmMI][kGemmNJ];
#pragma unroll
    for (int i = 0; i < kGemmMI; i++)
#pragma unroll
      for (int j = 0; j < kGemmNJ; j++) acc[i][j] = f32x16_t{};

    const int nk = (int)((K + kGemmBK - 1) / kGemmBK);
    // Stage ks (operands of its step 0 and its scales already in registers):
    //   steps 0..2: the 16 instructions of the step, with the operand reads
    //     of the next step in between;
    //   wait until this wave's LDS reads are done and its loads of stage
    //     ks + 1 have landed, then the barrier: ring[(ks + 1) % 2] is whole
    //     and nobody reads ring[ks % 2] any more;
    //   issue the loads of stage ks + 2 into ring[ks % 2] (first: they get
    //     the most time, and the TA works through them during step 3);
    //   step 3, with the reads of stage ks + 1's scales and step-0 operands.
    // The loads of a stage have four steps (64 instructions) to arrive.
    gemm_issue_stage(ring[0], q, ra, rb, rsa, rsb, rowb, srow, mr, nr, 0);
    gemm_issue_stage(ring[1], q, ra, rb, rsa, rsb, rowb, srow, mr, nr, 1);
    wait_vmcnt<kGemmLoadsPerStage, false>();
    gemm_barrier();
    GemmOps o0, o1;
    GemmScales rs;
    GemmScaleWords sc, nsc;
    gemm_read_scales(ring[0], rs);
    gemm_scale_words(rs, sc);
    gemm_read_ops(ring[0], 0, o0);
    // the two buffers alternate by name (unrolled by two), so that the
    // compiler sees which one each LDS read and direct load touches
    auto stage = [&](GemmStageLds& cur, GemmStageLds& nxt, int ks) {
      gemm_read_ops(cur, 1, o1);
      gemm_mfma_step<0>(acc, o0, sc);
      gemm_read_ops(cur, 2, o0);
      gemm_mfma_step<1>(acc, o1, sc);
      gemm_read_ops(cur, 3, o1);
      gemm_mfma_step<2>(acc, o0, sc);
      gemm_order_steps012();
      wait_vmcnt<0, true>();
      gemm_barrier();
      gemm_issue_stage(cur, q, ra, rb, rsa, rsb, rowb, srow, mr, nr, ks + 2);
      gemm_read_scales(nxt, rs);
      gemm_read_ops(nxt, 0, o0);
      gemm_scale_words(rs, nsc);
      gemm_mfma_step<3>(acc, o1, sc);
      sc = nsc;
    };
    for (int ks = 0; ks < nk; ks += 2) {
      stage(ring[0], ring[1], ks);
      if (ks + 1 < nk) stage(ring[1], ring[0], ks + 1);
    }
    wait_vmcnt<0, false>();     // the zero-filled loads past the last stage

    // C tile: lane holds D[8 (v / 4) + 4 g + v % 4][r] of each 32 x 32 block;
    // each store writes two 128-byte row pieces.  Non-temporal hint: C is not
    // read again here and should not push the operand slabs out of L2.
    // Columns past N are dropped by the test, rows past M by the buffer bounds.
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1, r = lane & 31, g = lane >> 5;
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
                                                  (int)((row * N + n0 + col) * 4), 0,
                                                  kCachePolicyNt);
          }
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
