// nvfp4_2d_kernels.h -- NVFP4 with one E4M3 scale per 16x16 tile (weights),
// optional Four Over Six, optional transposed output.
//
// Method: NVIDIA NVFP4 article sec. 2 and sec. 7 (2D block scaling keeps W
// and W^T quantized identically, as the chain rule needs); "Four Over Six"
// sec. 1 (per-block choice between scaling the max to 6 or to 4).
//
// Mapping onto the chip: 16 consecutive lanes hold one tile, one tile row
// per lane (32 B of bf16, two 16-byte loads).  A wave covers 16 rows x 64
// columns (4 tiles side by side: each row segment is one 128-byte line); a
// workgroup's 4 waves stack to 64 rows and walk 4 such strips to the right.
// The tile maximum and the 4/6 error sum are xor-butterflies over the 16
// lanes (offsets 1, 2, 4, 8), i.e. a pairwise tree over the 16 row errors
// whose result is bit-identical in every lane.  The transposed codes are
// the row-wise codes transposed inside the tile's 16 lanes (DPP exchanges
// and byte/nibble merges): a tile has one scale, so the transpose's code of
// an element is its row-wise code.  The codes of a workgroup tile (64 x 256 values) are
// staged in LDS and leave in 16-byte runs: 128 bytes per row row-wise, 32
// bytes per row of the transposed codes (a store that scatters 8-byte
// pieces over 64 lines costs far more).  Workgroups are persistent (the
// next tile is loaded while the current one is computed; three per CU, so
// the per-tile barrier of one is covered by the others) and take tiles in
// XCD-aware order (16x4 tiles per XCD super-tile, grid a multiple of 8) so
// the transposed codes and the scale bytes that neighbouring tiles write
// into one 64-byte segment are completed in the same L2.
#pragma once

#include "device_common.h"
#include "nvfp4_kernels.h"

namespace fp4q {

constexpr bool kHave2D = true;
constexpr int k2dStrips = 4;                 // 64-column strips per workgroup
constexpr int k2dSuperY = 16, k2dSuperX = 4; // workgroups per XCD super-tile (1024x1024 values)
// Code staging per workgroup tile (64 rows x 256 columns), two buffers:
// row-wise codes 64 rows x 128 B, transposed codes 256 rows x 32 B (pitches
// padded against bank conflicts).
constexpr int k2dRowPitch = 128 + 8;
constexpr int k2dColPitch = 32 + 8;
typedef unsigned int u32x4_nt_t __attribute__((ext_vector_type(4)));
#ifndef FP4Q_2D_WG_PER_CU
#define FP4Q_2D_WG_PER_CU 3
#endif
constexpr int k2dWgPerCu = FP4Q_2D_WG_PER_CU; // persistent workgroups per CU (LDS 48 KiB each)

struct Strips {   // one lane's tile row in each of the k2dStrips strips
  uint4 v[2 * k2dStrips];
};

// Sum over the 16 lanes of a tile, same bits in every lane.  After the
// xor-1 and xor-2 steps every group of 4 lanes holds one value, after the
// half-row mirror every group of 8, so the mirrors pair exactly the groups
// an xor-4 / xor-8 butterfly would: the sum is the pairwise tree
// ((r0+r1)+(r2+r3))+((r4+r5)+(r6+r7)) + (same for 8..15).
__device__ __forceinline__ float tile_sum(float v) {
  v = v + dpp_f<kDppXor1>(v);
  v = v + dpp_f<kDppXor2>(v);
  v = v + dpp_f<kDppHalfMirror>(v);
  return v + dpp_f<kDppMirror>(v);
}

constexpr int kDppRor8 = 0x128;           // lane i <- lane (i + 8) % 16 = i ^ 8
constexpr int kDppQuadReverse = 0x1B;     // quad_perm [3,2,1,0]

// Per-lane constants of transpose16 (lane r of its 16-lane row).
struct NibbleT {
  uint32_t sel4, sel2, mask1, rot1;
  __device__ __forceinline__ explicit NibbleT(int r)
      : sel4((r & 4) ? 0x03020706u : 0x05040100u),
        sel2((r & 2) ? 0x03070105u : 0x06020400u),
        mask1((r & 1) ? 0xF0F0F0F0u : 0x0F0F0F0Fu),
        rot1((r & 1) ? 4u : 28u) {}
};

// One 8x8 nibble matrix per 8-lane group (lane i: row i, element j in
// nibble j) -> its transpose (lane i: column i), by exchanging 4x4, 2x2 and
// 1x1 blocks with lane i ^ 4, i ^ 2, i ^ 1.
__device__ __forceinline__ uint32_t transpose8_nibbles(uint32_t v, const NibbleT& k) {
  // i ^ 4 inside each 8 lanes: half-row mirror (i -> 7 - i), then quad reverse
  uint32_t p = dpp_row_u<kDppQuadReverse>(dpp_row_u<kDppHalfMirror>(v));
  v = __builtin_amdgcn_perm(p, v, k.sel4);    // 16-bit halves: keep own, take partner's
  p = dpp_row_u<kDppXor2>(v);
  v = __builtin_amdgcn_perm(p, v, k.sel2);    // bytes
  p = dpp_row_u<kDppXor1>(v);
  p = __builtin_amdgcn_alignbit(p, p, k.rot1);
  return (k.mask1 & v) | (~k.mask1 & p);      // nibbles (one v_bfi_b32)
}

// Transpose of a 16x16 tile's 4-bit codes held one row per lane of a
// 16-lane DPP row (lane r: w0 = elements (r, 0..7), w1 = (r, 8..15), element
// j in nibble j): lane c gets column c, t0 = elements (0..7, c), t1 =
// (8..15, c).  The 8x8 blocks are exchanged with lane r ^ 8, then each 8x8
// block is transposed inside its 8 lanes.  A tile's transposed codes are its
// codes transposed (same values, same scale), so this is exact.
__device__ __forceinline__ void transpose16_nibbles(uint32_t w0, uint32_t w1, int r,
                                                    const NibbleT& k, uint32_t& t0,
                                                    uint32_t& t1) {
  const uint32_t p0 = dpp_row_u<kDppRor8>(w0), p1 = dpp_row_u<kDppRor8>(w1);
  const bool hi = (r & 8) != 0;
  t0 = transpose8_nibbles(hi ? p1 : w0, k);    // rows 0..7 of this lane's 8 columns
  t1 = transpose8_nibbles(hi ? w1 : p0, k);    // rows 8..15
}

template <bool FOUR_SIX, bool TRANSPOSE>
__global__ __launch_bounds__(kThreads) void nvfp4_2d_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols,
    const uint32_t* __restrict__ amax_bits, int namax, float* __restrict__ alpha_out,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ choice,
    uint8_t* __restrict__ codes_t, uint8_t* __restrict__ scales_t) {
  __shared__ float2 tab[128];
  __shared__ uint32_t red[kThreads / 64];
  __shared__ __align__(16) uint8_t cst_r[2][64 * k2dRowPitch];
  __shared__ __align__(16) uint8_t cst_t[2][TRANSPOSE ? 256 * k2dColPitch : 8];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int tile = lane >> 4, r = lane & 15;                 // tile in wave, row in tile
  const int64_t bcols = cols / 16, brows = rows / 16;
  const uint32_t TY = (uint32_t)((brows + 3) / 4);
  const uint32_t TX = (uint32_t)((bcols + 4 * k2dStrips - 1) / (4 * k2dStrips));
  const uint32_t nslots = (uint32_t)xcd_grid(TY, TX, k2dSuperY, k2dSuperX);

  uint32_t m = 0;
  for (int i = threadIdx.x; i < namax; i += kThreads) {
    const uint32_t a = amax_bits[i];
    m = m > a ? m : a;
  }
  m = block_max_u32(m, red);
  const TensorScale ts = tensor_scale(__uint_as_float(m), FOUR_SIX);
  if (blockIdx.x == 0 && threadIdx.x == 0) *alpha_out = ts.alpha;
  build_scale_table(tab, ts.alpha);
  __syncthreads();
  if (nslots == 0) return;                   // empty tensor: only the tensor scale

  const NibbleT nt(r);
  // Decode `slot` and load this lane's row of its 4 strips.  Every load is
  // issued (addresses clamped into the tensor) so the compiler keeps the
  // next workgroup tile's loads in flight while this one is computed;
  // values of positions outside the tensor are never stored.
  auto load = [&](uint32_t slot, Strips& in, TileOrder& to) {
    const bool valid = slot < nslots && xcd_tile<k2dSuperY, k2dSuperX>(slot, TY, TX, to);
    if (!valid) to.ty = to.tx = -1;
    const int64_t row = valid ? (to.ty * 4 + wave) * 16 + r : 0;
    const int64_t rr = row < rows ? row : rows - 1;
    const int64_t bc0 = valid ? to.tx * k2dStrips * 4 + tile : 0;
#pragma unroll
    for (int s = 0; s < k2dStrips; s++) {
      int64_t bc = bc0 + 4 * s;
      bc = bc < bcols ? bc : bcols - 1;
      const uint4* src = (const uint4*)(x + rr * cols + bc * 16);
      in.v[2 * s] = src[0];
      in.v[2 * s + 1] = src[1];
    }
  };

  // Tile work; `to.ty < 0` (a slot with no tile) is uniform over the workgroup.
  auto process = [&](const Strips& cur, const TileOrder& to, int buf) {
    if (to.ty < 0) return;
    uint8_t* cs_row = cst_r[buf];
    uint8_t* cs_col = cst_t[buf];
    const int64_t br = to.ty * 4 + wave;                 // tile row of this wave
    const bool row_ok = br < brows;
#pragma unroll
    for (int s = 0; s < k2dStrips; s++) {
      const int64_t bc = (to.tx * k2dStrips + s) * 4 + tile;   // tile column
      const bool ok = row_ok && bc < bcols;
      const uint4 v0 = cur.v[2 * s], v1 = cur.v[2 * s + 1];
      float y[16];
      unpack8(v0, y);
      unpack8(v1, y + 8);
      float amax_r = 0.0f;
#pragma unroll
      for (int k = 0; k < 16; k++) amax_r = fmaxf(amax_r, fabsf(y[k]));
      const float amax_b = tile_max(amax_r);

      uint32_t e6, e4;
      e4m3_pair(amax_b * ts.k6, amax_b * ts.k4, e6, e4);
      const float2 sr = tab[e6];
      uint32_t w0, w1, scale = e6, pick4 = 0;
      const float err6 = tile_sum(quant16_rtn(y, sr.x, sr.y, w0, w1));
      if constexpr (FOUR_SIX) {
        const float2 sr4 = tab[e4];
        uint32_t u0, u1;
        const float err4 = tile_sum(quant16_rtn(y, sr4.x, sr4.y, u0, u1));
        if (err4 < err6) {  // ties keep M = 6; identical in all 16 lanes
          w0 = u0; w1 = u1; scale = e4; pick4 = 1;
        }
      }
      *(uint2*)(cs_row + (wave * 16 + r) * k2dRowPitch + (s * 4 + tile) * 8) = make_uint2(w0, w1);
      if (ok) {
        if (r == 0) {
          scales[br * bcols + bc] = (uint8_t)scale;
          if (choice) choice[br * bcols + bc] = (uint8_t)pick4;
        }
      }
      if constexpr (TRANSPOSE) {
        // the tile's column r of codes: the row codes transposed across the
        // tile's 16 lanes (column 16*tile + r of the strip, tile row `wave`)
        uint32_t t0, t1;
        transpose16_nibbles(w0, w1, r, nt, t0, t1);
        *(uint2*)(cs_col + ((s * 4 + tile) * 16 + r) * k2dColPitch + wave * 8) = make_uint2(t0, t1);
        if (ok && r == 0) scales_t[bc * brows + br] = (uint8_t)scale;
      }
    }
    // Every wave's codes of this workgroup tile are staged: write them out
    // in contiguous runs of 16 bytes (two tiles' codes in one row).
    // Row-wise, 8 lanes cover one row's 128 bytes (a wave 8 rows);
    // transposed, 2 lanes cover the 32 bytes this tile adds to one row of
    // the transposed codes (a wave 32 rows).  At the tensor's edge a run may
    // hold one valid tile: then only its 8 bytes are stored.  The other
    // buffer takes the next tile, so one barrier per tile suffices.
    __syncthreads();
    const int64_t r0 = (int64_t)to.ty * 64, c0 = (int64_t)to.tx * 256;
#pragma unroll
    for (int i = 0; i < 2; i++) {
      const int k = (int)threadIdx.x + kThreads * i;
      const int rr = k >> 3, j = k & 7;                  // 16 bytes: tiles 2j, 2j+1
      const int64_t t0 = (int64_t)to.tx * 16 + 2 * j;
      const uint8_t* src = cs_row + rr * k2dRowPitch + j * 16;
      uint8_t* dst = codes + (r0 + rr) * (cols / 2) + (c0 >> 1) + j * 16;
      if (r0 + rr < rows && t0 < bcols) {
        const uint2 lo = *(const uint2*)src;
        if (t0 + 1 < bcols) {
          const uint2 hi = *(const uint2*)(src + 8);
          if (((uintptr_t)dst & 15) == 0) {
            // a row's 128 bytes leave whole from one wave: streaming store
            u32x4_nt_t v;
            v.x = lo.x;
            v.y = lo.y;
            v.z = hi.x;
            v.w = hi.y;
            __builtin_nontemporal_store(v, (u32x4_nt_t*)dst);
          } else {                         // rows of cols/2 bytes: 8-byte aligned only
            *(uint2*)dst = lo;
            *(uint2*)(dst + 8) = hi;
          }
        } else {
          *(uint2*)dst = lo;
        }
      }
    }
    if constexpr (TRANSPOSE) {
#pragma unroll
      for (int i = 0; i < 2; i++) {
        const int k = (int)threadIdx.x + kThreads * i;
        const int cc = k >> 1, j = k & 1;                // 16 bytes: tile rows 2j, 2j+1
        const int64_t t0 = (int64_t)to.ty * 4 + 2 * j;
        const uint8_t* src = cs_col + cc * k2dColPitch + j * 16;
        uint8_t* dst = codes_t + (c0 + cc) * (rows / 2) + (r0 >> 1) + j * 16;
        if (c0 + cc < cols && t0 < brows) {
          const uint2 lo = *(const uint2*)src;
          if (t0 + 1 < brows) {
            const uint2 hi = *(const uint2*)(src + 8);
            if (((uintptr_t)dst & 15) == 0) {
              *(uint4*)dst = make_uint4(lo.x, lo.y, hi.x, hi.y);
            } else {
              *(uint2*)dst = lo;
              *(uint2*)(dst + 8) = hi;
            }
          } else {
            *(uint2*)dst = lo;
          }
        }
      }
    }
  };

  // Two register sets in turn (no copy between them, so the wait for a
  // tile's loads never includes the previous tile's stores).
  Strips sa, sb;
  TileOrder oa, ob;
  uint32_t slot = blockIdx.x;
  load(slot, sa, oa);
  while (slot < nslots) {
    const uint32_t s1 = slot + gridDim.x;    // grid is a multiple of 8: same XCD
    load(s1, sb, ob);
    process(sa, oa, 0);
    if (s1 >= nslots) break;
    const uint32_t s2 = s1 + gridDim.x;
    load(s2, sa, oa);
    process(sb, ob, 1);
    slot = s2;
  }
}

inline hipError_t launch_nvfp4_2d(const uint16_t* x, int64_t rows, int64_t cols, bool f46,
                            const uint32_t* abits, int namax, float* alpha_out, uint8_t* codes,
                            uint8_t* scales, uint8_t* choice, uint8_t* codes_t,
                            uint8_t* scales_t, hipStream_t st, int num_cus) {
  const int64_t bcols = cols / 16, brows = rows / 16;
  const int64_t tiles_x = (bcols + 4 * k2dStrips - 1) / (4 * k2dStrips);
  const int64_t tiles_y = (brows + 3) / 4;
  const int64_t nslots = xcd_grid(tiles_y, tiles_x, k2dSuperY, k2dSuperX);
  // persistent: a multiple of 8 workgroups (XCD count); at least one, so
  // the tensor scale is written even for an empty tensor
  int64_t grid = (int64_t)num_cus * k2dWgPerCu;
  if (grid > nslots) grid = nslots;
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  if (grid < 1) grid = 1;
  const bool tr = codes_t != nullptr;
#define FP4Q_2D(F, T)                                                                     \
  launch(nvfp4_2d_kernel<F, T>, (unsigned)grid, kThreads, st, x, rows, cols, abits, namax, \
         alpha_out, codes, scales, choice, codes_t, scales_t)
  if (f46 && tr) return FP4Q_2D(true, true);
  if (f46) return FP4Q_2D(true, false);
  if (tr) return FP4Q_2D(false, true);
  return FP4Q_2D(false, false);
#undef FP4Q_2D
}

}  // namespace fp4q
