// fp4q.hip -- C ABI of libfp4q.so: argument checks on the host, then kernel
// launches on the caller's stream.  See include/fp4q.h for the contract.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "../../include/fp4q.h"
#include "msed_kernels.h"
#include "mxgemm_kernels.h"
#include "mx_kernels.h"
#include "nvfp4_2d_kernels.h"
#include "nvfp4_kernels.h"
#include "requant_kernels.h"
#include "rows_kernels.h"

using namespace fp4q;

// Workspace of nvfp4_quantize_noalloc: the amax pass's per-workgroup partial
// maxima, in a fixed device array instead of caller memory.  Each device
// holds its own copy (at its own address) until the process ends.  In host
// code `scratch` names a host-side stand-in, never the device memory: the
// device address comes from hipGetSymbolAddress (scratch_address below).
constexpr size_t kScratchBytes = 4096;
static __device__ __align__(256) uint32_t scratch[kScratchBytes / sizeof(uint32_t)];

namespace {

constexpr int64_t kMaxElems = (int64_t)1 << 40;
constexpr uint32_t kNvfp4Flags = FP4_FOUR_OVER_SIX | FP4_SR | FP4_RHT16 | FP4_BLOCK2D |
                                 FP4_ROWWISE | FP4_COLWISE | FP4_MSEDEN;
constexpr uint32_t kMxFlags = FP4_HAD32 | FP4_ROWWISE | FP4_COLWISE;

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int check_shape(int64_t rows, int64_t cols) {
  if (rows < 0 || cols < 0) return FP4_E_SHAPE;
  if (rows > 0 && cols > 0 && (rows >= kMaxElems || cols >= kMaxElems || rows * cols >= kMaxElems))
    return FP4_E_SHAPE;
  return FP4_OK;
}

int check_nvfp4_flags(uint32_t flags) {
  if (flags & ~kNvfp4Flags) return FP4_E_FLAGS;
  if ((flags & FP4_SR) && (flags & FP4_FOUR_OVER_SIX)) return FP4_E_FLAGS;
  if ((flags & FP4_BLOCK2D) && (flags & (FP4_SR | FP4_RHT16))) return FP4_E_FLAGS;
  if ((flags & FP4_COLWISE) && !(flags & FP4_BLOCK2D)) return FP4_E_FLAGS;
  if ((flags & FP4_MSEDEN) &&
      (!(flags & FP4_RHT16) || (flags & (FP4_SR | FP4_FOUR_OVER_SIX | FP4_BLOCK2D))))
    return FP4_E_FLAGS;
  return FP4_OK;
}

// The amax pass with the 1D quantizer's smaller workgroups: neither 2D
// tiles nor the rotation (whose pass is bound by the butterflies).
bool amax_one_d(uint32_t flags) { return !(flags & (FP4_BLOCK2D | FP4_RHT16)); }

// Workgroups of the amax pass: the 1D quantizer's (one_d) or the others'.
int amax_groups(int64_t ngroups16, bool one_d) {
  const int64_t per_group =                                          // uint4 loads per workgroup pass
      (int64_t)(one_d ? kAmaxThreads1d : kAmaxThreads) * kAmaxUnroll;
  const int64_t cap = one_d ? kAmaxMaxGroups1d : kAmaxMaxGroups;
  int64_t g = cdiv(ngroups16 * 2, per_group);
  if (g < 1) g = 1;
  if (g > cap) g = cap;
  return (int)g;
}

// Status of the launches an entry point queued (each launch reports its own
// result, see launch(); the thread's last-error state is never read).
int launched(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_E_HIP; }

// First failure of a sequence of launches.
hipError_t first(hipError_t a, hipError_t b) { return a != hipSuccess ? a : b; }

// Compute units of the current device (queried once per device; 256 on MI355X).
int num_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}

// Queue the amax pass: partial maxima into ws (as uint32), `groups` of them.
hipError_t launch_amax_partial(const uint16_t* x, int64_t ngroups16, uint32_t flags,
                               uint64_t seed, uint32_t* ws, int groups, bool one_d,
                               hipStream_t st) {
  const uint32_t lo = (uint32_t)seed, hi = (uint32_t)(seed >> 32);
  if (flags & FP4_RHT16)                 // one_d is false here (amax_one_d)
    return launch(amax_partial_kernel<true, kAmaxThreads>, groups, kAmaxThreads, st,
                  (const uint4*)x, ngroups16, ws, lo, hi);
  if (one_d)
    return launch(amax_partial_kernel<false, kAmaxThreads1d>, groups, kAmaxThreads1d, st,
                  (const uint4*)x, ngroups16, ws, lo, hi);
  return launch(amax_partial_kernel<false, kAmaxThreads>, groups, kAmaxThreads, st,
                (const uint4*)x, ngroups16, ws, lo, hi);
}

template <bool F46, bool SR, bool RHT>
hipError_t launch_1d(const uint16_t* x, int64_t nblocks, const uint32_t* abits, int namax,
                     float* alpha_out, uint8_t* codes, uint8_t* scales, uint8_t* choice,
                     uint64_t seed, hipStream_t st) {
  int64_t grid = nblocks > 0 ? cdiv(nblocks, (int64_t)kThreads) : 1;
  const int64_t resident = (int64_t)num_cus() * (SR ? kWgPerCu : kWgPerCuNoSr);
  if (grid > resident) grid = resident;
  return launch(nvfp4_1d_kernel<F46, SR, RHT>, (unsigned)grid, kThreads, st, (const uint4*)x,
                nblocks, abits, namax, alpha_out, (uint2*)codes, scales, choice, (uint32_t)seed,
                (uint32_t)(seed >> 32));
}

// Device address of `scratch` on the current device, looked up once per
// device (with that device current) and kept.
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return FP4_E_HIP;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return FP4_E_HIP;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return FP4_OK;
}

template <bool F46, bool SR, bool RHT>
hipError_t launch_requant(const uint8_t* codes, const uint8_t* scales, const float* alpha, int64_t rows,
                    int64_t cols, const float* amax_in, uint32_t* ws, float* alpha_out,
                    uint8_t* codes_t, uint8_t* scales_t, uint8_t* choice_t, uint64_t seed,
                    hipStream_t st) {
  const uint32_t lo = (uint32_t)seed, hi = (uint32_t)(seed >> 32);
  // grids are multiples of 8 (one equal share of the tiles per XCD) once
  // there are 8 tiles
  const uint32_t TY = (uint32_t)cdiv(rows, kRqTileRows), TX = (uint32_t)cdiv(cols, kRqTileCols);
  const int64_t ntiles = (int64_t)TY * TX;
  auto grid = [&](int64_t cap) {
    int64_t g = ntiles < cap ? ntiles : cap;
    if (g >= 8) g -= g % 8;
    return g < 1 ? (int64_t)1 : g;
  };
  const int64_t launched = (int64_t)num_cus() * kRqWgPerCu;
  const uint32_t* abits = (const uint32_t*)amax_in;
  int namax = 1;
  hipError_t e = hipSuccess;
  if (!amax_in) {
    const int64_t ga = grid(launched < kRqAmaxGroups ? launched : kRqAmaxGroups);
    e = launch(rq_amax_kernel<RHT>, (unsigned)ga, kRqThreads, st, codes, scales, alpha, rows,
               cols, TY, TX, ws, lo, hi);
    abits = ws;
    namax = (int)ga;
  }
  return first(e, launch(rq_quant_kernel<F46, SR, RHT>, (unsigned)grid(launched), kRqThreads, st,
                         codes, scales, alpha, rows, cols, TY, TX, abits, namax, alpha_out,
                         codes_t, scales_t, choice_t, lo, hi));
}

// Persistent grid: `over` times as many workgroups of `kernel` as fit on
// the chip at once (its register use sets that; queried once per kernel),
// at most `want`.
int64_t resident_grid(const void* kernel, int& per_cu, int64_t want, int over = 1) {
  if (per_cu == 0) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, kRowThreads, 0) != hipSuccess ||
        n < 1)
      n = 2;
    per_cu = n < kRowWgPerCu ? n : kRowWgPerCu;
  }
  const int64_t cap = (int64_t)num_cus() * per_cu * over;
  int64_t g = want < cap ? want : cap;
  return g < 1 ? 1 : g;
}

template <bool F46, bool SR, bool RHT, int NB>
hipError_t launch_rows_wave(const uint16_t* x, int64_t rows, int64_t cols, float* alpha_rows,
                            uint8_t* codes, uint8_t* scales, uint8_t* choice, uint64_t seed,
                            hipStream_t st) {
  static int per_cu = 0;
  const int64_t grid = resident_grid((const void*)nvfp4_rows_kernel<F46, SR, RHT, NB>, per_cu,
                                     cdiv(rows, kRowWaves));
  return launch(nvfp4_rows_kernel<F46, SR, RHT, NB>, (unsigned)grid, kRowThreads, st, x, rows,
                cols, alpha_rows, codes, scales, choice, (uint32_t)seed, (uint32_t)(seed >> 32));
}

template <bool F46, bool SR, bool RHT, int NB, bool ONE>
hipError_t launch_rows_wg(const uint16_t* x, int64_t rows, int64_t cols, float* alpha_rows,
                          uint8_t* codes, uint8_t* scales, uint8_t* choice, uint64_t seed,
                          hipStream_t st) {
  static int per_cu = 0;
  const int64_t grid =
      resident_grid((const void*)nvfp4_rows_wg_kernel<F46, SR, RHT, NB, ONE>, per_cu, rows,
                    kRowWgLaunch);
  return launch(nvfp4_rows_wg_kernel<F46, SR, RHT, NB, ONE>, (unsigned)grid, kRowThreads, st, x,
                rows, cols, alpha_rows, codes, scales, choice, (uint32_t)seed,
                (uint32_t)(seed >> 32));
}

// Rows of up to 128 blocks: one wave per row (1 or 2 blocks per lane).
// Longer rows: one workgroup per row, 1, 2 or 4 blocks per thread held in
// registers (rows up to 16384 values are read once); beyond that two
// sweeps over the row, the second from cache.
template <bool F46, bool SR, bool RHT>
hipError_t launch_rows(const uint16_t* x, int64_t rows, int64_t cols, float* alpha_rows,
                       uint8_t* codes, uint8_t* scales, uint8_t* choice, uint64_t seed,
                       hipStream_t st) {
  const int64_t nblk = cols / 16;
#define FP4Q_ARGS x, rows, cols, alpha_rows, codes, scales, choice, seed, st
  if (nblk <= 64) return launch_rows_wave<F46, SR, RHT, 1>(FP4Q_ARGS);
  if (nblk <= 128) return launch_rows_wave<F46, SR, RHT, 2>(FP4Q_ARGS);
  if (nblk <= 256) return launch_rows_wg<F46, SR, RHT, 1, true>(FP4Q_ARGS);
  if (nblk <= 512) return launch_rows_wg<F46, SR, RHT, 2, true>(FP4Q_ARGS);
  if (nblk <= 1024) return launch_rows_wg<F46, SR, RHT, 4, true>(FP4Q_ARGS);
  return launch_rows_wg<F46, SR, RHT, 4, false>(FP4Q_ARGS);
#undef FP4Q_ARGS
}

}  // namespace

extern "C" {

int fp4_abi_version(void) { return 2; }

const char* fp4_status_str(int status) {
  switch (status) {
    case FP4_OK: return "ok";
    case FP4_E_NULL: return "a required pointer is NULL";
    case FP4_E_SHAPE: return "shape not supported (negative, not a block multiple, or too large)";
    case FP4_E_ALIGN: return "pointer misaligned (tensors and code buffers need 16-byte alignment)";
    case FP4_E_FLAGS: return "unsupported flag combination";
    case FP4_E_WORKSPACE: return "workspace smaller than fp4_workspace_bytes()";
    case FP4_E_HIP: return "HIP kernel launch failed";
    default: return "unknown status";
  }
}

size_t fp4_workspace_bytes(int64_t rows, int64_t cols, uint32_t flags) {
  (void)rows; (void)cols;
  if (flags & FP4_HAD32) return 0;
  const int groups = kAmaxMaxGroupsAll > kRqAmaxGroups ? kAmaxMaxGroupsAll : kRqAmaxGroups;
  return (size_t)groups * sizeof(uint32_t);
}

int fp4_tensor_amax(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                    uint64_t seed, float* amax_out, void* ws, size_t ws_bytes, void* stream) {
  const int64_t n = rows * cols;
  if (!amax_out || !ws || (n > 0 && !x)) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  if (cols % 16) return FP4_E_SHAPE;
  if (int rc = check_nvfp4_flags(flags)) return rc;
  if (!aligned(x, 16) || !aligned(amax_out, 4) || !aligned(ws, 4)) return FP4_E_ALIGN;
  if (ws_bytes < fp4_workspace_bytes(rows, cols, flags)) return FP4_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  const int64_t ng = n / 16;
  const bool one_d = amax_one_d(flags);
  const int groups = amax_groups(ng, one_d);
  const hipError_t e = launch_amax_partial(x, ng, flags, seed, (uint32_t*)ws, groups, one_d, st);
  return launched(first(e, launch(amax_finalize_kernel, 1, kThreads, st, (const uint32_t*)ws,
                                  groups, amax_out)));
}

}  // extern "C"

namespace {

// Argument checks of nvfp4_quantize (and its no-allocation variant, with
// the library's array as ws).
int check_nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                         const float* amax_in, const float* alpha_out, const uint8_t* codes,
                         const uint8_t* scales, const uint8_t* codes_t, const uint8_t* scales_t,
                         const void* ws, size_t ws_bytes) {
  const int64_t n = rows * cols;
  const bool two_d = (flags & FP4_BLOCK2D) != 0;
  const bool want_t = two_d && (flags & FP4_COLWISE);
  if (!alpha_out) return FP4_E_NULL;
  if (n > 0 && (!x || !codes || !scales)) return FP4_E_NULL;
  if (n > 0 && want_t && (!codes_t || !scales_t)) return FP4_E_NULL;
  if (!amax_in && !ws) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  if (cols % 16 || (two_d && rows % 16)) return FP4_E_SHAPE;
  if (int rc = check_nvfp4_flags(flags)) return rc;
  if (two_d && !kHave2D) return FP4_E_FLAGS;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(alpha_out, 4) || !aligned(amax_in, 4) ||
      !aligned(ws, 4) || (want_t && !aligned(codes_t, 16)))
    return FP4_E_ALIGN;
  if (!amax_in && ws_bytes < fp4_workspace_bytes(rows, cols, flags)) return FP4_E_WORKSPACE;
  return FP4_OK;
}

}  // namespace

extern "C" {

int nvfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
                   const float* amax_in, float* alpha_out, uint8_t* codes, uint8_t* scales,
                   uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t, void* ws,
                   size_t ws_bytes, void* stream) {
  if (int rc = check_nvfp4_quantize(x, rows, cols, flags, amax_in, alpha_out, codes, scales,
                                    codes_t, scales_t, ws, ws_bytes))
    return rc;
  const int64_t n = rows * cols;
  const bool two_d = (flags & FP4_BLOCK2D) != 0;
  const bool want_t = two_d && (flags & FP4_COLWISE);
  hipStream_t st = (hipStream_t)stream;
  const int64_t nblocks = n / 16;
  const uint32_t* abits = (const uint32_t*)amax_in;
  int namax = 1;
  hipError_t e = hipSuccess;
  if (!amax_in) {
    const bool one_d = amax_one_d(flags);
    namax = amax_groups(nblocks, one_d);
    e = launch_amax_partial(x, nblocks, flags, seed, (uint32_t*)ws, namax, one_d, st);
    abits = (const uint32_t*)ws;
  }
  if (two_d) {
    const bool f46 = (flags & FP4_FOUR_OVER_SIX) != 0;
    return launched(first(e, launch_nvfp4_2d(x, rows, cols, f46, abits, namax, alpha_out, codes,
                                             scales, choice, want_t ? codes_t : nullptr,
                                             want_t ? scales_t : nullptr, st, num_cus())));
  }
  if (flags & FP4_MSEDEN) {              // always with RHT16 (checked above)
    int64_t grid = nblocks > 0 ? cdiv(nblocks, (int64_t)kThreads) : 1;
    if (grid > (int64_t)num_cus() * kWgPerCu) grid = (int64_t)num_cus() * kWgPerCu;
    return launched(first(e, launch(nvfp4_msed_kernel<true>, (unsigned)grid, kThreads, st,
                                    (const uint4*)x, nblocks, abits, namax, alpha_out,
                                    (uint2*)codes, scales, choice, (uint32_t)seed,
                                    (uint32_t)(seed >> 32))));
  }
  const bool f46 = flags & FP4_FOUR_OVER_SIX, sr = flags & FP4_SR, rht = flags & FP4_RHT16;
#define FP4Q_1D(F, S, R) \
  launch_1d<F, S, R>(x, nblocks, abits, namax, alpha_out, codes, scales, choice, seed, st)
  if (f46 && rht) e = first(e, FP4Q_1D(true, false, true));
  else if (f46) e = first(e, FP4Q_1D(true, false, false));
  else if (sr && rht) e = first(e, FP4Q_1D(false, true, true));
  else if (sr) e = first(e, FP4Q_1D(false, true, false));
  else if (rht) e = first(e, FP4Q_1D(false, false, true));
  else e = first(e, FP4Q_1D(false, false, false));
#undef FP4Q_1D
  return launched(e);
}

int nvfp4_quantize_noalloc(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                           uint64_t seed, const float* amax_in, float* alpha_out, uint8_t* codes,
                           uint8_t* scales, uint8_t* choice, uint8_t* codes_t, uint8_t* scales_t,
                           void* stream) {
  static_assert(kAmaxMaxGroupsAll * sizeof(uint32_t) <= kScratchBytes, "amax partials fit");
  if (amax_in)                           // no amax pass: no workspace at all
    return nvfp4_quantize(x, rows, cols, flags, seed, amax_in, alpha_out, codes, scales, choice,
                          codes_t, scales_t, nullptr, 0, stream);
  // every argument check first (the array stands in for ws), then the
  // array's device address
  if (int rc = check_nvfp4_quantize(x, rows, cols, flags, amax_in, alpha_out, codes, scales,
                                    codes_t, scales_t, &g_scratch, kScratchBytes))
    return rc;
  void* ws = nullptr;
  if (int rc = scratch_address(&ws)) return rc;
  return nvfp4_quantize(x, rows, cols, flags, seed, nullptr, alpha_out, codes, scales, choice,
                        codes_t, scales_t, ws, kScratchBytes, stream);
}

int nvfp4_requantize_t(const uint8_t* codes, const uint8_t* scales, const float* alpha,
                       int64_t rows, int64_t cols, uint32_t flags, uint64_t seed,
                       const float* amax_in, float* alpha_out, uint8_t* codes_t,
                       uint8_t* scales_t, uint8_t* choice_t, void* ws, size_t ws_bytes,
                       void* stream) {
  const int64_t n = rows * cols;
  if (!alpha || !alpha_out || (!amax_in && !ws)) return FP4_E_NULL;
  if (n > 0 && (!codes || !scales || !codes_t || !scales_t)) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  if (rows % 16 || cols % 16) return FP4_E_SHAPE;
  if (flags & ~(uint32_t)(FP4_FOUR_OVER_SIX | FP4_SR | FP4_RHT16)) return FP4_E_FLAGS;
  if (int rc = check_nvfp4_flags(flags)) return rc;
  if (!aligned(codes, 16) || !aligned(codes_t, 16) || !aligned(alpha, 4) ||
      !aligned(alpha_out, 4) || !aligned(amax_in, 4) || !aligned(ws, 4))
    return FP4_E_ALIGN;
  if (!amax_in && ws_bytes < fp4_workspace_bytes(rows, cols, flags)) return FP4_E_WORKSPACE;
  hipStream_t st = (hipStream_t)stream;
  uint32_t* w = (uint32_t*)ws;
  const bool f46 = flags & FP4_FOUR_OVER_SIX, sr = flags & FP4_SR, rht = flags & FP4_RHT16;
#define FP4Q_RQ(F, S, R)                                                                     \
  launch_requant<F, S, R>(codes, scales, alpha, rows, cols, amax_in, w, alpha_out, codes_t, \
                          scales_t, choice_t, seed, st)
  hipError_t e;
  if (f46 && rht) e = FP4Q_RQ(true, false, true);
  else if (f46) e = FP4Q_RQ(true, false, false);
  else if (sr && rht) e = FP4Q_RQ(false, true, true);
  else if (sr) e = FP4Q_RQ(false, true, false);
  else if (rht) e = FP4Q_RQ(false, false, true);
  else e = FP4Q_RQ(false, false, false);
#undef FP4Q_RQ
  return launched(e);
}

int nvfp4_quantize_rows(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                        uint64_t seed, float* alpha_rows, uint8_t* codes, uint8_t* scales,
                        uint8_t* choice, void* stream) {
  const int64_t n = rows * cols;
  if (n > 0 && (!x || !alpha_rows || !codes || !scales)) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  if (cols % 16) return FP4_E_SHAPE;
  if (flags & ~(uint32_t)(FP4_FOUR_OVER_SIX | FP4_SR | FP4_RHT16)) return FP4_E_FLAGS;
  if (int rc = check_nvfp4_flags(flags)) return rc;
  if (!aligned(x, 16) || !aligned(codes, 16) || !aligned(alpha_rows, 4)) return FP4_E_ALIGN;
  if (n == 0) return FP4_OK;
  hipStream_t st = (hipStream_t)stream;
  const bool f46 = flags & FP4_FOUR_OVER_SIX, sr = flags & FP4_SR, rht = flags & FP4_RHT16;
#define FP4Q_ROWS(F, S, R) \
  launch_rows<F, S, R>(x, rows, cols, alpha_rows, codes, scales, choice, seed, st)
  hipError_t e;
  if (f46 && rht) e = FP4Q_ROWS(true, false, true);
  else if (f46) e = FP4Q_ROWS(true, false, false);
  else if (sr && rht) e = FP4Q_ROWS(false, true, true);
  else if (sr) e = FP4Q_ROWS(false, true, false);
  else if (rht) e = FP4Q_ROWS(false, false, true);
  else e = FP4Q_ROWS(false, false, false);
#undef FP4Q_ROWS
  return launched(e);
}

int mxfp4_quantize(const uint16_t* x, int64_t rows, int64_t cols, uint32_t flags,
                   uint8_t* codes_r, uint8_t* scales_r, uint8_t* codes_c, uint8_t* scales_c,
                   void* stream) {
  const int64_t n = rows * cols;
  const bool rw = flags & FP4_ROWWISE, cw = flags & FP4_COLWISE;
  if (n > 0 && !x) return FP4_E_NULL;
  if (n > 0 && rw && (!codes_r || !scales_r)) return FP4_E_NULL;
  if (n > 0 && cw && (!codes_c || !scales_c)) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  if ((flags & ~kMxFlags) || !(rw || cw) || !kHaveMx) return FP4_E_FLAGS;
  if (cols % 8 || (rw && cols % 32) || (cw && rows % 32)) return FP4_E_SHAPE;
  if (!aligned(x, 16) || (rw && !aligned(codes_r, 16)) || (cw && !aligned(codes_c, 16)))
    return FP4_E_ALIGN;
  if (n == 0) return FP4_OK;
  return launched(launch_mxfp4(x, rows, cols, (flags & FP4_HAD32) != 0, rw ? codes_r : nullptr,
                              rw ? scales_r : nullptr, cw ? codes_c : nullptr,
                              cw ? scales_c : nullptr, (hipStream_t)stream, num_cus()));
}

int mxfp4_gemm(const uint8_t* a_codes, const uint8_t* a_scales, const uint8_t* bt_codes,
               const uint8_t* bt_scales, int64_t M, int64_t N, int64_t K, float* c,
               void* stream) {
  if (M < 0 || N < 0 || K < 0) return FP4_E_SHAPE;
  if (K % kGemmKMultiple) return FP4_E_SHAPE;
  if ((M > 0 && K > 0 && (!a_codes || !a_scales)) || (N > 0 && K > 0 && (!bt_codes || !bt_scales)) ||
      (M > 0 && N > 0 && !c))
    return FP4_E_NULL;
  // buffer resources and offsets span one 256-row tile: K < 2^23 and
  // N < 2^20 keep them below 2^30 bytes
  if (K >= ((int64_t)1 << 23) || N >= ((int64_t)1 << 20) || M >= ((int64_t)1 << 40) / (N > 0 ? N : 1))
    return FP4_E_SHAPE;
  if (!aligned(a_codes, 16) || !aligned(bt_codes, 16) || !aligned(a_scales, 4) ||
      !aligned(bt_scales, 4) || !aligned(c, 4))
    return FP4_E_ALIGN;
  if (M == 0 || N == 0) return FP4_OK;
  if (K == 0) {                           // empty sum: C = 0
    int64_t grid = cdiv(M * N, 256);
    if (grid > 4096) grid = 4096;
    return launched(launch(fill_zero_kernel, (unsigned)grid, 256, (hipStream_t)stream, c, M * N));
  }
  const int64_t tiles_m = cdiv(M, kGemmBM), tiles_n = cdiv(N, kGemmBN);
  // persistent: one workgroup per CU (its LDS ring fills most of the CU's),
  // a multiple of 8 of them
  const int64_t slots = xcd_grid(tiles_m, tiles_n, kGemmSuperY, kGemmSuperX);
  int64_t grid = slots < num_cus() ? slots : num_cus();
  grid = (grid + kXcds - 1) / kXcds * kXcds;
  return launched(launch(mxfp4_gemm_kernel, (unsigned)grid, kGemmThreads, (hipStream_t)stream,
                         a_codes, a_scales, bt_codes, bt_scales, M, N, K, c, (uint32_t)tiles_m,
                         (uint32_t)tiles_n));
}

int fp4_dequantize(int format, const uint8_t* codes, const uint8_t* scales, const float* alpha,
                   int64_t rows, int64_t cols, uint32_t flags, float* out, void* stream) {
  const int64_t n = rows * cols;
  if (format != FP4_FORMAT_NVFP4 && format != FP4_FORMAT_MXFP4) return FP4_E_FLAGS;
  if (n > 0 && (!codes || !scales || !out)) return FP4_E_NULL;
  if (format == FP4_FORMAT_NVFP4 && !alpha) return FP4_E_NULL;
  if (int rc = check_shape(rows, cols)) return rc;
  const bool two_d = (flags & FP4_BLOCK2D) != 0;
  if (format == FP4_FORMAT_NVFP4) {
    if (flags & ~(uint32_t)FP4_BLOCK2D) return FP4_E_FLAGS;
    if (cols % 16 || (two_d && rows % 16)) return FP4_E_SHAPE;
  } else {
    if (flags) return FP4_E_FLAGS;
    if (cols % 32) return FP4_E_SHAPE;
  }
  if (!aligned(codes, 16) || !aligned(out, 16) || !aligned(alpha, 4)) return FP4_E_ALIGN;
  if (n == 0) return FP4_OK;
  hipStream_t st = (hipStream_t)stream;
  if (format == FP4_FORMAT_NVFP4) {
    const int64_t nb = n / 16;
    return launched(launch(nvfp4_dequant_kernel, (unsigned)cdiv(nb, kThreads), kThreads, st,
                           (const uint2*)codes, scales, alpha, nb, cols / 16, two_d,
                           (float4*)out));
  }
  const int64_t ng = n / 32;
  return launched(launch(mxfp4_dequant_kernel, (unsigned)cdiv(ng, kThreads), kThreads, st,
                         (const uint4*)codes, scales, ng, (float4*)out));
}

}  // extern "C"
