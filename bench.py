#!/usr/bin/env python3
"""Throughput of block-scaled FP4 quantization on one MI355X.

Headline: NVFP4 Four-Over-Six quantization of an 8192x4096 bf16 activation
tensor.  A step is one full pass of the path over one input: the tensor amax
pass (Eq. 1 of "Four Over Six") and the block quantizer (Eq. 2-3 with the
4/6 choice), i.e. one ``nvfp4_quantize`` call with the amax computed inside.
Inputs rotate over >= 1 GiB of resident copies, so no step finds its input
in the 256 MB last-level cache.  Every launch goes through the library's C
entry points with preallocated buffers, so the GPU, not the host, sets the
pace.  Every timed loop follows about 30 ms of the same calls, untimed: after
an idle spell the first milliseconds of heavy memory traffic run slower, and
the figures are meant to be a stream's steady state.

Reported on one JSON line:
  * value / ms_per_step: effective GB/s of the whole step over the
    algorithmic bytes (bf16 read + FP4 codes + E4M3 scales + 4 B tensor
    scale), timed over exactly --steps steps with HIP events;
  * the quantize kernel alone (amax given), over >= 250 launches: the mean
    of back-to-back launches (events around the whole run) and the median,
    p10 and p90 over batches of 25 back-to-back launches (per-launch
    durations of single kernels are in the rocprofv3 kernel-trace summary);
  * the roofline of that kernel: HBM (algorithmic bytes / mean launch time
    against 8 TB/s) and vector-ALU issue (SQ_ACTIVE_INST_VALU per launch
    from the committed rocprofv3 counter summary: one per wave64 VALU
    instruction, two for the 8-cycle conversions, against 1228.8 G per second:
    256 CUs x 4 SIMDs x 2.4 GHz / 2 cycles); `bound` names the
    larger fraction.  Traffic (FETCH_SIZE + WRITE_SIZE, calibrated) and the
    issue slots come from that summary only while the kernel sources it was
    taken on are unchanged, else null;
  * the same figures for the other workloads under "rows";
  * the CPU oracle on the host, single-threaded and on all cores of the
    host's share (rows split over worker processes, arithmetic unchanged),
    with the core count and CPU model.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--no-cpu] [--no-rows]
                    [--rows c3,f3,...]
    python bench.py --summarize OUT.md DIR [DIR...]   # rocprofv3 output -> summary
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
# wave64 VALU instructions per second: 256 CUs x 4 SIMDs, one wave64 fp32
# FMA per SIMD every 2 cycles at 2.4 GHz -- the rate behind the published
# 157.3 TFLOP/s fp32 vector peak (a non-packed v_fma_f32 measures 2.3-2.4
# cycles per wave64 instruction on gfx950; instructions with an SGPR operand,
# max3/med3, shifts and bit ops about 4.3, the fp4/fp8 conversions 8.4, so a
# real mix tops out well below this)
VALU_PEAK_GSLOTS = 256 * 4 * 2.4 / 2
MFMA_FP4_PEAK_TFLOPS = 10100.0                  # dense FP4 matrix peak of MI355X
MIN_LAUNCHES = 250                               # kernel-only figures: launches timed
# the kernel that does each workload's quantization (amax given)
KERNEL_OF = {"c1": "nvfp4_1d_kernel<false, false, false>",
             "c2": "nvfp4_1d_kernel<true, false, false>",
             "c3": "nvfp4_2d_kernel<true, true>",
             "c4": "nvfp4_1d_kernel<false, true, true>",
             "c5": "mxfp4_kernel<true, true, true>",
             "f1": "nvfp4_msed_kernel<true>",
             "f2": "nvfp4_rows_wg_kernel<true, false, false, 1, true>",
             "f3": "mxfp4_gemm_kernel",
             "f4a": "rq_quant_kernel<true, false, true>",
             "f4g": "rq_quant_kernel<false, true, true>"}
# the sources each workload's kernel is built from (a change to any of them
# makes that workload's committed counters stale)
SOURCES_OF = {"c1": ("device_common.h", "nvfp4_kernels.h"),
              "c2": ("device_common.h", "nvfp4_kernels.h"),
              "c3": ("device_common.h", "nvfp4_kernels.h", "nvfp4_2d_kernels.h"),
              "c4": ("device_common.h", "nvfp4_kernels.h"),
              "c5": ("device_common.h", "mx_kernels.h"),
              "f1": ("device_common.h", "nvfp4_kernels.h", "msed_kernels.h"),
              "f2": ("device_common.h", "nvfp4_kernels.h", "rows_kernels.h"),
              "f3": ("device_common.h", "mxgemm_kernels.h"),
              "f4a": ("device_common.h", "nvfp4_kernels.h", "requant_kernels.h"),
              "f4g": ("device_common.h", "nvfp4_kernels.h", "requant_kernels.h")}
METRIC = "NVFP4 4/6 quantize GB/s (bf16 in + fp4/scale out) and % of HBM peak"
COUNTERS_FILE = os.path.join(ROOT, "profiles", "counters_by_workload.json")

# workload -> (rows, cols, kind, flags, label)
ROWS = {
    "c1": (256, 1024, "nvfp4", 0, "nvfp4_rtn6_256x1024"),
    "c2": (8192, 4096, "nvfp4", 1, "nvfp4_four_over_six_8192x4096"),
    # not a bench row: c2's tensor and bytes with plain RTN6 (no 4/6
    # candidates, about half the vector work), the reference that shows
    # what the traffic alone costs
    "c2r": (8192, 4096, "nvfp4", 0, "nvfp4_rtn6_8192x4096_same_traffic"),
    "c3": (14336, 4096, "nvfp4", 1 | 8 | 64, "nvfp4_2d16x16_four_over_six_transposed_14336x4096"),
    "c4": (8192, 14336, "nvfp4", 2 | 4, "nvfp4_rht16_sr_8192x14336"),
    "c5": (16384, 8192, "mxfp4", 16 | 32 | 64, "mxfp4_had32_row_col_16384x8192"),
    # MS-EDEN on the gradient: RTN values, stochastic E4M3 scale
    "f1": (8192, 14336, "nvfp4", 4 | 128, "nvfp4_msed_rht16_8192x14336"),
    # one FP32 scale per row instead of per tensor: quantized in one read
    "f2": (8192, 4096, "rows", 1, "nvfp4_rowscale_four_over_six_8192x4096"),
    # the consumer: MXFP4 product of the 16384x8192 tensor's row-wise output
    # (M x K) with a second 8192x8192 tensor's (as B^T, N x K)
    "f3": (16384, 8192, "gemm", 16 | 32, "mxfp4_gemm_16384x8192x8192"),
    # requantization of a 1D NVFP4 tensor for the transposed operand; the
    # input is the activation (4/6) or the gradient (RHT16 + SR) quantized
    "f4a": (8192, 4096, "requant", 1 | 4, "nvfp4_requant_t_rht16_four_over_six_8192x4096"),
    "f4g": (8192, 14336, "requant", 2 | 4, "nvfp4_requant_t_rht16_sr_8192x14336"),
}
# workload -> the seeded tensor it quantizes, where that is another workload's
DATA_OF = {"f1": "c4", "f2": "c2", "f3": "c5", "c2r": "c2"}
GEMM_N = 8192                                   # f3: B^T rows (N); K = the tensor's cols
# requant workload -> (workload whose quantization is the input, its flags)
REQUANT_SRC = {"f4a": ("c2", 1), "f4g": ("c4", 2 | 4)}
SEED = 0x0123456789ABCDEF


def algorithmic_bytes(wl):
    rows, cols, kind, flags, _ = ROWS[wl]
    n = rows * cols
    if kind == "gemm":                               # A and B^T (codes + scales) in, fp32 C out
        return (rows * cols // 2 + rows * cols // 32) + (GEMM_N * cols // 2 + GEMM_N * cols // 32) \
            + 4 * rows * GEMM_N
    if kind == "requant":                            # NVFP4 in, NVFP4 of the transpose out
        return 2 * (n // 2 + n // 16 + 4)
    if kind == "rows":                               # one fp32 scale per row
        return 2 * n + n // 2 + n // 16 + 4 * rows
    if kind == "mxfp4":
        return 2 * n + 2 * (n // 2 + n // 32)
    if flags & 8:                                    # 16x16 tiles
        out = n // 2 + n // 256
        if flags & 64:
            out *= 2                                 # transposed codes and scales
        return 2 * n + out + 4
    return 2 * n + n // 2 + n // 16 + 4


def expected_items(wl):
    """Work-items of the workload's quantize launch where a profile can tell
    it apart from another row's by launch size only: the 1D RTN6 quantizer,
    which c1 shares with the same-traffic RTN6 reference row.  Follows the
    1D launch rule without SR: one 256-thread workgroup per 256 blocks, at
    most 6 per CU of the 256.  None for every other workload (its kernel
    instance is its own)."""
    rows, cols, kind, flags, _ = ROWS[wl]
    if kind != "nvfp4" or flags:
        return None
    nblocks = rows * cols // 16
    return min(-(-nblocks // 256), 256 * 6) * 256


def sources_sha(wl):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_reduce_amd", "csrc")
    for f in SOURCES_OF[wl]:
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def counters_of(wl):
    """Per-launch rocprofv3 figures of the workload's kernel from the
    committed summary, or None when missing or taken on other sources."""
    if not os.path.exists(COUNTERS_FILE):
        return None
    with open(COUNTERS_FILE) as f:
        p = json.load(f).get(wl)
    if not p or p.get("sources_sha") != sources_sha(wl):
        return None
    return p


def roofline(wl, us):
    """HBM and vector-ALU roofline of the workload's kernel at `us` per launch."""
    alg = algorithmic_bytes(wl)
    c = counters_of(wl) or {}
    hbm = {"achieved": round(alg / us / 1e3, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
           "frac": round(alg / us / 1e3 / HBM_PEAK_GBS, 4)}
    out = {"hbm": hbm, "traffic": c.get("hbm_bytes"),
           "traffic_source": "rocprofv3 FETCH_SIZE + WRITE_SIZE (calibrated), " + COUNTERS_FILE[len(ROOT) + 1:]
           if c.get("hbm_bytes") else None}
    slots = c.get("valu_issue_slots")
    if slots:
        ach = slots / us / 1e3                        # G slots per second
        out["valu"] = {"achieved": round(ach, 1), "peak": VALU_PEAK_GSLOTS,
                       "unit": "G wave64 VALU issues/s", "frac": round(ach / VALU_PEAK_GSLOTS, 4),
                       "issue_slots_per_launch": slots, "valu_insts_per_launch": c.get("valu_insts")}
        if c.get("clock_ghz"):                        # the same issue slots at the measured clock
            peak_at = 256 * 4 * c["clock_ghz"] / 2
            out["valu"].update(clock_ghz=c["clock_ghz"], peak_at_clock=round(peak_at, 1),
                               frac_at_clock=round(ach / peak_at, 4))
    if c.get("mfma_busy_frac") is not None:
        out["mfma_busy_frac"] = c["mfma_busy_frac"]
        out["clock_ghz"] = c.get("clock_ghz")
    return out


# ------------------------------------------------------------------ GPU side
class Row:
    """Preallocated buffers and raw C calls for one workload."""

    def __init__(self, wl, fp4, torch, synthetic, np):
        self.wl = wl
        rows, cols, kind, flags, label = ROWS[wl]
        self.rows, self.cols, self.kind, self.flags, self.label = rows, cols, kind, flags, label
        dev = torch.device("cuda:0")
        L = fp4.lib()
        self.L = L
        self.stream = torch.cuda.current_stream()
        self.sp = self.stream.cuda_stream
        u8 = torch.uint8
        if kind == "requant":
            self._init_requant(fp4, torch, synthetic, np, dev)
            return
        if kind == "gemm":
            self._init_gemm(fp4, torch, synthetic, np, dev)
            return
        x_np = synthetic.gen(DATA_OF.get(wl, wl))
        self.x_np = x_np
        x0 = torch.from_numpy(x_np.view(np.int16)).to(dev)
        nbytes = x0.numel() * 2
        self.nbuf = min(64, max(4, -(-(1 << 30) // nbytes)))   # >= 1 GiB of inputs (c1: 64 copies)
        self.xs = [x0] + [x0.clone() for _ in range(self.nbuf - 1)]
        self.outs = []
        if kind == "rows":
            for _ in range(self.nbuf):
                self.outs.append(dict(codes=torch.empty((rows, cols // 2), dtype=u8, device=dev),
                                      scales=torch.empty((rows, cols // 16), dtype=u8, device=dev),
                                      alpha=torch.empty(rows, dtype=torch.float32, device=dev)))
        elif kind == "nvfp4":
            two_d = bool(flags & 8)
            srows = rows // 16 if two_d else rows
            for _ in range(self.nbuf):
                o = dict(codes=torch.empty((rows, cols // 2), dtype=u8, device=dev),
                         scales=torch.empty((srows, cols // 16), dtype=u8, device=dev),
                         alpha=torch.empty(1, dtype=torch.float32, device=dev),
                         amax=torch.empty(1, dtype=torch.float32, device=dev))
                if flags & 64:
                    o["codes_t"] = torch.empty((cols, rows // 2), dtype=u8, device=dev)
                    o["scales_t"] = torch.empty((cols // 16, rows // 16), dtype=u8, device=dev)
                self.outs.append(o)
            self.ws = torch.empty(max(16, L.fp4_workspace_bytes(rows, cols, flags)), dtype=u8,
                                  device=dev)
            for k in range(self.nbuf):          # amax for the kernel-only timing
                rc = L.fp4_tensor_amax(self.xs[k].data_ptr(), rows, cols, flags, SEED,
                                       self.outs[k]["amax"].data_ptr(), self.ws.data_ptr(),
                                       self.ws.numel(), self.sp)
                assert rc == 0, rc
        else:
            for _ in range(self.nbuf):
                self.outs.append(dict(
                    codes_r=torch.empty((rows, cols // 2), dtype=u8, device=dev),
                    scales_r=torch.empty((rows, cols // 32), dtype=u8, device=dev),
                    codes_c=torch.empty((cols, rows // 2), dtype=u8, device=dev),
                    scales_c=torch.empty((cols, rows // 32), dtype=u8, device=dev)))
        # raw pointer tuples, prepared once
        self.args_step, self.args_kernel = [], []
        for k in range(self.nbuf):
            o, xp = self.outs[k], self.xs[k].data_ptr()
            if kind == "rows":              # a single kernel: step and kernel are one call
                a = (xp, rows, cols, flags, SEED, o["alpha"].data_ptr(), o["codes"].data_ptr(),
                     o["scales"].data_ptr(), None, self.sp)
                self.args_step.append(a)
                self.args_kernel.append(a)
            elif kind == "nvfp4":
                ct = o["codes_t"].data_ptr() if "codes_t" in o else None
                st = o["scales_t"].data_ptr() if "scales_t" in o else None
                common = (xp, rows, cols, flags, SEED)
                tail = (o["alpha"].data_ptr(), o["codes"].data_ptr(), o["scales"].data_ptr(),
                        None, ct, st)
                self.args_step.append(common + (None,) + tail +
                                      (self.ws.data_ptr(), self.ws.numel(), self.sp))
                self.args_kernel.append(common + (o["amax"].data_ptr(),) + tail +
                                        (None, 0, self.sp))
            else:
                a = (xp, rows, cols, flags, o["codes_r"].data_ptr(), o["scales_r"].data_ptr(),
                     o["codes_c"].data_ptr(), o["scales_c"].data_ptr(), self.sp)
                self.args_step.append(a)
                self.args_kernel.append(a)
        self.fn = {"nvfp4": L.nvfp4_quantize, "rows": L.nvfp4_quantize_rows,
                   "mxfp4": L.mxfp4_quantize}[kind]
        # one call per buffer set before any timing: the first write to a
        # freshly allocated output is slower (page mapping), and a short
        # warm-up touches only some of the sets
        for k in range(self.nbuf):
            self.step(k)
        torch.cuda.synchronize()

    def _init_gemm(self, fp4, torch, synthetic, np, dev):
        """A = row-wise MXFP4 of the tensor [rows][cols]; B^T = row-wise MXFP4
        of a second seeded tensor [GEMM_N][cols]; both made by the library."""
        rows, cols = self.rows, self.cols
        self.x_np = synthetic.gen(DATA_OF[self.wl])
        qa = fp4.mxfp4_quantize(torch.from_numpy(self.x_np.view(np.int16)).to(dev), self.flags)
        w = synthetic.gen(DATA_OF[self.wl], GEMM_N, cols, seed=4242)
        qb = fp4.mxfp4_quantize(torch.from_numpy(w.view(np.int16)).to(dev), self.flags)
        self.w_np = w
        self.nbuf = 1
        self.qa, self.qb = qa, qb
        self.c = torch.empty((rows, GEMM_N), dtype=torch.float32, device=dev)
        a = (qa["codes_r"].data_ptr(), qa["scales_r"].data_ptr(), qb["codes_r"].data_ptr(),
             qb["scales_r"].data_ptr(), rows, GEMM_N, cols, self.c.data_ptr(), self.sp)
        self.args_step, self.args_kernel = [a], [a]
        self.fn = self.L.mxfp4_gemm
        torch.cuda.synchronize()

    def _init_requant(self, fp4, torch, synthetic, np, dev):
        """Inputs: the source workload quantized by the library, copied to
        >= 1 GiB of resident buffers; outputs preallocated per copy."""
        rows, cols, flags = self.rows, self.cols, self.flags
        src, sflags = REQUANT_SRC[self.wl]
        self.x_np = synthetic.gen(src)
        q = fp4.nvfp4_quantize(torch.from_numpy(self.x_np.view(np.int16)).to(dev), sflags, seed=SEED)
        per = rows * cols // 2 + rows * cols // 16
        self.nbuf = min(64, max(4, -(-(1 << 30) // per)))
        u8, f32 = torch.uint8, torch.float32
        self.ins = [q] + [{k: v.clone() for k, v in q.items()} for _ in range(self.nbuf - 1)]
        self.outs = [dict(codes=torch.empty((cols, rows // 2), dtype=u8, device=dev),
                          scales=torch.empty((cols, rows // 16), dtype=u8, device=dev),
                          alpha=torch.empty(1, dtype=f32, device=dev),
                          amax=torch.empty(1, dtype=f32, device=dev)) for _ in range(self.nbuf)]
        L = self.L
        self.ws = torch.empty(max(16, L.fp4_workspace_bytes(rows, cols, flags)), dtype=u8, device=dev)
        self.args_step, self.args_kernel = [], []
        for k in range(self.nbuf):
            i, o = self.ins[k], self.outs[k]
            head = (i["codes"].data_ptr(), i["scales"].data_ptr(), i["alpha"].data_ptr(), rows, cols,
                    flags, SEED)
            tail = (o["alpha"].data_ptr(), o["codes"].data_ptr(), o["scales"].data_ptr(), None)
            self.args_step.append(head + (None,) + tail + (self.ws.data_ptr(), self.ws.numel(), self.sp))
            self.args_kernel.append(head + (o["amax"].data_ptr(),) + tail + (None, 0, self.sp))
        self.fn = L.nvfp4_requantize_t
        # the quantize pass alone runs with an amax given: the output's own
        # (recovered from its tensor scale; the work does not depend on it)
        C = 256.0 if flags & 1 else 448.0
        for k in range(self.nbuf):
            self.step(k)
            torch.mul(self.outs[k]["alpha"], 6.0 * C, out=self.outs[k]["amax"])
        torch.cuda.synchronize()

    def step(self, i):
        rc = self.fn(*self.args_step[i % self.nbuf])
        assert rc == 0, rc

    def kernel(self, i):
        rc = self.fn(*self.args_kernel[i % self.nbuf])
        assert rc == 0, rc


def head_start(torch, calls):
    """Keep the GPU busy for 0.5 ms (a spin kernel on the current stream)
    while the host starts enqueueing the timed launches: a ctypes call plus
    a launch costs the host about 4 us, longer than the shortest kernels
    (c1: 3 us) run.  The spin is kept short: after a longer one the chip's
    clock has dropped and the next kernels run slower for milliseconds
    (measured on the 4/6 kernel: 0.5 ms of spin 16.1 us per launch, 2 ms
    17.2 us, 8 ms 18.1 us).  It ends before the first timing event."""
    del calls
    torch.cuda._sleep(int(0.5e-3 * 2.4e9))


SETTLE_MS = 30.0


def settle(torch, stream, fn, ms=SETTLE_MS):
    """About `ms` of back-to-back calls of fn, untimed, before a timed loop.
    After the GPU has idled (a host-side phase, another workload's setup)
    the first milliseconds of heavy memory traffic run slower: on the 4/6
    kernel, 250 launches right after the full-step loop took 18.4 us each,
    and the three runs of 250 after them 16.1-16.7 us.  The timed figures
    are the steady state that a stream of such launches sees."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(3):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    per = max(e0.elapsed_time(e1) / 3, 1e-3)
    for i in range(int(min(20000, max(3, ms / per)))):
        fn(i)
    torch.cuda.synchronize()


def time_loop(torch, stream, fn, steps, warmup):
    """Mean ms per call of `steps` back-to-back calls (HIP events on the
    launch stream around the whole run, the calls queued behind a head
    start) and the host wall time; before them, the settling calls and
    `warmup` more, untimed."""
    settle(torch, stream, fn)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    head_start(torch, steps)
    e0.record(stream)
    for i in range(steps):
        fn(i)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return e0.elapsed_time(e1) / steps, wall


def launch_stats(torch, stream, fn, n, warmup, batch=25):
    """n calls: the mean of back-to-back calls (HIP events around the whole
    run; it includes the short dispatch gap between consecutive kernels,
    which rocprofv3's kernel duration excludes) and the median, p10 and p90
    over n / batch batches of `batch` back-to-back calls (an event pair per
    batch: each event costs about 5 us of pipeline drain, so batches of 25
    keep the median within 1 % of the back-to-back mean), as us per call."""
    mean_ms, _ = time_loop(torch, stream, fn, n, warmup)
    nb = max(1, n // batch)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    head_start(torch, n)
    ev[0].record(stream)
    for b in range(nb):
        for i in range(batch):
            fn(b * batch + i)
        ev[b + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[b].elapsed_time(ev[b + 1]) * 1e3 / batch for b in range(nb))
    q = lambda f: per[min(nb - 1, int(round(f * (nb - 1))))]
    return {"launches": n, "us_mean": round(mean_ms * 1e3, 3), "us_median": round(q(0.5), 3),
            "us_p10": round(q(0.1), 3), "us_p90": round(q(0.9), 3),
            "spread": "median/p10/p90 over %d batches of %d back-to-back calls" % (nb, batch)}


CAL_BYTES = 2 * 8192 * 4096          # one 64 MiB int16 tensor
CAL_KERNEL = "BitwiseOr"               # name fragment of the calibration kernel
AMAX_PASS = "amax_partial_kernel"      # the tensor-amax pass of a full step
AFTER_AMAX = " (after the amax pass)"


def copy_reference(torch, row):
    """Plain device copy of one input, from and to buffers that rotate over
    1.5 GiB (so neither side is still in the 256 MB last-level cache): the
    bandwidth a 1:1 read/write stream reaches on this machine.  Also runs, a few
    times, a 64 MiB elementwise bitwise-or (reads exactly CAL_BYTES, writes
    exactly CAL_BYTES) whose kernel name is unique in a profile: rocprofv3
    FETCH_SIZE / WRITE_SIZE of the quantizers are scaled by what the
    counters read for it."""
    srcs = row.xs
    dsts = [torch.empty_like(srcs[0]) for _ in range(8)]
    ms, _ = time_loop(torch, row.stream,
                      lambda i: dsts[i % len(dsts)].copy_(srcs[i % len(srcs)]), 24, 3)
    for _ in range(3):
        torch.bitwise_or(srcs[1], 0, out=dsts[0])
    torch.cuda.synchronize()
    gbs = 2 * srcs[0].numel() * 2 / (ms * 1e-3) / 1e9
    del dsts
    return gbs


# ------------------------------------------------------------------ CPU side
def cpu_info():
    """Host share used for the CPU baseline: at most the threads this
    process may run on, OMP_NUM_THREADS when set, and 16 (one GPU's share
    of a GPU host)."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    aff = len(os.sched_getaffinity(0))
    threads = aff
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        threads = min(threads, int(env))
    return {"nproc": os.cpu_count(), "affinity": aff, "threads": min(threads, 16), "model": model}


class CachedGen:
    """synthetic.gen with the arrays kept: the CPU baseline and the GPU
    rows quantize the same bytes without generating them twice."""

    def __init__(self, synthetic):
        self.s, self.cache = synthetic, {}

    def gen(self, *a, **k):
        key = (a, tuple(sorted(k.items())))
        if key not in self.cache:
            self.cache[key] = self.s.gen(*a, **k)
        return self.cache[key]

    def __getattr__(self, name):
        return getattr(self.s, name)


def cpu_oracle(wl, x_np, max_rows=None, budget_s=10.0, w_np=None):
    """The CPU oracle, as it stands (single-threaded C), on the workload or
    on its first max_rows rows; repeated until ~budget_s of work."""
    import numpy as np
    import oracle
    oracle.build()
    rows, cols, kind, flags, _ = ROWS[wl]
    x = x_np if max_rows is None else np.ascontiguousarray(x_np[:max_rows])
    times = []
    t_end = time.time() + budget_s
    while len(times) < 5 and (time.time() < t_end or len(times) < 1):
        if kind == "requant" and not times:                  # the input, made by the oracle
            q = oracle.nvfp4_quantize(x, REQUANT_SRC[wl][1], seed=SEED)
        if kind == "gemm" and not times:                     # operands, made by the oracle
            qa = oracle.mxfp4_quantize(x, flags)
            qb = oracle.mxfp4_quantize(np.ascontiguousarray(w_np[:GEMM_N]), flags)
        t0 = time.perf_counter()
        if kind == "nvfp4":
            oracle.nvfp4_quantize(x, flags, seed=SEED)
        elif kind == "rows":
            oracle.nvfp4_quantize_rows(x, flags, seed=SEED)
        elif kind == "requant":
            oracle.nvfp4_requantize_t(q["codes"], q["scales"], q["alpha"], x.shape[0], cols, flags,
                                      seed=SEED)
        elif kind == "gemm":                                 # BLAS held to one thread
            from threadpoolctl import threadpool_limits
            with threadpool_limits(limits=1):
                oracle.mxfp4_gemm(qa["codes_r"], qa["scales_r"], qb["codes_r"], qb["scales_r"],
                                  x.shape[0], GEMM_N, cols)
        else:
            oracle.mxfp4_quantize(x, flags)
        times.append(time.perf_counter() - t0)
    times.sort()
    med = times[len(times) // 2]
    frac = x.shape[0] / rows
    if kind == "gemm":
        tfl = 2.0 * x.shape[0] * GEMM_N * cols / med / 1e12
        return {"value": round(tfl, 5), "unit": "TFLOP/s", "cores": 1, "kind": "oracle",
                "sample": "first %d of %d rows of A (numpy float64 matmul after the C "
                          "dequantize), %d runs, median %.2f s" % (x.shape[0], rows, len(times), med)}
    gbs = algorithmic_bytes(wl) * frac / med / 1e9
    what = "full %dx%d workload" % (rows, cols) if max_rows is None else \
        "first %d of %d rows" % (x.shape[0], rows)
    return {"value": round(gbs, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": "%s, %d runs, median %.2f s" % (what, len(times), med)}


# worker-process state of the all-core oracle run (set before the fork)
_MC = {}


def _mc_amax(sl):
    import oracle
    return oracle.tensor_amax(_MC["x"][sl[0]:sl[1]], _MC["flags"], SEED)


def _mc_quant(args):
    import numpy as np
    import oracle
    (r0, r1), amax = args
    q = oracle.nvfp4_quantize(_MC["x"][r0:r1], _MC["flags"], seed=SEED, amax=amax)
    cols = _MC["x"].shape[1]
    codes = np.ndarray((_MC["rows"], cols // 2), np.uint8, buffer=_MC["shm_c"].buf)
    scales = np.ndarray((_MC["rows"], cols // 16), np.uint8, buffer=_MC["shm_s"].buf)
    codes[r0:r1] = q["codes"]
    scales[r0:r1] = q["scales"]
    return float(q["alpha"])


def cpu_oracle_all_cores(wl, x_np, threads, runs=3):
    """The oracle on all `threads` host cores for a 1D NVFP4 workload without
    SR (its SR counter is the element index in the whole tensor): rows split
    over worker processes, first the tensor amax of each slice (the max over
    slices is exact), then each slice quantized with that amax.  Results go
    to shared memory and must equal the single-process oracle bit for bit.
    Worker processes are forked before this process touches the GPU."""
    import multiprocessing as mp
    from multiprocessing import shared_memory

    import numpy as np
    import oracle
    oracle.build()
    rows, cols, kind, flags, _ = ROWS[wl]
    assert kind == "nvfp4" and not (flags & (2 | 8)), wl
    shm_c = shared_memory.SharedMemory(create=True, size=rows * cols // 2)
    shm_s = shared_memory.SharedMemory(create=True, size=rows * cols // 16)
    try:
        _MC.update(x=x_np, flags=flags, rows=rows, shm_c=shm_c, shm_s=shm_s)
        step = -(-rows // threads)
        slices = [(r, min(rows, r + step)) for r in range(0, rows, step)]
        times = []
        with mp.get_context("fork").Pool(threads) as pool:
            pool.map(_mc_amax, slices)                       # start-up, untimed
            for _ in range(runs):
                t0 = time.perf_counter()
                amax = max(pool.map(_mc_amax, slices))
                pool.map(_mc_quant, [(sl, amax) for sl in slices])
                times.append(time.perf_counter() - t0)
        want = oracle.nvfp4_quantize(x_np, flags, seed=SEED)
        codes = np.ndarray((rows, cols // 2), np.uint8, buffer=shm_c.buf)
        scales = np.ndarray((rows, cols // 16), np.uint8, buffer=shm_s.buf)
        same = bool(np.array_equal(codes, want["codes"]) and np.array_equal(scales, want["scales"]))
        del codes, scales
    finally:
        _MC.clear()
        shm_c.close()
        shm_c.unlink()
        shm_s.close()
        shm_s.unlink()
    assert same, "all-core oracle differs from the single-process oracle"
    med = sorted(times)[len(times) // 2]
    return {"value": round(algorithmic_bytes(wl) / med / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "full %dx%d workload, rows split over %d processes (amax of each slice, "
                      "then each slice quantized with the tensor amax; bit-identical to one "
                      "process), %d runs, median %.3f s" % (rows, cols, threads, runs, med)}


# ------------------------------------------------------------------ profile summaries
def summarize(out_path, dirs, command):
    """Summarize rocprofv3 output directories (kernel trace and/or --pmc
    counters) into a short markdown file, and merge the per-workload
    figures (calibrated HBM bytes, VALU instructions and issue slots, mean
    kernel time) into COUNTERS_FILE.  Traffic is scaled by what the same
    counter reads for the plain 64 MiB bitwise-or the benchmark runs (its
    true bytes are known)."""
    import glob
    import re
    import sqlite3
    import statistics

    def short(n):
        return re.sub(r"\(.*", "", n).replace("void fp4q::", "").replace("fp4q::", "")

    durations, counters = {}, {}
    for d in dirs:
        for db in glob.glob(os.path.join(d, "**", "*.db"), recursive=True):
            c = sqlite3.connect(db)
            tabs = {r[0] for r in c.execute("select name from sqlite_master")}
            if "kernels" in tabs:
                # a launch that directly follows an amax pass re-reads what that
                # pass just read (a full quantization step): listed apart
                prev = ""
                for n, dur, g in c.execute("select name, duration, grid_x * grid_y * grid_z "
                                           "from kernels order by start"):
                    k = short(n)
                    if prev.startswith(AMAX_PASS) and not k.startswith(AMAX_PASS):
                        k += AFTER_AMAX
                    durations.setdefault((k, g), []).append(dur / 1000.0)
                    prev = short(n)
            if "counters_collection" in tabs:
                for n, cn, v, g in c.execute(
                        "select kernel_name, counter_name, value, grid_size from counters_collection"):
                    counters.setdefault((short(n), cn, g), []).append(v)
    def wl_durations(wl, kern):                      # this workload's launches of its kernel
        grid = expected_items(wl)
        return [x for (k, g), v in durations.items() if k == kern and (grid is None or g == grid)
                for x in v]

    lines = ["# rocprofv3 summary", "", "Command:", "", "```", command, "```", ""]
    if durations:
        lines += ["| kernel | work-items | launches | avg us | median us | p10 us | p90 us | "
                  "min us | max us |", "|---|---|---|---|---|---|---|---|---|"]
        for (k, g), v in sorted(durations.items(), key=lambda kv: -sum(kv[1])):
            sv = sorted(v)
            pq = lambda f: sv[min(len(sv) - 1, int(round(f * (len(sv) - 1))))]
            lines.append("| %s | %d | %d | %.2f | %.2f | %.2f | %.2f | %.2f | %.2f |" % (
                k, g, len(v), sum(v) / len(v), statistics.median(v), pq(0.1), pq(0.9), min(v),
                max(v)))
        lines.append("")
    merged = {}
    if os.path.exists(COUNTERS_FILE):
        with open(COUNTERS_FILE) as f:
            merged = json.load(f)
    if counters:
        lines += ["| kernel | grid | counter | mean per dispatch |", "|---|---|---|---|"]
        for (k, cn, g), v in sorted(counters.items()):
            lines.append("| %s | %d | %s | %.1f |" % (k, g, cn, sum(v) / len(v)))
        cal = {}
        for cn in ("FETCH_SIZE", "WRITE_SIZE"):
            vs = [x for (k, c2, g), v in counters.items() if c2 == cn and CAL_KERNEL in k for x in v]
            if vs:
                cal[cn] = CAL_BYTES / (sum(vs) / len(vs) * 1024.0)
        if cal:
            lines += ["", "Calibration (64 MiB int16 bitwise-or: %d B read, %d B written): "
                      "FETCH_SIZE x %.3f, WRITE_SIZE x %.3f" % (
                          CAL_BYTES, CAL_BYTES, cal.get("FETCH_SIZE", 0), cal.get("WRITE_SIZE", 0))]
        lines += ["", "| workload | kernel | fetched B | written B | total / algorithmic | "
                  "VALU insts | VALU issue slots |", "|---|---|---|---|---|---|---|"]
        for wl, kern in KERNEL_OF.items():
            q = {}
            grid = expected_items(wl)
            for (k, cn, g), v in counters.items():
                if k.startswith(kern) and (grid is None or g == grid):
                    q.setdefault(cn, []).extend(v)
            q = {cn: sum(v) / len(v) for cn, v in q.items()}
            if not q:
                continue
            e = merged.get(wl, {})
            if e.get("sources_sha") != sources_sha(wl):
                e = {}
            e.update(kernel=kern, sources_sha=sources_sha(wl), command=command)
            raw = e.setdefault("raw", {})
            raw.update({cn: round(v, 1) for cn, v in q.items()})
            if "FETCH_SIZE" in q and "FETCH_SIZE" in cal:
                e["fetch_bytes"] = round(q["FETCH_SIZE"] * 1024 * cal["FETCH_SIZE"])
            if "WRITE_SIZE" in q and "WRITE_SIZE" in cal:
                e["write_bytes"] = round(q["WRITE_SIZE"] * 1024 * cal["WRITE_SIZE"])
            if "fetch_bytes" in e and "write_bytes" in e:
                e["hbm_bytes"] = e["fetch_bytes"] + e["write_bytes"]
            if "SQ_INSTS_VALU" in q:
                e["valu_insts"] = round(q["SQ_INSTS_VALU"])
            if "SQ_ACTIVE_INST_VALU" in q:            # wave64 VALU issues (8-cycle ones count 2)
                e["valu_issue_slots"] = round(q["SQ_ACTIVE_INST_VALU"])
            dur = wl_durations(wl, kern)
            if dur:
                e["avg_us_trace"] = round(sum(dur) / len(dur), 3)
            # shader clock over the kernel: GRBM_GUI_ACTIVE counts busy cycles
            # on each of the 8 XCDs over the profiled dispatch, which adds a
            # few us of launch and drain to the kernel's duration, so the
            # figure is kept for kernels of 150 us and more only (there the
            # excess is under 2 %)
            if "GRBM_GUI_ACTIVE" in q and dur:
                us = statistics.median(dur)
                if us >= 150.0:
                    e["clock_ghz"] = round(q["GRBM_GUI_ACTIVE"] / 8 / (us * 1e3), 3)
            # matrix-core busy cycles (summed over SIMDs) over the CU busy
            # cycles of 4 SIMDs each
            if "SQ_VALU_MFMA_BUSY_CYCLES" in q and q.get("SQ_BUSY_CU_CYCLES"):
                e["mfma_busy_frac"] = round(q["SQ_VALU_MFMA_BUSY_CYCLES"] /
                                            (4 * q["SQ_BUSY_CU_CYCLES"]), 4)
            merged[wl] = e
            alg = algorithmic_bytes(wl)
            lines.append("| %s | %s | %s | %s | %s | %s | %s |" % (
                ROWS[wl][4], kern, e.get("fetch_bytes", "-"), e.get("write_bytes", "-"),
                "%.3f" % (e["hbm_bytes"] / alg) if "hbm_bytes" in e else "-",
                e.get("valu_insts", "-"), e.get("valu_issue_slots", "-")))
    elif durations:
        for wl, kern in KERNEL_OF.items():
            dur = wl_durations(wl, kern)
            if dur and wl in merged and merged[wl].get("sources_sha") == sources_sha(wl):
                merged[wl]["avg_us_trace"] = round(sum(dur) / len(dur), 3)
    with open(out_path, "w") as f:
        f.write("\n".join(lines) + "\n")
    if merged:
        with open(COUNTERS_FILE, "w") as f:
            json.dump(merged, f, indent=1, sort_keys=True)
    print("\n".join(lines))


# ------------------------------------------------------------------ main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle timings")
    ap.add_argument("--no-rows", action="store_true", help="headline workload only")
    ap.add_argument("--rows", default="", help="comma-separated subset of the other workloads "
                    "(for profiling runs)")
    ap.add_argument("--launches", type=int, default=MIN_LAUNCHES,
                    help="launches per kernel-only figure (default %d; fewer only for "
                         "profiler runs)" % MIN_LAUNCHES)
    ap.add_argument("--summarize", nargs="+", metavar=("OUT", "DIR"),
                    help="summarize rocprofv3 output directories into OUT")
    ap.add_argument("--command", default="", help="command recorded in a --summarize output")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize[0], args.summarize[1:], args.command)
        return
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this quantizer has no multi-GPU path "
              "(sharding needs one all-reduce(max) of the amax)", file=sys.stderr)
        sys.exit(2)

    import numpy as np

    import synthetic as synthetic_mod
    synthetic = CachedGen(synthetic_mod)
    row_wls = () if args.no_rows else ("c1", "c3", "c4", "c5", "f1", "f2", "f3", "f4a", "f4g")
    if args.rows:
        row_wls = tuple(w for w in args.rows.split(",") if w in row_wls)

    # CPU oracle first, before this process touches the GPU (its all-core
    # run forks worker processes)
    cpu = {}
    if not args.no_cpu:
        info = cpu_info()
        x2 = synthetic.gen("c2")
        single = cpu_oracle("c2", x2, budget_s=4.0)
        cpu["baseline"] = dict(cpu_oracle_all_cores("c2", x2, info["threads"]),
                               single_core=single, host=info)
        for wl in row_wls:
            _, _, kind, _, _ = ROWS[wl]
            x = synthetic.gen(DATA_OF.get(wl, wl)) if kind != "requant" else \
                synthetic.gen(REQUANT_SRC[wl][0])
            w = synthetic.gen(DATA_OF[wl], GEMM_N, ROWS[wl][1], seed=4242) if kind == "gemm" else None
            cpu[wl] = cpu_oracle(wl, x, max_rows=32 if kind == "gemm" else
                                 (None if wl == "c1" else 512), budget_s=3.0, w_np=w)
        print("cpu oracle done", flush=True)

    import torch

    import block_scaled_fp4_reduce_amd as fp4

    torch.cuda.set_device(0)
    head = Row("c2", fp4, torch, synthetic, np)
    ms_step, wall = time_loop(torch, head.stream, head.step, args.steps, args.warmup)
    kst = launch_stats(torch, head.stream, head.kernel, args.launches, args.warmup)
    sst = launch_stats(torch, head.stream, head.step, args.launches, args.warmup)
    copy_gbs = copy_reference(torch, head)
    ref = Row("c2r", fp4, torch, synthetic, np)
    rst = launch_stats(torch, ref.stream, ref.kernel, args.launches, args.warmup)
    del ref
    torch.cuda.empty_cache()
    alg = algorithmic_bytes("c2")
    value = alg / (ms_step * 1e-3) / 1e9
    rl = roofline("c2", kst["us_mean"])
    fracs = {"hbm": rl["hbm"]["frac"]}
    if "valu" in rl:
        fracs["alu"] = rl["valu"]["frac"]
    bound = max(fracs, key=fracs.get)
    main_roof = rl["hbm"] if bound == "hbm" else rl["valu"]
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": head.label + "_bf16", "rows": 8192, "cols": 4096,
                   "input_dtype": "bf16", "compute_dtype": "f32",
                   "values": "Student-t(4) x per-column lognormal(0,1), bf16",
                   "flags": "FOUR_OVER_SIX", "amax": "computed in-step",
                   "global_batch": 1, "parallelism": "none"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "step": dict(sst, gbs_mean=round(alg / sst["us_mean"] / 1e3, 1)),
        "quantize_kernel": dict(kst, gbs_mean=round(alg / kst["us_mean"] / 1e3, 1),
                                gbs_median=round(alg / kst["us_median"] / 1e3, 1),
                                note="amax given: one kernel per call"),
        "target_70pct_of_hbm": {"A_quantize_kernel_mean": rl["hbm"]["frac"] >= 0.7,
                                "B_full_step": value / HBM_PEAK_GBS >= 0.7},
        "copy_kernel_gbs": round(copy_gbs, 1),
        "same_traffic_rtn6_kernel": dict(rst, note="the same tensor and bytes quantized with plain "
                                         "RTN6: no 4/6 candidates, about half the vector work"),
        "roofline": {"bound": "alu" if bound == "alu" else "hbm",
                     "achieved": main_roof["achieved"], "peak": main_roof["peak"],
                     "unit": main_roof["unit"], "frac": main_roof["frac"],
                     "traffic": rl["traffic"], "traffic_source": rl["traffic_source"],
                     "hbm": rl["hbm"], "valu": rl.get("valu"),
                     "kernel": KERNEL_OF["c2"], "algorithmic_bytes": alg},
        "wall_s": round(wall, 4),
    }
    if row_wls:
        rows = []
        for wl in row_wls:
            r = Row(wl, fp4, torch, synthetic, np)
            st, _ = time_loop(torch, r.stream, r.step, max(10, args.steps // 2), 3)
            ks = launch_stats(torch, r.stream, r.kernel, args.launches, 3)
            if r.kind == "gemm":
                fl = 2.0 * r.rows * GEMM_N * r.cols
                tf = fl / ks["us_mean"] / 1e6
                rw = roofline(wl, ks["us_mean"])
                entry = {"workload": r.label, "flops": fl, "kernel": ks,
                         "tflops": round(tf, 1), "kernel_frac_mfma_fp4": round(tf / MFMA_FP4_PEAK_TFLOPS, 4),
                         "bound": "mfma", "hbm": rw["hbm"], "traffic": rw["traffic"],
                         "mfma_busy_frac": rw.get("mfma_busy_frac"), "clock_ghz": rw.get("clock_ghz")}
                if rw.get("clock_ghz"):               # the FP4 peak at the measured clock
                    entry["kernel_frac_mfma_fp4_at_clock"] = round(
                        tf / (MFMA_FP4_PEAK_TFLOPS * rw["clock_ghz"] / 2.4), 4)
            else:
                a = algorithmic_bytes(wl)
                rw = roofline(wl, ks["us_mean"])
                fr = {"hbm": rw["hbm"]["frac"]}
                if "valu" in rw:
                    fr["alu"] = rw["valu"]["frac"]
                entry = {"workload": r.label, "algorithmic_bytes": a,
                         "step_us": round(st * 1e3, 3), "step_gbs": round(a / (st * 1e-3) / 1e9, 1),
                         "kernel": ks, "kernel_gbs": round(a / ks["us_mean"] / 1e3, 1),
                         "kernel_frac_hbm": rw["hbm"]["frac"], "bound": max(fr, key=fr.get),
                         "valu": rw.get("valu"), "traffic": rw["traffic"]}
            if wl in cpu:
                entry["cpu_oracle"] = cpu[wl]
            rows.append(entry)
            del r
            torch.cuda.empty_cache()
        line["rows"] = rows
    if cpu:
        line["cpu_baseline"] = cpu["baseline"]
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
