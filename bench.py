#!/usr/bin/env python3
"""Throughput of NVFP4 Four-Over-Six quantization of an 8192x4096 bf16
activation tensor on one MI355X.

A step is one full pass of the path over one input: the tensor amax pass
(Eq. 1) and the block quantizer (Eq. 2-3 with the 4/6 choice), i.e. one
``nvfp4_quantize`` call with amax computed inside.  Inputs rotate over
enough resident copies (> 1 GiB together) that no step finds its input in
the 256 MB last-level cache.

Reported: effective GB/s over the algorithmic bytes (bf16 read + FP4 codes
+ E4M3 scales + 4 B tensor scale written), its fraction of the 8 TB/s HBM
peak, the quantize kernel alone (amax given) timed live with HIP events on
its stream, optional rocprofv3 traffic for that kernel, and the CPU oracle
timed on the host as a baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10]
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
ROWS, COLS = 8192, 4096
WORKLOAD = "nvfp4_four_over_six_8192x4096_bf16"
METRIC = "NVFP4 4/6 quantize GB/s (bf16 in + fp4/scale out) and % of HBM peak"


def algorithmic_bytes(rows, cols):
    n = rows * cols
    return 2 * n + n // 2 + n // 16 + 4


def kernel_source_sha():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "block_scaled_fp4_reduce_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def traffic_from_profile(per_launch_alg):
    """HBM bytes per launch of the quantize kernel from the committed
    rocprofv3 counter summary, or None when it is missing or stale."""
    path = os.path.join(ROOT, "profiles", "nvfp4_4o6_8192x4096_counters.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        p = json.load(f)
    if p.get("kernel_source_sha") != kernel_source_sha():
        return None
    return p.get("hbm_bytes_per_launch")


def cpu_baseline(x_np):
    """The CPU oracle, as it stands, on the same workload (full tensor,
    repeated until ~10 s of work); single-threaded."""
    import oracle
    oracle.build()
    times = []
    t_end = time.time() + 10.0
    while time.time() < t_end or len(times) < 2:
        t0 = time.perf_counter()
        oracle.nvfp4_quantize(x_np, oracle.FOUR_OVER_SIX)
        times.append(time.perf_counter() - t0)
        if len(times) >= 5:
            break
    times.sort()
    med = times[len(times) // 2]
    return {"value": round(algorithmic_bytes(*x_np.shape) / med / 1e9, 4), "unit": "GB/s",
            "cores": 1, "kind": "oracle",
            "sample": "full 8192x4096 workload, %d runs, median %.2f s" % (len(times), med)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this quantizer has no multi-GPU path "
              "(sharding needs one all-reduce(max) of the amax; see DESIGN.md)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import block_scaled_fp4_reduce_amd as fp4
    import synthetic

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    x_np = synthetic.gen("c2")
    x0 = torch.from_numpy(x_np.view(np.int16)).to(dev)
    in_bytes = x0.numel() * 2
    nbuf = max(4, -(-(1 << 30) // in_bytes))            # >= 1 GiB of rotating inputs
    xs = [x0] + [x0.clone() for _ in range(nbuf - 1)]
    flags = fp4.FOUR_OVER_SIX
    outs = [fp4.nvfp4_quantize(x, flags) for x in xs]   # allocates every output once
    ws = torch.empty(fp4.fp4_workspace_bytes(ROWS, COLS, flags), dtype=torch.uint8, device=dev)
    amaxes = [fp4.fp4_tensor_amax(x, flags, ws=ws) for x in xs]
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(i):
        k = i % nbuf
        fp4.nvfp4_quantize(xs[k], flags, ws=ws, out=outs[k], stream=stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for i in range(args.steps):
        step(i)
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = ev0.elapsed_time(ev1) / args.steps

    # dominant kernel alone: quantize with amax given (one kernel per call),
    # HIP events on the launch stream around every launch
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    for i in range(args.warmup):
        k = i % nbuf
        fp4.nvfp4_quantize(xs[k], flags, amax=amaxes[k], out=outs[k], stream=stream)
    torch.cuda.synchronize()
    for i in range(args.steps):
        k = i % nbuf
        evs[i][0].record(stream)
        fp4.nvfp4_quantize(xs[k], flags, amax=amaxes[k], out=outs[k], stream=stream)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    kms = sorted(a.elapsed_time(b) for a, b in evs)
    kernel_ms = sum(kms) / len(kms)

    # plain copy of the same size: the achievable bandwidth on this machine
    src, dst = xs[1], torch.empty_like(xs[1])
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(20):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * in_bytes * 20 / (c0.elapsed_time(c1) * 1e-3) / 1e9

    alg = algorithmic_bytes(ROWS, COLS)
    value = alg / (ms_step * 1e-3) / 1e9
    kernel_gbs = alg / (kernel_ms * 1e-3) / 1e9
    traffic = traffic_from_profile(alg)
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
        "config": {"workload": WORKLOAD, "rows": ROWS, "cols": COLS,
                   "values": "Student-t(4) x per-column lognormal(0,1), bf16",
                   "flags": "FOUR_OVER_SIX", "amax": "computed in-step",
                   "global_batch": 1, "parallelism": "none"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "quantize_kernel": {"ms_avg": round(kernel_ms, 5), "ms_p10": round(kms[len(kms) // 10], 5),
                            "ms_p90": round(kms[(9 * len(kms)) // 10], 5),
                            "gbs": round(kernel_gbs, 2)},
        "copy_kernel_gbs": round(copy_gbs, 1),
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
        "wall_s": round(wall, 4),
    }
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(x_np)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
