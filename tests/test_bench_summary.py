"""The profile summarizer of bench.py on a synthetic rocprofv3 database (CPU).

Two bench rows launch the same 1D quantizer instance: the 256x1024 RTN6
workload and the same-traffic RTN6 reference on 8192x4096.  The summary must
give each workload its own launch's durations and counters (told apart by
the launch's work-items), keep the quantize launches of full steps (those
right after an amax pass, which re-read what it read) out of the kernel's
own figure, and scale the traffic counters by the calibration kernel's
reading."""
import json
import sqlite3

import bench

RTN6 = "void fp4q::nvfp4_1d_kernel<false, false, false>(uint4 const*, long)"
F46 = "void fp4q::nvfp4_1d_kernel<true, false, false>(uint4 const*, long)"
CAL = "void at::native::BitwiseOrFunctor<short>(int)"
AMAX = "void fp4q::amax_partial_kernel<false>(uint4 const*, long)"


def _db(path):
    c = sqlite3.connect(path)
    c.execute("create table kernels (name text, duration integer, grid_x integer, "
              "grid_y integer, grid_z integer, start integer)")
    c.execute("create table counters_collection (kernel_name text, counter_name text, "
              "value real, grid_size integer)")
    small, big, f46 = bench.expected_items("c1"), 393216, 393216
    launches = []
    for _ in range(3):
        launches += [(RTN6, 3000, small), (RTN6, 16000, big), (F46, 17000, f46)]
    launches += [(AMAX, 10000, 262144), (F46, 14000, f46)]       # a full step: warm re-read
    for t, (n, dur, g) in enumerate(launches):
        c.execute("insert into kernels values (?, ?, ?, 1, 1, ?)", (n, dur, g, 100000 * t))
    rows = [(RTN6, "FETCH_SIZE", 512.0, small), (RTN6, "WRITE_SIZE", 160.0, small),
            (RTN6, "SQ_ACTIVE_INST_VALU", 1000.0, small),
            (RTN6, "FETCH_SIZE", 32768.0, big), (RTN6, "WRITE_SIZE", 9000.0, big),
            (RTN6, "SQ_ACTIVE_INST_VALU", 3.0e6, big),
            (F46, "FETCH_SIZE", 32768.0, f46), (F46, "SQ_ACTIVE_INST_VALU", 6.0e6, f46),
            (CAL, "FETCH_SIZE", bench.CAL_BYTES / 1024.0 / 2.0, 1 << 20),
            (CAL, "WRITE_SIZE", bench.CAL_BYTES / 1024.0, 1 << 20)]
    c.executemany("insert into counters_collection values (?, ?, ?, ?)", rows)
    c.commit()
    c.close()


def test_expected_items_follow_the_1d_launch_rule():
    assert bench.expected_items("c1") == 64 * 256          # 16384 blocks: 64 workgroups
    assert bench.expected_items("c2") is None              # 4/6: its own kernel instance
    assert bench.expected_items("c4") is None
    assert bench.expected_items("c3") is None


def test_shared_kernel_split_by_launch_size(tmp_path, monkeypatch):
    d = tmp_path / "prof"
    d.mkdir()
    _db(str(d / "run_results.db"))
    counters = tmp_path / "counters.json"
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(counters))
    out = tmp_path / "summary.md"
    bench.summarize(str(out), [str(d)], "synthetic")
    merged = json.loads(counters.read_text())
    c1, c2 = merged["c1"], merged["c2"]
    assert c1["avg_us_trace"] == 3.0                       # not the 16 us reference launches
    assert c1["valu_issue_slots"] == 1000
    assert c1["fetch_bytes"] == 512 * 1024 * 2             # FETCH_SIZE calibrated x2
    assert c1["write_bytes"] == 160 * 1024
    assert c2["avg_us_trace"] == 17.0 and c2["valu_issue_slots"] == 6000000
    text = out.read_text()
    assert "| nvfp4_1d_kernel<false, false, false> | 16384 | 3 |" in text
    assert "| nvfp4_1d_kernel<false, false, false> | 393216 | 3 |" in text
    assert "| nvfp4_1d_kernel<true, false, false> (after the amax pass) | 393216 | 1 | 14.00 |" in text
