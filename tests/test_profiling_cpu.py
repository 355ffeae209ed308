"""The rocprofv3 summary tool (paged_attention_decode_plan_amd.profiling) on
small synthetic CSVs whose answers are worked out by hand: the kernel-trace
table and the mean over the last dispatches of the focus kernel, the
copy-calibrated HBM traffic, the MFMA busy fraction and the per-CU counter
rates.  These are the numbers the committed summaries and the bench line's
traffic figure are made of.  Also: bench.py's refusal of more than one GPU."""

from __future__ import annotations

import csv
import json

import pytest

from paged_attention_decode_plan_amd import profiling as PR

TRACE_FIELDS = ["Kernel_Name", "Start_Timestamp", "End_Timestamp"]
COUNTER_FIELDS = ["Kernel_Name", "Counter_Name", "Counter_Value"]


def _write(path, fields, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=fields)
        w.writeheader()
        for r in rows:
            w.writerow(dict(zip(fields, r)))
    return str(path)


def test_trace_stats_last_dispatches(tmp_path):
    # decode dispatches of 10, 20, 30, 40 us (listed out of start order) and
    # two reducer dispatches of 5 us; timestamps in ns
    rows = [("void pa::pa_stream_kernel<128>(A)", 3000, 33000), ("void pa::pa_stream_kernel<128>(A)", 0, 10000),
            ("void pa::pa_stream_kernel<128>(A)", 5000, 45000), ("void pa::pa_stream_kernel<128>(A)", 1000, 21000),
            ("void pa::pa_reduce_kernel<128>(R)", 11000, 16000), ("void pa::pa_reduce_kernel<128>(R)", 50000, 55000)]
    trace = _write(tmp_path / "t.csv", TRACE_FIELDS, rows)
    table, focus = PR.kernel_trace_stats(trace, "pa_stream_kernel", 2)
    by = {k: (n, mean, mn, mx) for _, k, n, mean, mn, mx in table}
    assert by["void pa::pa_stream_kernel<128>(A)"] == (4, 25.0, 10.0, 40.0)
    assert by["void pa::pa_reduce_kernel<128>(R)"] == (2, 5.0, 5.0, 5.0)
    # the last two by start time are the dispatches started at 3000 and 5000
    assert focus[1] == 2 and focus[2] == pytest.approx(35.0)
    out = tmp_path / "s.txt"
    PR.main(["stats", "--trace", trace, "--focus", "pa_stream_kernel", "--last", "2", "--out", str(out)])
    assert out.read_text().rstrip().endswith("35.00 us")


def test_traffic_copy_calibration(tmp_path):
    # the copy of 1 MiB reads 2048 KiB and writes 4096 KiB by the counters'
    # own units: factors 0.5 and 0.25; the kernel's 1000 / 100 KiB per
    # dispatch are then 512000 and 25600 bytes
    rows = [("pa_stream_kernel", "FETCH_SIZE", 900.0), ("pa_stream_kernel", "FETCH_SIZE", 1100.0),
            ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 2048.0), ("__amd_rocclr_copyBuffer", "FETCH_SIZE", 8.0)]
    fetch = _write(tmp_path / "f.csv", COUNTER_FIELDS, rows)
    rows = [("pa_stream_kernel", "WRITE_SIZE", 100.0), ("__amd_rocclr_copyBuffer", "WRITE_SIZE", 4096.0)]
    write = _write(tmp_path / "w.csv", COUNTER_FIELDS, rows)
    out = tmp_path / "t.json"
    PR.main(["traffic", "--fetch", fetch, "--write", write, "--kernel", "pa_stream_kernel", "--copy-bytes",
             str(1 << 20), "--algorithmic-bytes", "512000", "--out", str(out)])
    r = json.loads(out.read_text())
    assert r["counters"]["FETCH_SIZE"]["scale"] == pytest.approx(0.5)
    assert r["counters"]["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(512000.0)
    assert r["counters"]["WRITE_SIZE"]["bytes_per_launch"] == pytest.approx(25600.0)
    assert r["hbm_bytes_per_launch"] == pytest.approx(537600.0)
    assert r["traffic_over_algorithmic"] == pytest.approx(1.05)


def test_mfma_busy_fraction(tmp_path):
    # 8 XCDs report 8000 GPU-active cycles in all (1000 per dispatch); 1024
    # SIMDs busy 256000 cycles in all: a quarter of the SIMD-cycles
    rows = [("pa_stream_kernel", "GRBM_GUI_ACTIVE", 8000.0), ("pa_stream_kernel", "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0),
            ("other_kernel", "GRBM_GUI_ACTIVE", 1.0)]
    path = _write(tmp_path / "m.csv", COUNTER_FIELDS, rows)
    out = tmp_path / "m.json"
    PR.main(["mfma", "--csv", path, "--kernel", "pa_stream_kernel", "--out", str(out)])
    r = json.loads(out.read_text())
    assert r["active_cycles"] == pytest.approx(1000.0)
    assert r["mfma_busy_fraction"] == pytest.approx(0.25)


def test_counters_per_cu_and_cycle(tmp_path):
    # two passes; the second holds GRBM_GUI_ACTIVE (8 XCDs x 500 cycles)
    p1 = _write(tmp_path / "g1.csv", COUNTER_FIELDS,
                [("pa_stream_kernel", "TCC_HIT_sum", 2560.0), ("pa_stream_kernel", "TCC_HIT_sum", 7680.0)])
    p2 = _write(tmp_path / "g2.csv", COUNTER_FIELDS,
                [("pa_stream_kernel", "TA_TA_BUSY_sum", 64000.0), ("pa_stream_kernel", "GRBM_GUI_ACTIVE", 4000.0)])
    out = tmp_path / "c.json"
    PR.main(["counters", "--csv", p1, p2, "--kernel", "pa_stream_kernel", "--out", str(out)])
    r = json.loads(out.read_text())
    assert r["counters_per_dispatch"]["TCC_HIT_sum"] == pytest.approx(5120.0)
    assert r["per_cu"]["TCC_HIT_sum"] == pytest.approx(20.0)
    assert r["active_cycles"] == pytest.approx(500.0)
    # 64000 busy cycles over 256 CUs and 500 active cycles: half the time
    assert r["per_cu_per_active_cycle"]["TA_TA_BUSY_sum"] == pytest.approx(0.5)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 ends with a message before
    any device work."""
    import os
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 1
    assert "one GPU" in r.stderr and r.stdout == ""
