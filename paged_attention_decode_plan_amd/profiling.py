"""Summaries of rocprofv3 output for the decode library.

  stats    kernel-trace CSV -> short text table (calls, mean / min / max
           duration per kernel, and the mean over the last N dispatches of a
           chosen kernel, i.e. the timed launches of a bench run)
  traffic  FETCH_SIZE / WRITE_SIZE counter CSVs -> HBM bytes per launch of a
           kernel, each counter scaled by what it reads for a device-to-device
           copy of known size run in the same process
  mfma     one counter CSV with SQ_VALU_MFMA_BUSY_CYCLES, GRBM_GUI_ACTIVE and
           instruction counts -> MFMA busy fraction of the kernel (busy cycles
           summed over SIMDs / (GPU-active cycles x SIMDs), GRBM_GUI_ACTIVE
           being summed over the XCDs) and MFMA / VALU instructions per launch
  counters any counter CSVs (one per rocprofv3 pass) -> per-dispatch means of
           a kernel's counters, per CU, and per CU and GPU-active cycle where
           a pass also holds GRBM_GUI_ACTIVE

The counters report KiB per dispatch; the copy calibration turns them into
bytes whatever request granularity the counter assumes.
"""

from __future__ import annotations

import argparse
import csv
import json
import re
import statistics
import sys

from .build import source_sha


def _rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _short(name: str, width: int = 72) -> str:
    name = re.sub(r"\s+", " ", name)
    return name if len(name) <= width else name[: width - 3] + "..."


def kernel_trace_stats(trace_csv: str, focus: str, last: int):
    rows = _rows(trace_csv)
    by = {}
    for r in rows:
        d = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3
        by.setdefault(r["Kernel_Name"], []).append((int(r["Start_Timestamp"]), d))
    table = []
    for k, v in by.items():
        ds = [d for _, d in v]
        table.append((sum(ds), k, len(ds), statistics.mean(ds), min(ds), max(ds)))
    table.sort(reverse=True)
    focus_last = None
    for k, v in by.items():
        if re.search(focus, k):
            v = sorted(v)
            tail = [d for _, d in v[-last:]] if last > 0 else [d for _, d in v]
            focus_last = (k, len(tail), statistics.mean(tail))
            break
    return table, focus_last


def cmd_stats(a):
    table, focus_last = kernel_trace_stats(a.trace, a.focus, a.last)
    total = sum(t[0] for t in table) or 1.0
    out = [f"# rocprofv3 kernel trace summary: {a.title}", "",
           f"command: {a.command}", f"summary: python -m paged_attention_decode_plan_amd.profiling stats "
           f"--trace <kernel_trace.csv> --focus '{a.focus}' --last {a.last}",
           f"library source sha: {source_sha()}", "",
           f"{'kernel':<74} {'calls':>6} {'mean us':>9} {'min us':>9} {'max us':>9} {'% time':>7}"]
    for tot, k, n, mean, mn, mx in table:
        out.append(f"{_short(k):<74} {n:>6} {mean:>9.2f} {mn:>9.2f} {mx:>9.2f} {100 * tot / total:>7.2f}")
    if focus_last:
        k, n, mean = focus_last
        out += ["", f"mean of the last {n} dispatches of {_short(k, 60)}: {mean:.2f} us"]
    text = "\n".join(out) + "\n"
    if a.out:
        with open(a.out, "w") as f:
            f.write(text)
    sys.stdout.write(text)


def _counter_means(path, counter):
    vals = {}
    for r in _rows(path):
        if r["Counter_Name"] != counter:
            continue
        vals.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return vals


def cmd_traffic(a):
    res = {"kernel": a.kernel, "workload": a.workload, "kernel_sha": source_sha(),
           "copy_bytes": a.copy_bytes, "command_fetch": a.command_fetch, "command_write": a.command_write}
    per = {}
    for counter, path in (("FETCH_SIZE", a.fetch), ("WRITE_SIZE", a.write)):
        vals = _counter_means(path, counter)
        kern = [v for k, vs in vals.items() if re.search(a.kernel, k) for v in vs]
        # the calibration copy is the largest copy-kernel dispatch of the run
        copy = [v for k, vs in vals.items() if re.search(a.copy_kernel, k) for v in vs]
        if not kern or not copy:
            raise SystemExit(f"{counter}: no dispatches of {a.kernel!r} or {a.copy_kernel!r} in {path}")
        copy_kib = max(copy)
        factor = a.copy_bytes / (copy_kib * 1024.0)
        kib = statistics.mean(kern)
        per[counter] = dict(kib_per_dispatch=kib, dispatches=len(kern), copy_kib=copy_kib, scale=factor,
                            bytes_per_launch=kib * 1024.0 * factor)
    res["counters"] = per
    res["hbm_bytes_per_launch"] = per["FETCH_SIZE"]["bytes_per_launch"] + per["WRITE_SIZE"]["bytes_per_launch"]
    if a.algorithmic_bytes:
        res["algorithmic_bytes_per_launch"] = a.algorithmic_bytes
        res["traffic_over_algorithmic"] = res["hbm_bytes_per_launch"] / a.algorithmic_bytes
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def cmd_mfma(a):
    rows = [r for r in _rows(a.csv) if re.search(a.kernel, r["Kernel_Name"])]
    if not rows:
        raise SystemExit(f"no dispatches of {a.kernel!r} in {a.csv}")
    per = {}
    for r in rows:
        per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
    means = {k: statistics.mean(v) for k, v in per.items()}
    simds = a.cu_count * 4
    res = {"kernel": a.kernel, "workload": a.workload, "kernel_sha": source_sha(), "command": a.command,
           "dispatches": len(per.get("GRBM_GUI_ACTIVE", [])), "counters_per_dispatch": means, "simds": simds,
           "xcds": a.xcds}
    if "SQ_VALU_MFMA_BUSY_CYCLES" in means and "GRBM_GUI_ACTIVE" in means:
        active = means["GRBM_GUI_ACTIVE"] / a.xcds  # GPU-active cycles of the dispatch
        res["active_cycles"] = active
        res["mfma_busy_fraction"] = means["SQ_VALU_MFMA_BUSY_CYCLES"] / (active * simds)
    if a.expected_mfma:
        res["expected_mfma_per_launch"] = a.expected_mfma
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def cmd_counters(a):
    means, active = {}, None
    for path in a.csv:
        rows = [r for r in _rows(path) if re.search(a.kernel, r["Kernel_Name"])]
        if not rows:
            raise SystemExit(f"no dispatches of {a.kernel!r} in {path}")
        per = {}
        for r in rows:
            per.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
        for k, v in per.items():
            means[k] = statistics.mean(v[-a.last:] if a.last > 0 else v)
    if "GRBM_GUI_ACTIVE" in means:
        active = means["GRBM_GUI_ACTIVE"] / a.xcds
    res = {"kernel": a.kernel, "workload": a.workload, "kernel_sha": source_sha(), "commands": a.command,
           "counters_per_dispatch": means,
           "per_cu": {k: v / a.cu_count for k, v in means.items() if k != "GRBM_GUI_ACTIVE"}}
    if active:
        res["active_cycles"] = active
        res["per_cu_per_active_cycle"] = {k: v / a.cu_count / active for k, v in means.items()
                                          if k != "GRBM_GUI_ACTIVE"}
    if a.note:
        res["note"] = a.note
    text = json.dumps(res, indent=1)
    if a.out:
        with open(a.out, "w") as f:
            f.write(text + "\n")
    print(text)


def main(argv=None):
    ap = argparse.ArgumentParser(prog="python -m paged_attention_decode_plan_amd.profiling")
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--trace", required=True, help="rocprofv3 *_kernel_trace.csv")
    s.add_argument("--focus", default="pa_stream_kernel|pa_decode_kernel")
    s.add_argument("--last", type=int, default=0, help="mean over the last N dispatches of the focus kernel")
    s.add_argument("--title", default="")
    s.add_argument("--command", default="")
    s.add_argument("--out")
    s.set_defaults(fn=cmd_stats)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True, help="counter_collection.csv of the FETCH_SIZE run")
    t.add_argument("--write", required=True, help="counter_collection.csv of the WRITE_SIZE run")
    t.add_argument("--kernel", default="pa_stream_kernel|pa_decode_kernel")
    t.add_argument("--copy-kernel", default="copyBuffer")
    t.add_argument("--copy-bytes", type=float, required=True)
    t.add_argument("--algorithmic-bytes", type=float, default=0.0)
    t.add_argument("--workload", default="")
    t.add_argument("--command-fetch", default="")
    t.add_argument("--command-write", default="")
    t.add_argument("--out")
    t.set_defaults(fn=cmd_traffic)
    m = sub.add_parser("mfma")
    m.add_argument("--csv", required=True, help="counter_collection.csv of the MFMA counter run")
    m.add_argument("--kernel", default="pa_stream_kernel|pa_decode_kernel")
    m.add_argument("--cu-count", type=int, default=256)
    m.add_argument("--xcds", type=int, default=8, help="XCDs whose GRBM_GUI_ACTIVE the counter sums")
    m.add_argument("--expected-mfma", type=float, default=0.0, help="MFMA instructions per launch by the algorithm")
    m.add_argument("--workload", default="")
    m.add_argument("--command", default="")
    m.add_argument("--out")
    m.set_defaults(fn=cmd_mfma)
    c = sub.add_parser("counters")
    c.add_argument("--csv", required=True, nargs="+", help="counter_collection.csv of each counter pass")
    c.add_argument("--kernel", default="pa_stream_kernel|pa_decode_kernel")
    c.add_argument("--last", type=int, default=0, help="mean over the last N dispatches of each pass")
    c.add_argument("--cu-count", type=int, default=256)
    c.add_argument("--xcds", type=int, default=8)
    c.add_argument("--workload", default="")
    c.add_argument("--command", nargs="*", default=[])
    c.add_argument("--note", default="")
    c.add_argument("--out")
    c.set_defaults(fn=cmd_counters)
    a = ap.parse_args(argv)
    a.fn(a)


if __name__ == "__main__":
    main()
