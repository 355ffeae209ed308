"""Benchmark of one split-KV paged-attention decode step on one MI355X.

A step is one pa_decode + pa_reduce call over a whole batch of synthetic
input already resident in HBM.  The default workload is the dense MTP4
verify batch with FP8 KV caches and per-token scales (32 sequences, Hq 16 /
Hkv 1, head dim 128, 4 causal query rows, page 128, lengths uniform in
[16384, 32768]).  Reported:

* value: achieved KV bandwidth (GB/s, decimal) of the algorithmic KV bytes —
  K and V (+ per-token K/V scales) of every (sequence, KV head)'s visible-token
  union, counted once per call — over the cold per-call time: one event pair
  brackets K calls that rotate over three copies of the KV caches, so no call
  finds its KV in the 256 MB Infinity Cache;
* roofline: the decode kernel's algorithmic bytes over its own average
  duration, timed the same way with the decode launches alone, against 8 TB/s;
* cpu_baseline: the CPU oracle on a bounded sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from paged_attention_decode_plan_amd import binding as B  # noqa: E402
from paged_attention_decode_plan_amd import workloads as W  # noqa: E402
from paged_attention_decode_plan_amd.build import source_sha  # noqa: E402

PEAK_GBPS = 8000.0  # MI355X HBM3E, AMD's published figure
WORKLOADS = {
    "dense_mtp4_fp8": "dense MTP4 verify, FP8 KV, per-token scales: B32 Hq16/Hkv1 D128 QL4 page128 L~U[16K,32K]",
    "dense_mtp4_bf16": "dense MTP4 verify, BF16 KV: B32 Hq16/Hkv1 D128 QL4 page128 L~U[16K,32K]",
    "dense_mtp2_fp8": "supplementary: the dense MTP4 FP8 batch with QL2 (32 rows per KV head), same caches and tables",
    "long_mtp4_c200k": "supplementary: the pages' MI355X shape: B200 QL4 Hq16/Hkv1 D128 page128, every context "
                       "200000, FP8 per-token, plain V; 5 partitions per sequence (the pages' best NP)",
    "long_d256": "long-context D256: B4 Hkv2 GQA8 QL4 page64 L=131072 window 8193, transposed V, per-tensor",
    "long_d256_nowindow": "supplementary: the long-context D256 batch with the window off (all 131072 tokens visible)",
    "ragged": "ragged batch: B128 Hkv4 GQA4 D128 QL1 page16 log-uniform L, window 257, sinks, per-token",
    "sparse": "sparse decode: 64 rows Hq16/Hkv1 D128 page16, 2048 of 65536 slots, per-token, 4 partitions",
    "tiny": "tiny decode: B2 Hq8/Hkv1 D128 QL1 page16 L=37,100, per-tensor, one partition",
}


# The pages' own MI355X figure for a workload, where they give one: the
# achieved KV bandwidth of aiter PR #4332 for B200 / MTP4 / C=200k at five
# partitions per sequence (KV and scales counted once per call).
PAGES_GBPS = {"long_mtp4_c200k": 5163.9}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def load_traffic(workload: str, launches_kv_bytes: float):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_traffic.json"))):
        with open(path) as f:
            t = json.load(f)
        if t.get("kernel_sha") == source_sha():
            return t.get("hbm_bytes_per_launch")
    return None


def load_mfma(workload: str):
    """MFMA busy fraction of the decode kernel from a committed rocprofv3
    counter run, if it was taken on the current kernel source."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_mfma.json"))):
        with open(path) as f:
            t = json.load(f)
        if t.get("kernel_sha") == source_sha():
            return round(t.get("mfma_busy_fraction"), 4)
    return None


def make_inputs(workload: str):
    if workload == "sparse":
        return W.config_sparse(), dict(partition_tokens=512)
    if workload == "tiny":
        return W.config_tiny(), dict(max_partitions=1)
    if workload == "long_d256":
        return W.config_long_d256(), {}
    if workload == "long_d256_nowindow":
        return W.config_long_d256(window=0), {}
    if workload == "ragged":
        return W.config_ragged(), {}
    if workload == "dense_mtp4_bf16":
        return W.config_dense_mtp4("bf16"), {}
    if workload == "dense_mtp2_fp8":
        return W.config_dense_mtp4("fp8", query_len=2), {}
    if workload == "long_mtp4_c200k":  # drawn on the device: 10.56 GB of KV
        return W.config_long_mtp4_device(torch.device("cuda:0")), dict(partition_tokens=40064)
    return W.config_dense_mtp4("fp8"), {}


def cpu_baseline(inp, budget_s: float = 12.0):
    """Oracle on whole sequences of the workload until ~budget_s of wall time;
    reported as KV GB/s of the sequences it completed."""
    from oracle import oracle as O

    p = inp.problem
    lens = inp.context_lens.numpy()
    order = np.argsort(lens)  # shortest first, so the sample completes quickly
    elem = 1 if p.kv_dtype == "fp8" else 2
    per_tok = 2 * p.head_dim * elem + (8 if (p.kv_dtype == "fp8" and p.scale_mode == "token") else 0)
    done_bytes, done_seqs, t_used, threads = 0, 0, 0.0, 1
    for s in order.tolist():
        sel = [(s * p.query_len + i, h) for i in range(p.query_len) for h in range(p.num_q_heads)]
        t0 = time.perf_counter()
        _, threads = O.attend(inp, sel=sel, return_threads=True)
        t_used += time.perf_counter() - t0
        L = int(min(max(lens[s], 0), p.table_stride if p.token_table else p.table_stride * p.page_size))
        if p.token_table:
            n = L
        else:
            lo, hi = W.visible_span(L, p.query_len, p.sliding_window, p.causal)
            n = hi - lo
        done_bytes += n * p.num_kv_heads * per_tok
        done_seqs += 1
        if t_used >= budget_s:
            break
    gbps = done_bytes / t_used / 1e9 if t_used > 0 else 0.0
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"all {p.query_len * p.num_q_heads} (row, head) outputs of the {done_seqs} shortest "
                      f"sequences of the workload ({done_bytes / 1e6:.1f} MB of KV) in {t_used:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense_mtp4_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="run one device-to-device copy of MIB MiB first (counter calibration)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: this decode engine runs on a single MI355X; "
              "--gpus above 1 is not supported", file=sys.stderr)
        sys.exit(1)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    t_gen = time.perf_counter()
    inp, plan_kw = make_inputs(args.workload)
    log(f"inputs {args.workload} built in {time.perf_counter() - t_gen:.1f}s")
    p = inp.problem
    d = {k: (None if v is None else v.to(dev).contiguous()) for k, v in dict(
        q=inp.q, k=inp.k_cache, v=inp.v_cache, bt=inp.block_tables, cl=inp.context_lens, ks=inp.k_scale,
        vs=inp.v_scale, sk=inp.sinks).items()}
    plan = B.Plan(B.problem_of(p), inp.context_lens, **plan_kw).allocate(dev)
    info = plan.info()
    out = torch.empty_like(d["q"])
    stream = torch.cuda.current_stream()
    kv_bytes = W.kv_bytes_visible(inp)

    def step():
        B.pa_decode(plan, out, d["q"], d["k"], d["v"], d["bt"], d["cl"], d["ks"], d["vs"], d["sk"], stream)
        B.pa_reduce(plan, out, d["sk"], stream)

    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: {n} bytes read, {n} bytes written")

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all(), "non-finite output"

    # Timing: one pair of HIP events around a region of K launches on the
    # launch stream, divided by K (events around every launch would add their
    # own dispatch overhead to each call).  Warm: K calls on one copy of the
    # inputs.  Cold: the calls rotate over three copies of the KV caches and
    # scales at different addresses (3x the KV bytes, well past the 256 MB
    # Infinity Cache), so each call reads KV that the two calls before it
    # have evicted.
    K = args.steps
    copies = [(d["k"], d["v"], d["ks"], d["vs"])]
    for _ in range(2):
        copies.append(tuple(None if t is None else t.clone() for t in copies[0]))

    def call(c, reduce=True):
        kc, vc, ksc, vsc = copies[c]
        B.pa_decode(plan, out, d["q"], kc, vc, d["bt"], d["cl"], ksc, vsc, d["sk"], stream)
        if reduce:
            B.pa_reduce(plan, out, d["sk"], stream)

    def region(body):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(K):
            body(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    t_start = time.perf_counter()
    us_warm = region(lambda k: call(0))
    for k in range(3):
        call(k)  # first touch of every copy
    us_cold = region(lambda k: call(k % 3))
    dec_us = region(lambda k: call(k % 3, reduce=False))
    timed_wall = time.perf_counter() - t_start
    del copies
    achieved = kv_bytes / (dec_us * 1e-6) / 1e9
    traffic = load_traffic(args.workload, kv_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic}
    on_device = inp.k_cache.is_cuda  # too large for the host oracle's timing loop
    cpu = None if (args.no_cpu or on_device) else cpu_baseline(inp, args.cpu_budget)
    gbps = kv_bytes / (us_cold * 1e-6) / 1e9
    res = {
        "metric": "achieved HBM GB/s of KV bytes (and us/call), FP8 paged decode",
        "value": round(gbps, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(us_cold / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": round(gbps / PAGES_GBPS[args.workload], 4) if args.workload in PAGES_GBPS else None,
        "dtype": "f16" if p.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": WORKLOADS[args.workload],
                   "kv_bytes_per_call": kv_bytes, "work_items": info.num_items, "partials": info.num_slots,
                   "cu_count": info.cu_count},
        "us_per_call_cold": round(us_cold, 2),
        "us_per_call_warm": round(us_warm, 2),
        "decode_us_cold": round(dec_us, 2),
        "warm_gbps": round(kv_bytes / (us_warm * 1e-6) / 1e9, 1),
        "frac_of_peak_cold": round(gbps / PEAK_GBPS, 4),
        "wall_s_timed_regions": round(timed_wall, 3),
        "roofline": roofline,
        "mfma_busy_fraction": load_mfma(args.workload),
        "cpu_baseline": cpu,
        "kernel_sha": source_sha(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
