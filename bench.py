"""Benchmark of one split-KV paged-attention decode step on one MI355X.

A step is one pa_decode + pa_reduce call over a whole batch of synthetic
input already resident in HBM.  The default workload is the dense MTP4
verify batch with FP8 KV caches and per-token scales (32 sequences, Hq 16 /
Hkv 1, head dim 128, 4 causal query rows, page 128, lengths uniform in
[16384, 32768]).  Reported:

* value: achieved KV bandwidth (GB/s, decimal) of the algorithmic KV bytes —
  K and V (+ per-token K/V scales) of every (sequence, KV head)'s visible-token
  union, counted once per call — over the cold per-call time (a 2.5 GiB read
  flush precedes every timed call so the Infinity Cache cannot serve KV);
* roofline: the decode kernel's algorithmic bytes over its own average
  duration (HIP events around that launch on its stream), against 8 TB/s;
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
    "long_d256": "long-context D256: B4 Hkv2 GQA8 QL4 page64 L=131072 window 8193, transposed V, per-tensor",
    "ragged": "ragged batch: B128 Hkv4 GQA4 D128 QL1 page16 log-uniform L, window 257, sinks, per-token",
    "sparse": "sparse decode: 64 rows Hq16/Hkv1 D128 page16, 2048 of 65536 slots, per-token, 4 partitions",
    "tiny": "tiny decode: B2 Hq8/Hkv1 D128 QL1 page16 L=37,100, per-tensor, one partition",
}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def load_traffic(workload: str, launches_kv_bytes: float):
    """HBM bytes per decode launch from committed rocprofv3 counter runs, if
    they were taken on the current kernel source."""
    path = os.path.join(ROOT, "profiles", f"pa_decode_kernel_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_sha") != source_sha():
        return None
    return t.get("hbm_bytes_per_launch")


def make_inputs(workload: str):
    if workload == "sparse":
        return W.config_sparse(), dict(partition_tokens=512)
    if workload == "tiny":
        return W.config_tiny(), dict(max_partitions=1)
    if workload == "long_d256":
        return W.config_long_d256(), {}
    if workload == "ragged":
        return W.config_ragged(), {}
    if workload == "dense_mtp4_bf16":
        return W.config_dense_mtp4("bf16"), {}
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

    # warm: back-to-back calls, events around each call
    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(K)]
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        ev[k][0].record(stream)
        step()
        ev[k][1].record(stream)
    torch.cuda.synchronize()
    warm_wall = time.perf_counter() - t_start
    warm_call = np.array([ev[k][0].elapsed_time(ev[k][1]) * 1e3 for k in range(K)])

    # cold: a 2.5 GiB read flush before every timed call; the calls are timed
    # with events around the whole call only, the decode launch alone in a
    # second pass (an event between the two launches would add its own gap)
    flush = torch.empty(int(2.5 * 2**30) // 4, dtype=torch.float32, device=dev).fill_(1.0)
    evc = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    sink = torch.zeros((), device=dev)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    for k in range(K):
        sink += flush.sum()
        evc[k][0].record(stream)
        step()
        evc[k][1].record(stream)
    for k in range(K):
        sink += flush.sum()
        evc[k][2].record(stream)
        B.pa_decode(plan, out, d["q"], d["k"], d["v"], d["bt"], d["cl"], d["ks"], d["vs"], d["sk"], stream)
        evc[k][3].record(stream)
        B.pa_reduce(plan, out, d["sk"], stream)
    torch.cuda.synchronize()
    cold_wall = time.perf_counter() - t_start
    cold_call = np.array([evc[k][0].elapsed_time(evc[k][1]) * 1e3 for k in range(K)])
    cold_dec = np.array([evc[k][2].elapsed_time(evc[k][3]) * 1e3 for k in range(K)])
    del flush

    us_cold = float(np.mean(cold_call))
    us_warm = float(np.mean(warm_call))
    dec_us = float(np.mean(cold_dec))
    achieved = kv_bytes / (dec_us * 1e-6) / 1e9
    traffic = load_traffic(args.workload, kv_bytes)
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": traffic}
    cpu = None if args.no_cpu else cpu_baseline(inp, args.cpu_budget)
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
        "vs_baseline": None,
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
        "wall_s_timed_regions": round(warm_wall + cold_wall, 3),
        "roofline": roofline,
        "cpu_baseline": cpu,
        "kernel_sha": source_sha(),
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
