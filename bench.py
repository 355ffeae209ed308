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
* cpu_baseline: the CPU oracle on a bounded sample of the same workload;
* workloads: the same measurement (cold and warm us per call, KV GB/s, the
  decode launch's roofline fraction where the shape is HBM-bound) for every
  other configuration: the tiny, sparse, long-context D256 (with and without
  its window), ragged and dense BF16 batches, the MTP2 shape and the pages'
  own MI355X shape (B200, MTP4, 200 000-token contexts).  --only skips them.
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
SETTLE_MS = 100.0  # untimed calls before the warm-up steps, so that the GPU clocks have settled
MERGE = {"reducer": B.MERGE_REDUCER, "in-kernel": B.MERGE_IN_KERNEL}
merge_mode = B.MERGE_AUTO  # --merge
settle_ms_target = SETTLE_MS  # --settle-ms
WORKLOADS = {
    "dense_mtp4_fp8": "dense MTP4 verify, FP8 KV, per-token scales: B32 Hq16/Hkv1 D128 QL4 page128 L~U[16K,32K]",
    "dense_mtp4_bf16": "dense MTP4 verify, BF16 KV: B32 Hq16/Hkv1 D128 QL4 page128 L~U[16K,32K]",
    "dense_mtp2_fp8": "supplementary: the dense MTP4 FP8 batch with QL2 (32 rows per KV head), same caches and tables",
    "dense_mtp4_mxfp4": "supplementary: the dense MTP4 batch with MXFP4 KV (E2M1 codes, an E8M0 scale per 32 dims), "
                        "256-token partitions",
    "long_mtp4_c200k": "supplementary: the pages' MI355X shape: B200 QL4 Hq16/Hkv1 D128 page128, every context "
                       "200000, FP8 per-token, plain V; 5 partitions per sequence (the pages' best NP)",
    "long_d256": "long-context D256: B4 Hkv2 GQA8 QL4 page64 L=131072 window 8193, transposed V, per-tensor",
    "long_d256_nowindow": "supplementary: the long-context D256 batch with the window off (all 131072 tokens visible)",
    "ragged": "ragged batch: B128 Hkv4 GQA4 D128 QL1 page16 log-uniform L, window 257, sinks, per-token",
    "sparse": "sparse decode: 64 rows Hq16/Hkv1 D128 page16, 2048 of 65536 slots, per-token, 4 partitions",
    "sparse_topk": "the sparse decode batch with two-level indices: 2048 top-k logical positions per row resolved "
                   "through a 4096-page block table in the kernel, 4 partitions",
    "tiny": "tiny decode: B2 Hq8/Hkv1 D128 QL1 page16 L=37,100, per-tensor, one partition",
}
# Measured after the headline line by default, into its "workloads" object.
EXTRA_WORKLOADS = ["tiny", "sparse", "sparse_topk", "long_d256", "long_d256_nowindow", "ragged", "dense_mtp4_bf16",
                   "dense_mtp2_fp8", "dense_mtp4_mxfp4", "long_mtp4_c200k"]
# Shapes whose time is HBM streaming of the KV bytes (a roofline claim); the
# tiny and ragged batches are latency-bound and the sparse batches gather
# from a pool that stays in the 256 MB Infinity Cache: for those the
# bandwidth figure is an effective rate, not a roofline fraction.
ROOFLINE_CLAIM = {"dense_mtp4_fp8", "dense_mtp4_bf16", "dense_mtp2_fp8", "dense_mtp4_mxfp4", "long_d256",
                  "long_d256_nowindow", "long_mtp4_c200k"}


# The pages' own MI355X figure for a workload, where they give one: the
# achieved KV bandwidth of aiter PR #4332 for B200 / MTP4 / C=200k at five
# partitions per sequence (KV and scales counted once per call).  Context
# only: another machine's run, never a baseline of this one.
PAGES_GBPS = {"long_mtp4_c200k": 5163.9}


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _profile_json(workload: str, kind: str):
    """A committed rocprofv3 summary for the workload, if it was taken on the
    current kernel source."""
    import glob

    for path in sorted(glob.glob(os.path.join(ROOT, "profiles", f"*_{workload}_{kind}.json"))):
        with open(path) as f:
            t = json.load(f)
        if t.get("kernel_sha") == source_sha():
            return t
    return None


def load_traffic(workload: str):
    """HBM bytes per decode launch from committed rocprofv3 counter runs."""
    t = _profile_json(workload, "traffic")
    return None if t is None else t.get("hbm_bytes_per_launch")


def load_mfma(workload: str):
    """MFMA busy fraction of the decode kernel from a committed counter run."""
    t = _profile_json(workload, "mfma")
    return None if t is None else round(t.get("mfma_busy_fraction"), 4)


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def make_inputs(workload: str):
    if workload == "sparse":
        return W.config_sparse(), dict(partition_tokens=512)
    if workload == "sparse_topk":
        return W.config_sparse_topk(), dict(partition_tokens=512)
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
    if workload == "dense_mtp4_mxfp4":
        return W.config_dense_mtp4("mxfp4"), {}
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
        cap = {0: p.table_stride * p.page_size, 1: p.table_stride, 2: p.index_stride}[p.token_table]
        L = int(min(max(lens[s], 0), cap))
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
    return {"value": round(gbps, 4), "unit": "GB/s", "cores": threads, "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"all {p.query_len * p.num_q_heads} (row, head) outputs of the {done_seqs} shortest "
                      f"sequences of the workload ({done_bytes / 1e6:.1f} MB of KV) in {t_used:.1f} s"}


def kernel_of(p, info) -> str:
    """Which decode kernel the library launches for a plan (its dispatch rule)."""
    if p.token_table or info.rows_per_group <= 16:
        return "pa_decode_kernel"
    if p.kv_dtype == "bf16" and p.head_dim == 128 and p.page_size >= 32:
        return "pa_stream_kernel"
    if p.kv_dtype == "fp8" and (p.head_dim == 128 or (p.head_dim == 256 and info.rows_per_group <= 32)):
        return "pa_stream_kernel"
    return "pa_decode_kernel"


def measure(workload: str, steps: int, warmup: int, dev):
    """Time pa_decode + pa_reduce calls of one workload with its inputs
    resident in HBM.  Timing: one pair of HIP events on the launch stream
    around a region of K calls, divided by K (events around every launch
    would add their own dispatch overhead to each call).  Warm: K calls on
    one copy of the inputs.  Cold: the calls rotate over three copies of the
    KV caches and scales at different addresses (3x the KV bytes, past the
    256 MB Infinity Cache), so each call reads KV that the two calls before it
    have evicted; a workload whose KV alone is far larger than that cache
    (drawn on the device) uses one copy.  Decode: the cold region with the
    decode launches alone."""
    t_gen = time.perf_counter()
    inp, plan_kw = make_inputs(workload)
    log(f"inputs {workload} built in {time.perf_counter() - t_gen:.1f}s")
    p = inp.problem
    d = {k: (None if v is None else v.to(dev).contiguous()) for k, v in dict(
        q=inp.q, k=inp.k_cache, v=inp.v_cache, bt=inp.block_tables, cl=inp.context_lens, ks=inp.k_scale,
        vs=inp.v_scale, sk=inp.sinks, tk=inp.topk_indices).items()}
    plan = B.Plan(B.problem_of(p), inp.context_lens, merge=merge_mode, **plan_kw).allocate(dev)
    info = plan.info()
    out = torch.empty_like(d["q"])
    stream = torch.cuda.current_stream()
    kv_bytes = W.kv_bytes_visible(inp)
    on_device = inp.k_cache.is_cuda
    copies = [(d["k"], d["v"], d["ks"], d["vs"])]
    if not on_device:
        for _ in range(2):
            copies.append(tuple(None if t is None else t.clone() for t in copies[0]))
    nc = len(copies)

    def call(c, reduce=True):
        kc, vc, ksc, vsc = copies[c]
        if p.token_table == 2:
            B.pa_decode_sparse(plan, out, d["q"], kc, vc, d["bt"], d["tk"], d["cl"], ksc, vsc, d["sk"], stream)
        else:
            B.pa_decode(plan, out, d["q"], kc, vc, d["bt"], d["cl"], ksc, vsc, d["sk"], stream)
        if reduce:
            B.pa_reduce(plan, out, d["sk"], stream)

    def region(body):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(steps):
            body(k)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / steps

    # Clock settle: untimed calls for about SETTLE_MS of GPU time before the
    # warm-up steps.  A GPU that was idle runs its first few hundred calls at
    # lower clocks (20-call decode regions of the dense MTP4 batch measured
    # back to back in a fresh process: 102, 54, 59, 61, 59, 57, 56, 55, 54,
    # 53, 52.5, 52, 51.8, 51.4 us).
    settle_ms = 0.0
    while settle_ms < settle_ms_target:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for k in range(20):
            call(k % nc)
        e1.record(stream)
        torch.cuda.synchronize()
        settle_ms += e0.elapsed_time(e1)
    for k in range(max(warmup, nc)):
        call(k % nc)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    us_warm = region(lambda k: call(0))
    us_cold = region(lambda k: call(k % nc))
    dec_us = region(lambda k: call(k % nc, reduce=False))
    timed_wall = time.perf_counter() - t_start
    # Checked after the timed regions: the first torch kernels of a process
    # load their code objects, and the GPU idling meanwhile lowers its clocks
    # for the next milliseconds (a check placed before the regions cost the
    # dense MTP4 batch 3-5 us per call in the first measurement of a process).
    call(0)
    assert torch.isfinite(out.float()).all(), f"{workload}: non-finite output"
    res = {
        "description": WORKLOADS[workload],
        "kernel": kernel_of(p, info),
        "kv_bytes_per_call": kv_bytes,
        "us_per_call_cold": round(us_cold, 2),
        "us_per_call_warm": round(us_warm, 2),
        "decode_us_cold": round(dec_us, 2),
        "gbps_cold": round(kv_bytes / (us_cold * 1e-6) / 1e9, 1),
        "gbps_warm": round(kv_bytes / (us_warm * 1e-6) / 1e9, 1),
        "decode_gbps_cold": round(kv_bytes / (dec_us * 1e-6) / 1e9, 1),
        "roofline_claim": workload in ROOFLINE_CLAIM,
        "work_items": info.num_items,
        "partials": info.num_slots,
        # how multi-partition units are merged: the reducer launch, the
        # last-arriving work item, or nothing to merge (every unit wrote its
        # rows directly)
        "merge": ("none (direct output)" if info.max_parts < 2 else
                  "in-kernel last arriver" if merge_mode == B.MERGE_IN_KERNEL else "reducer launch"),
        "cu_count": info.cu_count,
        "cold_copies": nc,
        "clock_settle_ms": round(settle_ms, 1),
        "wall_s_timed_regions": round(timed_wall, 3),
    }
    if workload in ROOFLINE_CLAIM:
        res["decode_frac"] = round(kv_bytes / (dec_us * 1e-6) / 1e9 / PEAK_GBPS, 4)
        res["traffic"] = load_traffic(workload)
        res["mfma_busy_fraction"] = load_mfma(workload)
    if workload in PAGES_GBPS:
        res["pages_gbps_context"] = {"value": PAGES_GBPS[workload],
                                     "note": "the pages' own MI355X figure for this shape (aiter PR #4332); "
                                             "another machine's run, context only"}
    del copies, d, plan, out
    torch.cuda.empty_cache()
    return res, inp


# The sparse front end's indexer (pa_mqa_logits, then pa_topk), measured
# into the same "workloads" object; bound by the FP8 matrix cores.
PEAK_FP8_TFLOPS = 5000.0  # MI355X dense FP8 MFMA, AMD's published figure
INDEXER_WORKLOADS = {
    "indexer_decode": "indexer of the sparse decode batch: 64 rows x 65536 FP8 index keys, 64 heads of dim 128, "
                      "full windows, then the top 2048 of every row",
    "mqa_logits_4095x36863": "supplementary: FP8 MQA logits alone at the pages' MI355X timing shape, 4095 rows x "
                             "36863 keys, 64 heads of dim 128, full windows",
}
# The pages' MI355X (gfx950) time for FlyDSL fp8_mqa_logits at that shape
# (aiter PR "LDS-staged fp8_mqa_logits for gfx942", gfx950 section): context
# only; the pages do not state its windows.
PAGES_US = {"mqa_logits_4095x36863": 1635.0}


def measure_indexer(workload: str, steps: int, warmup: int, dev):
    """Time pa_mqa_logits (and, for indexer_decode, pa_topk) with inputs
    resident in HBM: one pair of HIP events on the launch stream around K
    calls, after the clock settle and warm-up calls."""
    if workload == "indexer_decode":
        x, k = W.config_indexer_decode(), 2048
    else:
        x, k = W.make_indexer_case(W.config_seed(8), 4095, 36863, heads=64, windows="full", name=workload), 0
    d = {n: getattr(x, n).to(dev).contiguous() for n in ("q", "kv", "kv_scale", "weights", "ks", "ke")}
    logits = torch.empty((x.rows, x.num_kv), dtype=torch.float32, device=dev)
    idx = torch.empty((x.rows, max(k, 1)), dtype=torch.int32, device=dev)
    cnt = torch.empty((x.rows,), dtype=torch.int32, device=dev)
    ws = torch.empty(max(B.topk_workspace_bytes(x.rows, x.num_kv, max(k, 1)), 16), dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def lg():
        B.pa_mqa_logits(logits, d["q"], d["kv"], d["kv_scale"], d["weights"], d["ks"], d["ke"], True, stream)

    def tk():
        B.pa_topk(idx, cnt, logits, d["ks"], d["ke"], None, stream, workspace=ws)

    def region(body, n):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for _ in range(n):
            body()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / n

    settle_ms = 0.0
    while settle_ms < settle_ms_target:
        settle_ms += region(lg, 5) * 5 / 1e3
    for _ in range(warmup):
        lg()
        if k:
            tk()
    lo = x.ks.numpy().clip(0, x.num_kv)
    hi = np.maximum(x.ke.numpy(), lo).clip(0, x.num_kv)
    pairs = int((hi - lo).sum())  # (row, key) scores computed
    heads = x.q.shape[1]
    flops = 2.0 * pairs * heads * 128
    us_lg = region(lg, steps)
    res = {"description": INDEXER_WORKLOADS[workload], "kernel": "mqa_logits_kernel",
           "rows": x.rows, "keys": x.num_kv, "heads": heads, "flops_per_call": flops,
           "logits_us": round(us_lg, 2), "logits_tflops": round(flops / us_lg / 1e6, 1),
           "logits_bytes_written": x.rows * x.num_kv * 4,
           "roofline": {"bound": "mfma", "achieved": round(flops / us_lg / 1e6, 1), "peak": PEAK_FP8_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(flops / us_lg / 1e6 / PEAK_FP8_TFLOPS, 4)},
           "clock_settle_ms": round(settle_ms, 1)}
    if k:
        us_tk = region(tk, steps)
        us_both = region(lambda: (lg(), tk()), steps)
        res.update({"topk": k, "topk_us": round(us_tk, 2), "indexer_us": round(us_both, 2),
                    "topk_gbps_logits_read": round(x.rows * x.num_kv * 4 / us_tk / 1e3, 1)})
    if workload in PAGES_US:
        res["pages_us_context"] = {"value": PAGES_US[workload], "note": "FlyDSL on MI355X, windows not stated"}
    return res


def ceiling(args, dev):
    """What the memory system gives for the decode's access pattern: the
    read-only probes of libpa_ceiling.so over the dense MTP4 FP8 batch's own
    pages and work list (the streaming kernel's register loads; the same
    bytes through an LDS ring), the decode launch itself, and a plain read of
    a contiguous 2 GiB buffer, timed alike (cold: three rotating copies of the
    caches).  Prints one JSON line."""
    import ctypes

    from paged_attention_decode_plan_amd.build import CEILING_LIB

    if not os.path.exists(CEILING_LIB):
        raise SystemExit(f"{CEILING_LIB} not built (paged_attention_decode_plan_amd.build)")
    C = ctypes.CDLL(CEILING_LIB)
    vp = ctypes.c_void_p
    C.pa_ceiling_gather.restype = ctypes.c_int
    C.pa_ceiling_gather.argtypes = [ctypes.c_int] + [vp] * 7 + [ctypes.c_int, vp] + [ctypes.c_int] * 3 + [vp]
    C.pa_ceiling_read.restype = ctypes.c_int
    C.pa_ceiling_read.argtypes = [vp, ctypes.c_size_t, vp, ctypes.c_int, vp]
    inp, plan_kw = make_inputs("dense_mtp4_fp8")
    p = inp.problem
    d = {k: v.to(dev).contiguous() for k, v in dict(q=inp.q, k=inp.k_cache, v=inp.v_cache, bt=inp.block_tables,
                                                       cl=inp.context_lens, ks=inp.k_scale, vs=inp.v_scale).items()}
    plan = B.Plan(B.problem_of(p), inp.context_lens, **plan_kw).allocate(dev)
    items = plan.work_list_device()
    n = items.shape[0]
    out = torch.empty(n * 256, dtype=torch.int32, device=dev)
    qout = torch.empty_like(d["q"])
    copies = [(d["k"], d["v"], d["ks"], d["vs"])] + [tuple(t.clone() for t in (d["k"], d["v"], d["ks"], d["vs"]))
                                                      for _ in range(2)]
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream
    kv_bytes = W.kv_bytes_visible(inp)

    def probe(mode, c):
        kc, vc, ksc, vsc = copies[c]
        st = C.pa_ceiling_gather(mode, kc.data_ptr(), vc.data_ptr(), ksc.data_ptr(), vsc.data_ptr(),
                                 d["bt"].data_ptr(), d["cl"].data_ptr(), items.data_ptr(), n, out.data_ptr(),
                                 p.num_kv_heads, p.page_size, p.table_stride, sp)
        assert st == 0, f"probe mode {mode}: status {st}"

    def decode(c):
        kc, vc, ksc, vsc = copies[c]
        B.pa_decode(plan, qout, d["q"], kc, vc, d["bt"], d["cl"], ksc, vsc, None, stream)

    def region(body, K):
        for k in range(3):
            body(k % 3)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for k in range(K):
            body(k % 3)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / K

    K = args.steps
    res = {"metric": "read bandwidth of the decode's KV access pattern (ceiling probes)", "workload": "dense_mtp4_fp8",
           "kv_bytes_per_call": kv_bytes, "work_items": n, "steps": K, "kernel_sha": source_sha()}
    rounds = {"registers": [], "registers_full_rows": [], "lds_ring": [], "decode": []}
    for _ in range(3):  # interleaved rounds, best of three
        rounds["registers"].append(region(lambda c: probe(0, c), K))
        rounds["registers_full_rows"].append(region(lambda c: probe(2, c), K))
        rounds["lds_ring"].append(region(lambda c: probe(1, c), K))
        rounds["decode"].append(region(decode, K))
    for name, v in rounds.items():
        us = min(v)
        res[name] = {"us": round(us, 2), "gbps": round(kv_bytes / (us * 1e-6) / 1e9, 1),
                     "frac": round(kv_bytes / (us * 1e-6) / 1e9 / PEAK_GBPS, 4), "rounds_us": [round(x, 2) for x in v]}
    del copies
    torch.cuda.empty_cache()
    nbytes = 2 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    best = None
    for grid in (1024, 2048, 4096, 8192):
        rout = torch.empty(grid * 256, dtype=torch.int32, device=dev)
        us = region(lambda c: C.pa_ceiling_read(buf.data_ptr(), nbytes, rout.data_ptr(), grid, sp), max(5, K // 4))
        gbps = nbytes / (us * 1e-6) / 1e9
        res.setdefault("plain_read", {})[str(grid)] = round(gbps, 1)
        best = gbps if best is None else max(best, gbps)
    res["plain_read_best_gbps"] = round(best, 1)
    print(json.dumps(res), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="dense_mtp4_fp8", choices=sorted(WORKLOADS))
    ap.add_argument("--only", action="store_true", help="measure the chosen workload alone (no workloads object)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-budget", type=float, default=12.0)
    ap.add_argument("--indexer", choices=sorted(INDEXER_WORKLOADS), default=None,
                    help="measure one indexer workload alone and print its JSON")
    ap.add_argument("--settle-ms", type=float, default=SETTLE_MS,
                    help="untimed calls of each workload before its warm-up steps, in ms of GPU time")
    ap.add_argument("--merge", choices=sorted(MERGE), default=None,
                    help="merge of multi-partition units (default: the library's choice, the reducer)")
    ap.add_argument("--ceiling", action="store_true",
                    help="run the read-only bandwidth probes of the decode's access pattern instead")
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
    global merge_mode, settle_ms_target
    settle_ms_target = args.settle_ms
    if args.merge:
        merge_mode = MERGE[args.merge]
    if args.ceiling:
        ceiling(args, dev)
        return
    if args.copy_calibration > 0:
        n = args.copy_calibration << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log(f"calibration copy: {n} bytes read, {n} bytes written")
    if args.indexer:
        r = measure_indexer(args.indexer, args.steps, args.warmup, dev)
        r.update({"workload": args.indexer, "kernel_sha": source_sha()})
        print(json.dumps(r), flush=True)
        return

    head, inp = measure(args.workload, args.steps, args.warmup, dev)
    p = inp.problem
    on_device = inp.k_cache.is_cuda  # too large for the host oracle's timing loop
    cpu = None if (args.no_cpu or on_device) else cpu_baseline(inp, args.cpu_budget)
    del inp
    kv_bytes = head["kv_bytes_per_call"]
    achieved = head["decode_gbps_cold"]
    roofline = {"bound": "hbm", "achieved": achieved, "peak": PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / PEAK_GBPS, 4), "traffic": load_traffic(args.workload)}
    extra = {}
    if not args.only:
        for wl in EXTRA_WORKLOADS:
            if wl == args.workload:
                continue
            r, _ = measure(wl, args.steps, args.warmup, dev)
            extra[wl] = r
            log(f"{wl}: {r['us_per_call_cold']} us cold, {r['gbps_cold']} GB/s")
        for wl in INDEXER_WORKLOADS:
            r = measure_indexer(wl, max(3, args.steps // 5) if wl != "indexer_decode" else args.steps,
                                min(args.warmup, 3), dev)
            extra[wl] = r
            log(f"{wl}: logits {r['logits_us']} us, {r['logits_tflops']} TFLOP/s")
    res = {
        "metric": "achieved HBM GB/s of KV bytes (and us/call), FP8 paged decode",
        "value": head["gbps_cold"],
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["us_per_call_cold"] / 1e3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if p.kv_dtype == "fp8" else "bf16",
        "data": "synthetic",
        "config": {"workload": args.workload, "description": WORKLOADS[args.workload],
                   "kv_bytes_per_call": kv_bytes, "work_items": head["work_items"], "partials": head["partials"],
                   "merge": head["merge"],
                   "cu_count": head["cu_count"]},
        "us_per_call_cold": head["us_per_call_cold"],
        "us_per_call_warm": head["us_per_call_warm"],
        "decode_us_cold": head["decode_us_cold"],
        "warm_gbps": head["gbps_warm"],
        "frac_of_peak_cold": round(head["gbps_cold"] / PEAK_GBPS, 4),
        "wall_s_timed_regions": head["wall_s_timed_regions"],
        "clock_settle_ms": head["clock_settle_ms"],
        "roofline": roofline,
        "mfma_busy_fraction": load_mfma(args.workload),
        "cpu_baseline": cpu,
        "kernel": head["kernel"],
        "kernel_sha": source_sha(),
    }
    if args.workload in PAGES_GBPS:
        res["pages_gbps_context"] = head["pages_gbps_context"]
    if extra:
        res["workloads"] = extra
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
