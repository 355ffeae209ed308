"""Shared helpers of the GPU tests: run the library on workload inputs with
NaN-poisoned output and workspace, and compare with the oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

from paged_attention_decode_plan_amd import binding as B

ATOL = 0.005
RTOL = 0.005


def announce(msg: str):
    print(f"[case] {msg}", flush=True)
    sys.stdout.flush()


def to_device(inp, device="cuda"):
    def d(t):
        return None if t is None else t.to(device).contiguous()

    return dict(q=d(inp.q), k_cache=d(inp.k_cache), v_cache=d(inp.v_cache), block_tables=d(inp.block_tables),
                context_lens=d(inp.context_lens), k_scale=d(inp.k_scale), v_scale=d(inp.v_scale), sinks=d(inp.sinks),
                topk_indices=d(getattr(inp, "topk_indices", None)))


def check_shapes(inp, dev):
    """Host-side check that the tensors match the problem before any launch."""
    p = inp.problem
    per_page = p.num_kv_heads * p.head_dim * p.page_size
    cache_bytes = {"fp8": per_page, "bf16": 2 * per_page, "mxfp4": per_page // 2}[p.kv_dtype] * p.num_pages
    assert dev["q"].shape == (p.rows, p.num_q_heads, p.head_dim)
    assert dev["k_cache"].numel() * dev["k_cache"].element_size() == cache_bytes
    assert dev["v_cache"].numel() * dev["v_cache"].element_size() == cache_bytes
    assert dev["block_tables"].shape == (p.num_seqs, p.table_stride)
    assert dev["context_lens"].shape == (p.num_seqs,)
    bt = inp.block_tables.cpu().numpy()
    lens = inp.context_lens.cpu().numpy()
    for s in range(p.num_seqs):
        if p.token_table == 2:  # the whole page table is reachable (positions are clamped into it)
            used, lim = bt[s], p.num_pages
            assert dev["topk_indices"].shape == (p.num_seqs, p.index_stride)
        else:
            n = int(min(max(lens[s], 0), p.table_stride if p.token_table else p.table_stride * p.page_size))
            used = bt[s, :n] if p.token_table else bt[s, : (n + p.page_size - 1) // p.page_size]
            lim = p.num_pages * p.page_size if p.token_table else p.num_pages
        assert (used >= 0).all() and (used < lim).all(), "table entry out of range"
    if p.kv_dtype == "fp8" and p.scale_mode == "token":
        assert dev["k_scale"].shape == (p.num_pages, p.num_kv_heads, p.page_size)
    if p.kv_dtype == "mxfp4":
        for t in (dev["k_scale"], dev["v_scale"]):
            assert t.dtype == torch.uint8 and t.shape == (p.num_pages, p.num_kv_heads, p.page_size, p.head_dim // 32)


def run(inp, dev=None, plan=None, lens_for_plan=None, **plan_kw):
    """Decode + reduce on the GPU; returns (out float32 cpu, plan)."""
    p = inp.problem
    if dev is None:
        dev = to_device(inp)
    check_shapes(inp, dev)
    if plan is None:
        lens = inp.context_lens if lens_for_plan is None else lens_for_plan
        plan = B.Plan(B.problem_of(p), lens, **plan_kw).allocate("cuda")
    plan.workspace.fill_(float("nan"))
    out = torch.full_like(dev["q"], float("nan"))
    if p.token_table == 2:
        B.pa_decode_sparse(plan, out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"],
                           dev["topk_indices"], dev["context_lens"], dev["k_scale"], dev["v_scale"], dev["sinks"])
        B.pa_reduce(plan, out, dev["sinks"])
    else:
        B.attend(plan, out, dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"],
                 dev["k_scale"], dev["v_scale"], dev["sinks"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), plan


def compare(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref)
    bad = err > ATOL + RTOL * np.abs(ref)
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {bad.sum()} of {bad.size} outside tolerance; max err {err.max():.3g}; "
                             f"first {idx.tolist()} got {got[bad][:5]} ref {ref[bad][:5]}")
    return float(err.max())
