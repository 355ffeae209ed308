"""pa_attend_static (metadata and partials in the library's static device
array, no device allocation) against pa_decode + pa_reduce on caller-owned
buffers: bit-identical outputs, on two calls in a row (the second with a
smaller input and plan), then the first plan again (its metadata is copied
back into the shared array)."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, to_device
from oracle import oracle as O
from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W


def test_static_scratch_refuses_oversized_plans():
    """No device needed: a plan whose metadata and partials exceed the
    static array is refused before anything is launched."""
    prob = B.make_problem(4, 4, 16, 1, 128, 128, 4096, 1024, "bf16", "fp8", False, "token", 1, 0, 0, 0, 0.0)
    plan = B.Plan(prob, [131072] * 4, cu_count=256, partition_tokens=128)
    need = plan.workspace_bytes + plan.meta_bytes
    assert need > B.STATIC_SCRATCH_BYTES
    L = B.load_library()
    p = ctypes.c_void_p(0x1000)
    assert L.pa_attend_static(plan.handle, *([p] * 9), None, None) == B.PA_ERR_WORKSPACE
    assert b"static scratch" in L.pa_last_error()


def _run_both(inp, **plan_kw):
    d = to_device(inp)
    plan = B.Plan(B.problem_of(inp.problem), inp.context_lens, **plan_kw)
    assert plan.workspace_bytes + plan.meta_bytes <= B.STATIC_SCRATCH_BYTES
    args = (d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"], d["k_scale"], d["v_scale"],
            d["sinks"])
    out_s = torch.full_like(d["q"], float("nan"))
    B.pa_attend_static(plan, out_s, *args)  # no allocation: plan.meta / plan.workspace stay None
    torch.cuda.synchronize()
    assert plan.meta is None and plan.workspace is None
    plan.allocate("cuda")
    plan.workspace.fill_(float("nan"))
    out_e = torch.full_like(d["q"], float("nan"))
    B.attend(plan, out_e, *args)
    torch.cuda.synchronize()
    return out_s.float().cpu().numpy(), out_e.float().cpu().numpy(), plan


@pytest.mark.gpu
def test_static_scratch_matches_caller_buffers():
    big = W.make_dense_case(191, [9000, 5000, 700, 1, 0], query_len=4, num_q_heads=16, num_kv_heads=1,
                            page_size=128, scale_mode="token", has_sinks=True)
    small = W.make_dense_case(192, [900, 40], query_len=1, num_q_heads=8, num_kv_heads=1, page_size=16,
                              scale_mode="tensor", sliding_window=257)
    announce("static scratch: multi-partition streaming-kernel plan")
    s1, e1, p1 = _run_both(big, cu_count=64)
    assert p1.info().num_slots > 0
    assert np.array_equal(s1, e1)
    compare(s1, O.attend(big), "static scratch, first call")
    announce("static scratch: smaller tile-kernel plan")
    s2, e2, p2 = _run_both(small, cu_count=64)
    assert p2.meta_bytes + p2.workspace_bytes < p1.meta_bytes + p1.workspace_bytes
    assert np.array_equal(s2, e2)
    compare(s2, O.attend(small), "static scratch, second call")
    announce("static scratch: first plan again")
    d = to_device(big)
    out = torch.full_like(d["q"], float("nan"))
    B.pa_attend_static(p1, out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"],
                       d["k_scale"], d["v_scale"], d["sinks"])
    torch.cuda.synchronize()
    assert np.array_equal(out.float().cpu().numpy(), e1)


@pytest.mark.gpu
def test_static_scratch_mxfp4_plans():
    """MXFP4 caches (tile kernel, 256-token partitions): a multi-partition
    plan, then a smaller one, each bit-identical to the caller-buffer path."""
    big = W.make_dense_case(193, [7000, 3000, 300, 0], query_len=4, num_q_heads=16, num_kv_heads=1,
                            page_size=64, kv_dtype="mxfp4", has_sinks=True)
    small = W.make_dense_case(194, [700, 33], query_len=2, num_q_heads=8, num_kv_heads=1, page_size=32,
                              kv_dtype="mxfp4", sliding_window=300)
    announce("static scratch: MXFP4 multi-partition plan")
    s1, e1, p1 = _run_both(big, cu_count=64)
    assert p1.info().num_slots > 0
    assert np.array_equal(s1, e1)
    compare(s1, O.attend(big), "static scratch MXFP4, first call")
    announce("static scratch: smaller MXFP4 plan")
    s2, e2, p2 = _run_both(small, cu_count=64)
    assert p2.meta_bytes + p2.workspace_bytes < p1.meta_bytes + p1.workspace_bytes
    assert np.array_equal(s2, e2)
    compare(s2, O.attend(small), "static scratch MXFP4, second call")
