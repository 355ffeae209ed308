"""GPU tests of the in-kernel merge (plan option merge = 2): the last work
item of each multi-partition unit to arrive merges the unit's partials in
the decode launch (aiter PR #7079, "Partition merges": last-arriving CTA,
arrival counters reset by the last arrival so that graph replays need no
host work).  Every output is compared bit for bit with the reducer launch
on the same plan shape, with NaN-poisoned workspace and output before every
call, over consecutive calls whose queries change (a stale partial or a
counter left non-zero would show), in every decode kernel, and under HIP
graph replays; and within tolerance with the oracle."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run, to_device
from oracle import oracle as O
from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu


def _case(kind):
    lens = [3000, 0, 1, 700, 129, 2049]
    if kind == "tile16":  # 16-row tile kernel: ragged batch shape (GQA 4, window, sinks, per-token)
        return W.make_dense_case(501, lens, query_len=1, num_q_heads=16, num_kv_heads=4, page_size=16,
                                 scale_mode="token", sliding_window=257, has_sinks=True), dict(cu_count=64)
    if kind == "stream64":
        return W.make_dense_case(502, lens, query_len=4, num_q_heads=16, num_kv_heads=1, page_size=128,
                                 scale_mode="token"), dict(cu_count=64)
    if kind == "stream32":
        return W.make_dense_case(503, lens, query_len=2, num_q_heads=16, num_kv_heads=1, page_size=64,
                                 scale_mode="tensor", has_sinks=True, q_dtype="fp16"), dict(cu_count=64)
    if kind == "d256":
        return W.make_dense_case(504, lens, query_len=4, num_q_heads=16, num_kv_heads=2, head_dim=256,
                                 page_size=64, v_transposed=True, sliding_window=1000), dict(cu_count=64)
    if kind == "bf16":
        return W.make_dense_case(505, lens, query_len=4, num_q_heads=16, num_kv_heads=1, page_size=128,
                                 kv_dtype="bf16"), dict(cu_count=64)
    if kind == "mxfp4":  # MXFP4 caches: 256-token partitions, 64 rows (8-wave tile kernel)
        return W.make_dense_case(506, lens, query_len=4, num_q_heads=16, num_kv_heads=1, page_size=64,
                                 kv_dtype="mxfp4", has_sinks=True), dict(cu_count=64)
    if kind == "many_parts":  # a unit of 79 partitions: several round trips of the wider loads
        return W.make_dense_case(507, [20000, 3000, 0], query_len=4, num_q_heads=16, num_kv_heads=1, page_size=128,
                                 scale_mode="token", has_sinks=True), dict(partition_tokens=256, cu_count=256)
    if kind == "sparse":  # the sparse decode shape: 4 partitions of 512 slots per row
        return W.config_sparse(num_rows=8, selected=2048, pool_pages=256), dict(partition_tokens=512)
    if kind == "sparse_topk":
        return W.config_sparse_topk(num_rows=8, selected=2048, pool_pages=256), dict(partition_tokens=512)
    raise ValueError(kind)


KINDS = ["tile16", "stream64", "stream32", "d256", "bf16", "mxfp4", "many_parts", "sparse", "sparse_topk"]


def _with_queries(inp, k):
    """The same problem with the k-th query variant (k = 0: as drawn)."""
    if k == 0:
        return inp
    g = torch.Generator().manual_seed(900 + k)
    q = (inp.q.float() * (1.0 + 0.5 * k) + torch.randn(inp.q.shape, generator=g)).to(inp.q.dtype)
    return dataclasses.replace(inp, q=q)


@pytest.mark.parametrize("kind", KINDS)
def test_in_kernel_merge_bit_exact(kind):
    inp, kw = _case(kind)
    red = B.Plan(B.problem_of(inp.problem), inp.context_lens, merge=B.MERGE_REDUCER, **kw).allocate("cuda")
    ikm = B.Plan(B.problem_of(inp.problem), inp.context_lens, merge=B.MERGE_IN_KERNEL, **kw).allocate("cuda")
    assert ikm.info().max_parts > (32 if kind == "many_parts" else 1), "the case must have multi-partition units"
    for k in range(3):
        case = _with_queries(inp, k)
        announce(f"in-kernel merge {kind} call {k}")
        got, _ = run(case, plan=ikm)
        want, _ = run(case, plan=red)
        assert np.array_equal(got, want), f"{kind} call {k}: in-kernel merge differs from the reducer"
        if k == 0:
            compare(got, O.attend(case), f"in-kernel merge {kind}")


@pytest.mark.parametrize("kind", ["stream64", "tile16"])
def test_in_kernel_merge_graph_replays(kind):
    """pa_decode with the in-kernel merge captured once in a HIP graph and
    replayed with new queries and NaN-poisoned workspace and output before
    each replay (eager work between the replays): every replay bit-identical
    to an eager reducer-path call on the same inputs."""
    inp, kw = _case(kind)
    dev = to_device(inp)
    ikm = B.Plan(B.problem_of(inp.problem), inp.context_lens, merge=B.MERGE_IN_KERNEL, **kw).allocate("cuda")
    red = B.Plan(B.problem_of(inp.problem), inp.context_lens, merge=B.MERGE_REDUCER, **kw).allocate("cuda")
    out = torch.empty_like(dev["q"])
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], dev["context_lens"], dev["k_scale"],
            dev["v_scale"], dev["sinks"])
    B.attend(ikm, out, *args)  # an eager call before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.attend(ikm, out, *args)
    torch.cuda.synchronize()
    for k in range(4):
        announce(f"in-kernel merge graph replay {kind} {k}")
        case = _with_queries(inp, k)
        dev["q"].copy_(case.q.to("cuda"))
        ikm.workspace.fill_(float("nan"))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        want, _ = run(case, plan=red)
        assert np.array_equal(got, want), f"replay {k}"
