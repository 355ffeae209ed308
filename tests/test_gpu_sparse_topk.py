"""GPU parity of the two-level sparse gather (pa_decode_sparse): rows attend
top-k logical positions of a paged sequence, resolved in the kernel through
the block table (the sparse MLA decode of aiter PR #7079, Summary: a top-k
index stage selects token positions, a block-table stage maps them to
physical KV).  Checked against the oracle within atol = rtol = 0.005, bit for
bit against the same call with the positions resolved on the host (physical
token slots), with indices and counts outside their ranges (clamped), and
with planted-token integer probes whose digits encode the physical page and
slot the kernel read."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run
from oracle import oracle as O
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

PLANS = [dict(cu_count=64, partition_tokens=256), dict(cu_count=4, max_partitions=1, stage_limit=5),
         dict(cu_count=256, partition_tokens=512)]


@pytest.mark.parametrize("kw", PLANS, ids=["p256", "one_partition_staged5", "p512"])
def test_two_level_parity(kw):
    inp = W.config_sparse_topk(num_rows=6, selected=700, pool_pages=64)
    inp.context_lens[:] = torch.tensor([700, 0, 1, 333, 17, 699], dtype=torch.int32)
    announce(f"two-level parity {kw}")
    got, _ = run(inp, **kw)
    compare(got, O.attend(inp), f"two-level {kw}")


@pytest.mark.parametrize("kw", PLANS[:2], ids=["p256", "one_partition_staged5"])
def test_two_level_bit_identical_to_resolved(kw):
    """The kernel resolves positions to the slots the host resolution gives,
    in the same order, so the two calls agree bit for bit."""
    inp = W.config_sparse_topk(num_rows=6, selected=700, pool_pages=64)
    announce(f"two-level vs host-resolved {kw}")
    got2, _ = run(inp, **kw)
    got1, _ = run(W.resolve_topk(inp), **kw)
    assert np.array_equal(got2, got1)


def test_two_level_clamped_indices_and_counts():
    """Positions below 0 or past the block table's capacity are clamped into
    it; counts below 0 count as 0 and counts past the index row's stride as
    the stride."""
    inp = W.config_sparse_topk(num_rows=4, selected=300, pool_pages=32)
    p = inp.problem
    cap = p.table_stride * p.page_size
    tk = inp.topk_indices.clone()
    tk[0, ::7] = -5
    tk[1, ::5] = cap + 3
    tk[2, 10] = 1 << 30
    tk[3, 0] = -(1 << 30)
    lens = torch.tensor([p.index_stride + 9, -3, 1 << 30, 250], dtype=torch.int32)
    wild = dataclasses.replace(inp, topk_indices=tk, context_lens=lens)
    announce(f"two-level clamped indices cap={cap}")
    got, _ = run(wild, cu_count=64, partition_tokens=128)
    compare(got, O.attend(wild), "two-level clamped")


def test_two_level_full_size():
    """The benchmark's sparse_topk batch (64 rows, 2048 of 65536 positions,
    4096-page table) in its launch configuration: every output, and bit for
    bit the one-level call on the host-resolved slots."""
    from bench import make_inputs

    inp, plan_kw = make_inputs("sparse_topk")
    announce("two-level full size: every output")
    got, _ = run(inp, **plan_kw)
    compare(got, O.attend(inp), "two-level full size")
    got1, _ = run(W.resolve_topk(inp), **plan_kw)
    assert np.array_equal(got, got1)


def test_planted_digits_two_level():
    """One selected position's key agrees with the query and every other
    opposes it; the target's V digits encode its physical page and slot, so
    a wrong table lookup or position split shows as wrong digits."""
    inp = W.config_sparse_topk(num_rows=2, selected=600, pool_pages=64)
    p = inp.problem
    inp.q.fill_(1.0)
    g = torch.Generator().manual_seed(91)
    for t in (inp.k_scale, inp.v_scale):
        t.copy_(torch.exp2(torch.randint(-1, 3, t.shape, generator=g).float()))
    pos = inp.topk_indices[0].long()
    pid = inp.block_tables[0].long()[pos // p.page_size]
    slot = pos % p.page_size
    D = p.head_dim
    kc = inp.k_cache.view(p.num_pages, p.num_kv_heads, D // 16, p.page_size, 16)
    vc = inp.v_cache.view(p.num_pages, p.num_kv_heads, D, p.page_size)
    for j in [0, 1, 15, 16, 127, 128, 129, 300, 511, 512, 599]:
        tp, ts = int(pid[j]), int(slot[j])
        digits = (tp * 7 + ts * 3 + np.arange(D)) % 16
        codes = torch.full((len(pos),), 0xD8, dtype=torch.uint8)  # -16 in e4m3fn
        codes[j] = 0x58  # +16
        kc[pid, :, :, slot, :] = codes[:, None, None, None]
        vc[tp, :, :, ts] = W.to_fp8_bytes(torch.tensor(digits, dtype=torch.float32))
        announce(f"planted digits two-level j={j}")
        for kw in [dict(cu_count=4, max_partitions=1, stage_limit=5), dict(cu_count=64, partition_tokens=128)]:
            got, _ = run(inp, **kw)
            want = (digits * float(inp.v_scale[tp, 0, ts])).astype(np.float32)
            for h in range(p.num_q_heads):
                assert np.array_equal(got[0, h], want), (j, h, kw)
