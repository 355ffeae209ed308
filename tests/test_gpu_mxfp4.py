"""MXFP4 caches on the GPU (the tile kernel's MX path) against the CPU
oracle, atol = rtol = 0.005, and planted-token probes that check the
gather bit-exactly.

Parity: 8, 16, 32 and 64 query rows per KV head, pages of 32, 64 and 128
tokens, windows, sinks, FP16 queries, empty and one-token sequences, and
plans with one item per sequence, several 256-token partitions (a small CU
budget) and explicit 256-token partitions.  Outputs and partials start as
NaN, unreferenced pages and slots outside the visible spans carry NaN
scale bytes (0xFF)."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run
from oracle import oracle as O
from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

SHAPES = {8: (1, 8, 1), 16: (4, 16, 4), 32: (2, 16, 1), 64: (4, 16, 1)}  # rows -> (QL, Hq, Hkv)
LENS = [0, 1, 33, 300, 1000, 2100, 4097]


@pytest.mark.parametrize("rows", [8, 16, 32, 64])
@pytest.mark.parametrize("page", [32, 64, 128])
@pytest.mark.parametrize("window,sinks", [(0, False), (17, True), (257, False)])
def test_mxfp4_parity(rows, page, window, sinks):
    ql, hq, hkv = SHAPES[rows]
    x = W.make_dense_case(900 + rows + page + window, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv,
                          head_dim=128, page_size=page, kv_dtype="mxfp4", sliding_window=window, has_sinks=sinks)
    ref = O.attend(x)
    for kw in (dict(), dict(cu_count=8), dict(partition_tokens=256)):
        announce(f"mxfp4 rows={rows} page={page} window={window} sinks={sinks} {kw}")
        got, plan = run(x, **kw)
        work = plan.work().numpy()
        assert (work[:, 3] % 2 == 0).all(), "a partition starts inside a 256-token unit"
        compare(got, ref, f"mxfp4 rows={rows} page={page} window={window} {kw}")


def test_mxfp4_fp16_queries_and_scale_jumps():
    """FP16 queries; V block scales near 1 except one block of each
    sequence's last visible tokens, 2^5 above the rest: more than the
    reference band, so the V-scale reference of that block restarts.  (The
    jump stays moderate: with FP16 probabilities, V values thousands of times
    larger than the output cancel to more than the tolerance.)"""
    x = W.make_dense_case(951, [5, 700, 2600], query_len=4, num_q_heads=16, num_kv_heads=1, head_dim=128,
                          page_size=64, kv_dtype="mxfp4", q_dtype="fp16", poison=False)
    g = torch.Generator().manual_seed(3)
    x.v_scale.copy_(torch.randint(126, 129, x.v_scale.shape, generator=g).to(torch.uint8))
    bt = x.block_tables.numpy()
    for s_, L in enumerate(x.context_lens.tolist()):
        for t in range(max(0, L - 3), L):
            x.v_scale[int(bt[s_, t // 64]), 0, t % 64, t % 4] = 132
    announce("mxfp4 fp16 queries, V scale jumps")
    got, _ = run(x)
    compare(got, O.attend(x), "mxfp4 V scale jumps")


def test_mxfp4_rejections():
    x = W.make_dense_case(952, [100], query_len=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=32,
                          kv_dtype="mxfp4")
    with pytest.raises(Exception):
        B.Plan(B.problem_of(x.problem), x.context_lens, partition_tokens=512)
    with pytest.raises(Exception):
        B.Plan(B.problem_of(x.problem), x.context_lens, refreshable=1)


# ---- planted-token probes ----
POS4, NEG4 = 0x6, 0xE  # E2M1 +4.0 and -4.0


def _digit_codes(pid, slot, D):
    return (pid * 7 + slot * 3 + np.arange(D)) % 8  # non-negative E2M1 codes 0 .. 7


@pytest.mark.parametrize("rows", [8, 32, 64])
@pytest.mark.parametrize("page", [32, 128])
def test_mxfp4_planted_digits(rows, page):
    """One visible token's key agrees with the query of ones, every other
    opposes it: the output is that token's V row exactly (its digits times
    its block scales, random powers of two)."""
    ql, hq, hkv = SHAPES[rows]
    L, D = 700, 128
    x = W.make_dense_case(960 + rows + page, [L, 300], query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=D,
                          page_size=page, kv_dtype="mxfp4", fill="context", poison=True)
    p = x.problem
    x.q.fill_(1.0)
    kc = x.k_cache.view(p.num_pages, p.num_kv_heads, D // 32, page, 16)
    vc = x.v_cache.view(p.num_pages, p.num_kv_heads, D, page // 2)
    bt0 = x.block_tables[0].long()
    g = torch.Generator().manual_seed(rows + page)
    t = torch.arange(0, L)
    pids, slots = bt0[t // page], t % page
    x.k_scale[pids, :, slots] = 127
    x.v_scale[pids, :, slots] = torch.randint(125, 130, (L, p.num_kv_heads, D // 32), generator=g).to(torch.uint8)
    edges = sorted({0, 1, page - 1, page, 127, 128, 255, 256, 257, 511, 512, 5 * page, L - ql - 1, L - ql})
    for tgt in edges:
        tp, ts = int(bt0[tgt // page]), tgt % page
        kcode = torch.where(t == tgt, POS4, NEG4).to(torch.uint8)
        kc[pids, :, :, slots, :] = (kcode | (kcode << 4))[:, None, None, None]
        digits = _digit_codes(tp, ts, D)
        row = vc[tp, :, :, ts // 2]
        keep = (row >> 4) if ts % 2 == 0 else (row & 0xF)
        new = torch.from_numpy(digits.astype(np.uint8))[None, :]
        vc[tp, :, :, ts // 2] = (keep << 4) | new if ts % 2 == 0 else (new << 4) | keep
        for kw in (dict(cu_count=4, max_partitions=1, stage_limit=5), dict(cu_count=256, partition_tokens=256)):
            announce(f"mxfp4 probe rows={rows} page={page} target={tgt} {kw}")
            got, _ = run(x, **kw)
            for i in range(ql):
                if tgt > L - ql + i:
                    continue
                for h in range(hq):
                    kvh = h // (hq // hkv)
                    sc = np.exp2(x.v_scale[tp, kvh, ts].numpy().astype(np.float64) - 127)
                    want = (np.array(W.FP4_GRID)[digits] * np.repeat(sc, 32)).astype(np.float32)
                    assert np.array_equal(got[i, h], want), (tgt, i, h, kw, got[i, h][:8], want[:8])
