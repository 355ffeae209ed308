"""Bit-exact gather addressing on the GPU: planted-token integer probes.

One visible token's key agrees with the query of ones and every other
visible key opposes it (FP8 +16 / -16 codes, or BF16 +-16), so every other
weight underflows to exactly 0 and the output must equal the target
token's V row exactly.  That V row holds small-integer digits that encode
the token's physical page and slot, so a wrong page id, slot, layout offset
or scale index shows as wrong digits; tolerance parity could not see it on
long contexts, where one misplaced token moves an output by about 1/L.
Per-token scales are powers of two (random per token), so the expected
output is the target's V scale times its digits, still exact in BF16.

The target sweeps page, tile, partition, staged-bound and window edges, at
16, 32 and 64 query rows per KV head (the tile kernel and both row-block
counts of the streaming kernel), pages of 16, 64 and 128 tokens, plain and
transposed V, per-tensor and per-token scales; plus head dim 256, BF16
caches and token tables (the sparse gather)."""

from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from gpu_helpers import announce, run
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

POS, NEG = 0x58, 0xD8  # +16.0 and -16.0 in e4m3fn


def _digits(pid, slot, D):
    return (pid * 7 + slot * 3 + np.arange(D)) % 16


def _pow2_scales(inp, seed):
    """Per-token scales replaced by random powers of two (2^-1 .. 2^2) where
    they hold real data; poisoned slots keep their poison."""
    g = torch.Generator().manual_seed(seed)
    for t in (inp.k_scale, inp.v_scale):
        real = t < 1e29
        e = torch.randint(-1, 3, t.shape, generator=g).float()
        t[real] = torch.exp2(e)[real]


def _write_kv(inp, pid, slot, kcode, vrow):
    """K of tokens (pid, slot) set to one code/value in every dim (all KV
    heads); V of one token (vrow given) to the digits."""
    p = inp.problem
    D = p.head_dim
    if p.kv_dtype == "fp8":
        kc = inp.k_cache.view(p.num_pages, p.num_kv_heads, D // 16, p.page_size, 16)
        kc[pid, :, :, slot, :] = kcode[:, None, None, None]
    else:
        kc = inp.k_cache.view(torch.int16).view(p.num_pages, p.num_kv_heads, D // 8, p.page_size, 8)
        kc[pid, :, :, slot, :] = kcode[:, None, None, None]
    if vrow is not None:
        tp, ts, digits = vrow
        if p.kv_dtype == "fp8":
            vals = W.to_fp8_bytes(torch.tensor(digits, dtype=torch.float32))
            vc = inp.v_cache
            x = 16
        else:
            vals = torch.tensor(digits, dtype=torch.float32).to(torch.bfloat16).view(torch.int16)
            vc = inp.v_cache.view(torch.int16)
            x = 8
        if p.v_transposed:
            vc.view(p.num_pages, p.num_kv_heads, p.page_size // x, D, x)[tp, :, ts // x, :, ts % x] = vals
        else:
            vc.view(p.num_pages, p.num_kv_heads, D, p.page_size)[tp, :, :, ts] = vals


def _kvals(kv, n, target_mask):
    if kv == "fp8":
        return torch.where(target_mask, POS, NEG).to(torch.uint8)
    pos = torch.tensor([16.0], dtype=torch.bfloat16).view(torch.int16)[0]
    neg = torch.tensor([-16.0], dtype=torch.bfloat16).view(torch.int16)[0]
    return torch.where(target_mask, pos, neg).to(torch.int16)


def _dense_probe(ql, hq, hkv, d, page, vt, scale, kv="fp8", L=700, window=0, seed=300):
    base = W.make_dense_case(seed, [L, 300], query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                             page_size=page, kv_dtype=kv, v_transposed=vt, scale_mode=scale if kv == "fp8" else "none",
                             sliding_window=window, fill="context", poison=True)
    p = base.problem
    base.q.fill_(1.0)
    if kv == "fp8":
        if scale == "token":
            _pow2_scales(base, seed)
        else:
            base.k_scale.fill_(1.0)
            base.v_scale.fill_(1.0)
    lo = max(0, L - ql - window + 1) if window else 0
    # page, tile and partition edges, the staged-bound edge (5 pages with
    # stage_limit=5), the window's first tokens and the last visible ones
    edges = {lo, lo + 1, page - 1, page, 127, 128, 129, 255, 256, 511, 512, 5 * page - 1, 5 * page, L - ql - 1, L - ql}
    targets = sorted(e for e in edges if lo <= e <= L - ql)
    t = torch.arange(lo, L)
    bt0 = base.block_tables[0].long()
    pid_all, slot_all = bt0[t // page], t % page
    for tgt in targets:
        tp, ts = int(bt0[tgt // page]), tgt % page
        digits = _digits(tp, ts, d)
        _write_kv(base, pid_all, slot_all, _kvals(kv, len(t), t == tgt), (tp, ts, digits))
        for kw in [dict(cu_count=4, max_partitions=1, stage_limit=5), dict(cu_count=256, partition_tokens=128)]:
            got, _ = run(base, **kw)
            for i in range(ql):
                pos = L - ql + i
                vis_lo = max(0, pos - window + 1) if window else 0
                if not (vis_lo <= tgt <= pos):
                    continue
                for h in range(hq):
                    vs_h = float(base.v_scale[tp, h // (hq // hkv), ts]) if (kv == "fp8" and scale == "token") else 1.0
                    want = (digits * vs_h).astype(np.float32)
                    assert np.array_equal(got[i, h], want), (tgt, i, h, kw, got[i, h][:8], want[:8])
    return len(targets)


ROWS = {16: (1, 16), 32: (2, 16), 64: (4, 16)}


@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("page,vt,scale", list(itertools.product([16, 32, 64, 128], [False, True], ["tensor", "token"])))
def test_planted_digits_fp8(rows, page, vt, scale):
    ql, hq = ROWS[rows]
    announce(f"planted digits fp8 rows={rows} page={page} vt={vt} scale={scale}")
    n = _dense_probe(ql, hq, 1, 128, page, vt, scale, seed=300 + rows + page + 2 * vt + (scale == "token"))
    assert n >= 8


@pytest.mark.parametrize("ql,window,page", [(1, 0, 64), (4, 0, 64), (2, 33, 64), (4, 33, 64), (3, 0, 16), (4, 0, 16)])
@pytest.mark.parametrize("vt", [False, True])
def test_planted_digits_d256(ql, window, page, vt):
    """Head dim 256: 8 and 16 rows per KV head in the tile kernel, 24 and 32
    in the streaming kernel."""
    announce(f"planted digits d256 ql={ql} w={window} page={page} vt={vt}")
    _dense_probe(ql, 16, 2, 256, page, vt, "token" if ql >= 3 else "tensor", window=window,
                 seed=340 + ql + window + page)


@pytest.mark.parametrize("rows", [16, 32, 64])
@pytest.mark.parametrize("page,vt", [(256, False), (256, True), (512, False), (1024, True)])
def test_planted_digits_large_pages(rows, page, vt):
    """Pages above 128 tokens: the digits of the target encode its physical
    page and slot, so a wrong sub-page offset in K, V or the scales shows."""
    ql, hq = ROWS[rows]
    announce(f"planted digits large pages rows={rows} page={page} vt={vt}")
    _dense_probe(ql, hq, 1, 128, page, vt, "token", L=2 * page + 300, seed=390 + rows + page + vt)


@pytest.mark.parametrize("ql,page,vt,scale", [(1, 16, False, "tensor"), (4, 64, True, "token"), (2, 128, False, "token"),
                                            (4, 256, True, "tensor")])
def test_planted_digits_d512(ql, page, vt, scale):
    announce(f"planted digits d512 ql={ql} page={page} vt={vt} scale={scale}")
    _dense_probe(ql, 16, 1, 512, page, vt, scale, seed=395 + ql + page)


@pytest.mark.parametrize("kv,scale", [("fp8", "tensor"), ("fp8", "token"), ("bf16", "none")])
@pytest.mark.parametrize("ql,page,vt", [(1, 16, False), (4, 64, True), (2, 32, False)])
def test_planted_digits_d64(kv, scale, ql, page, vt):
    announce(f"planted digits d64 {kv} {scale} ql={ql} page={page} vt={vt}")
    _dense_probe(ql, 16, 1, 64, page, vt, scale, kv=kv, seed=380 + ql + page + (scale == "token"))


@pytest.mark.parametrize("page,vt,ql", [(16, False, 1), (128, True, 4), (64, False, 2)])
def test_planted_digits_bf16(page, vt, ql):
    announce(f"planted digits bf16 page={page} vt={vt} ql={ql}")
    _dense_probe(ql, 16, 1, 128, page, vt, "none", kv="bf16", seed=360 + page + ql)


def test_planted_digits_token_table():
    """The sparse gather: row 0's selected physical slots; the target's
    digits encode its physical page and slot."""
    inp = W.config_sparse(num_rows=2, selected=600, pool_pages=64)
    p = inp.problem
    inp.q.fill_(1.0)
    _pow2_scales(inp, 77)
    S = inp.block_tables[0].long()
    pid_all, slot_all = S // p.page_size, S % p.page_size
    targets = [0, 1, 15, 16, 127, 128, 129, 300, 511, 512, 599]
    for j in targets:
        tp, ts = int(pid_all[j]), int(slot_all[j])
        digits = _digits(tp, ts, p.head_dim)
        mask = torch.arange(len(S)) == j
        _write_kv(inp, pid_all, slot_all, _kvals("fp8", len(S), mask), (tp, ts, digits))
        announce(f"planted digits token table j={j}")
        for kw in [dict(cu_count=4, max_partitions=1, stage_limit=5), dict(cu_count=64, partition_tokens=128)]:
            got, _ = run(inp, **kw)
            want = (digits * float(inp.v_scale[tp, 0, ts])).astype(np.float32)
            for h in range(p.num_q_heads):
                assert np.array_equal(got[0, h], want), (j, h, kw)
