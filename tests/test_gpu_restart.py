"""GPU parity for inputs whose logits keep climbing along an item, so that
the online softmax's reference maximum must be raised again and again.

Every decode path keeps the probabilities against a per-row reference
maximum and redoes its share with a larger reference when a score climbs
too far above it (the accumulators are only ever written by the matrix
cores).  Here the logits climb by far more than the restart threshold over
one work item, many times over: a ramp of per-token k scales, or of the FP8
(or BF16) key values themselves, with a query of ones, and a ramp of
per-token V scales (2^100 across the context).  The result must still match
the oracle (aiter PR #4332, follow-up commit: silently wrong outputs are
blockers), at 16 rows (tile kernel), 32 and 64 rows (streaming kernel),
head dim 256 and BF16 caches, with one partition per sequence (the whole
climb inside one item) and with the automatic split."""

from __future__ import annotations

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run
from oracle import oracle as O
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

LENS = [6000, 1500, 0]


def _token_index(inp, s):
    """Physical page and slot of every token of sequence s (its whole length)."""
    p = inp.problem
    L = int(inp.context_lens[s])
    t = torch.arange(L)
    pid = inp.block_tables[s].long()[t // p.page_size]
    return t, pid, t % p.page_size


def _ramp_keys(inp, mode):
    """Query of ones; keys that make logit(t) climb by about 0.1 per token in
    base 2 (600 over 6000 tokens: a wave of the streaming kernel sees its
    logits climb past the restart threshold in every group of steps).

    token:  FP8 keys 1.0, k scale proportional to t + 1;
    stairs: FP8 keys 448 in the first n(t) dims and 0 in the rest, n(t)
            rising by one every 47 tokens, under a per-tensor scale;
    bf16:   BF16 keys proportional to t + 1."""
    p = inp.problem
    D = p.head_dim
    inp.q.fill_(1.0)
    x = 16 if p.kv_dtype == "fp8" else 8
    kc = (inp.k_cache if p.kv_dtype == "fp8" else inp.k_cache.view(torch.int16))
    kc = kc.view(p.num_pages, p.num_kv_heads, D // x, p.page_size, x)
    ln2 = float(np.log(2.0))
    per_unit = D * p.scale  # logit (natural) of key value 1 in every dim at scale 1
    for s in range(p.num_seqs):
        if int(inp.context_lens[s]) == 0:
            continue
        t, pid, slot = _token_index(inp, s)
        c = 0.1 * ln2 / per_unit
        if mode == "token":
            kc[pid, :, :, slot, :] = 0x38  # 1.0 in e4m3fn
            inp.k_scale[pid, :, slot] = (c * (t + 1).float())[:, None]
        elif mode == "stairs":
            n = torch.clamp(t // 47, max=D)
            codes = torch.where(torch.arange(D)[None, :] < n[:, None], 0x7E, 0).to(torch.uint8)  # 448 or 0
            kc[pid, :, :, slot, :] = codes.view(-1, D // 16, 16)[:, None]
            inp.k_scale.fill_(47 * c * D / 448.0)  # one more dim of 448: +4.7 in base 2
        else:
            vals = (c * (t + 1).float()).to(torch.bfloat16).view(torch.int16)
            kc[pid, :, :, slot, :] = vals[:, None, None, None]


def _ramp_vscales(inp):
    """Per-token V scales times 2^(t / 60) (2^100 at t = 6000); returns the
    largest multiplier of each sequence."""
    big = []
    for s in range(inp.problem.num_seqs):
        L = int(inp.context_lens[s])
        big.append(2.0 ** ((L - 1) / 60) if L > 0 else 1.0)
        if L == 0:
            continue
        t, pid, slot = _token_index(inp, s)
        inp.v_scale[pid, :, slot] *= torch.exp2(t.double() / 60).float()[:, None]
    return np.array(big)


CASES = [
    # name, query_len, Hq, Hkv, D, page, kv dtype, scale mode, key ramp
    ("tile16-token", 1, 16, 1, 128, 16, "fp8", "token", "token"),
    ("tile16-stairs", 1, 16, 1, 128, 64, "fp8", "tensor", "stairs"),
    ("stream32-token", 2, 16, 1, 128, 64, "fp8", "token", "token"),
    ("stream32-stairs", 2, 16, 1, 128, 16, "fp8", "tensor", "stairs"),
    ("stream64-token", 4, 16, 1, 128, 128, "fp8", "token", "token"),
    ("stream64-token-p16", 4, 16, 1, 128, 16, "fp8", "token", "token"),
    ("stream64-stairs", 4, 16, 1, 128, 128, "fp8", "tensor", "stairs"),
    ("d256-stairs", 4, 16, 2, 256, 64, "fp8", "tensor", "stairs"),
    ("d256-stream-token", 4, 16, 2, 256, 64, "fp8", "token", "token"),
    ("d256-stream-token-p16", 3, 16, 2, 256, 16, "fp8", "token", "token"),
    ("d256-token", 1, 8, 1, 256, 16, "fp8", "token", "token"),
    ("bf16-keys", 1, 8, 1, 128, 16, "bf16", "none", "bf16"),
    ("d64-token", 4, 16, 1, 64, 64, "fp8", "token", "token"),
    ("d512-token", 2, 16, 1, 512, 64, "fp8", "token", "token"),
    ("d512-stairs", 1, 8, 1, 512, 128, "fp8", "tensor", "stairs"),
    ("d64-bf16-keys", 2, 16, 1, 64, 16, "bf16", "none", "bf16"),
    ("bf16-keys-64rows", 4, 16, 1, 128, 128, "bf16", "none", "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_climbing_logits(case):
    name, ql, hq, hkv, d, page, kv, scale, ramp = case
    inp = W.make_dense_case(500 + len(name), LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                            page_size=page, kv_dtype=kv, scale_mode=scale, fill="context", name=name)
    _ramp_keys(inp, ramp)
    ref = O.attend(inp)
    for kw in (dict(cu_count=4, max_partitions=1), dict(cu_count=64)):
        announce(f"climbing logits {name} {kw}")
        got, _ = run(inp, **kw)
        compare(got, ref, f"{name} {kw}")


@pytest.mark.parametrize("ql,page,d", [(4, 128, 128), (2, 64, 128), (1, 16, 128), (4, 64, 256), (4, 16, 256)])
def test_climbing_v_scales(ql, page, d):
    """Per-token V scales climbing to 2^100 (the V-scale band of the tile
    kernel and the clamped V exponent of the streaming kernel restart again
    and again); each (row, head) output is compared after dividing both
    sides by the largest magnitude of the oracle's output for it."""
    hkv = 1 if d == 128 else 2  # head dim 256: 32 rows per KV head (the streaming kernel's one row block)
    inp = W.make_dense_case(560 + ql + page + d, LENS, query_len=ql, num_q_heads=16, num_kv_heads=hkv, head_dim=d,
                            page_size=page, scale_mode="token", fill="context", name="vramp")
    _ramp_vscales(inp)
    ref = O.attend(inp)
    big = np.abs(ref).max(axis=2, keepdims=True)  # each (row, head) normalised to a largest magnitude of 1
    big[big == 0] = 1.0
    ref = ref / big
    for kw in (dict(cu_count=4, max_partitions=1), dict(cu_count=64)):
        announce(f"climbing V scales d={d} rows={16 * ql // hkv} page={page} {kw}")
        got, _ = run(inp, **kw)
        compare(got / big, ref, f"V-scale ramp d={d} rows={16 * ql // hkv} {kw}")
