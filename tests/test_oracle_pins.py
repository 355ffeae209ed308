"""Pins of the CPU oracle against things other than itself.

* the FP8/BF16/FP16 decoders against the format definitions (OCP OFP8 spec
  values in tests/golden) and against torch/numpy library conversions;
* the full computation against a dense brute force with an explicit mask in
  long double, over lengths/query lengths/windows/pages/layouts/scales/sinks;
* invariants of attention (one visible token, uniform keys, window 1, split
  and merge, page permutation, sinks, power-of-two V scales, zero queries);
* a cross-check of the unmasked single-row case against torch's float64
  scaled_dot_product_attention.
"""

from __future__ import annotations

import dataclasses
import itertools
import math
import os

import numpy as np
import pytest
import torch

import bruteforce
from oracle import oracle as O
from paged_attention_decode_plan_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_fp8():
    rows = []
    with open(os.path.join(GOLDEN, "fp8_e4m3fn_spec.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            c, v = line.split()
            rows.append((int(c, 16), float(v)))
    return rows


def test_fp8_spec_values():
    for code, val in _golden_fp8():
        got = O.fp8_value(code)
        if math.isnan(val):
            assert math.isnan(got), hex(code)
        else:
            assert got == val and math.copysign(1, got) == math.copysign(1, val), hex(code)


def test_fp8_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([O.fp8_value(c) for c in range(256)])
    nan = np.isnan(ref)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == ref[~nan]).all()
    # monotone over positive finite codes, symmetric in sign
    pos = got[:0x7F]
    assert (np.diff(pos) > 0).all()
    assert (got[0x80:0xFF] == -got[:0x7F]).all()


def test_bf16_fp16_decoders():
    bits = np.arange(0, 65536, 7, dtype=np.uint32)
    ref16 = bits.astype(np.uint16).view(np.float16).astype(np.float64)
    got16 = np.array([O.fp16_value(int(b)) for b in bits])
    nan = np.isnan(ref16)
    assert (np.isnan(got16) == nan).all() and (got16[~nan] == ref16[~nan]).all()
    refb = torch.from_numpy(bits.astype(np.uint16).view(np.int16)).view(torch.bfloat16).double().numpy()
    gotb = np.array([O.bf16_value(int(b)) for b in bits])
    nanb = np.isnan(refb)
    assert (np.isnan(gotb) == nanb).all() and (gotb[~nanb] == refb[~nanb]).all()


LENS = [0, 1, 2, 15, 16, 17, 33]


@pytest.mark.parametrize("page", [16, 64])
@pytest.mark.parametrize("vt", [False, True])
@pytest.mark.parametrize("scale", ["tensor", "token", "bf16"])
@pytest.mark.parametrize("sinks", [False, True])
def test_oracle_vs_bruteforce(page, vt, scale, sinks):
    kv = "bf16" if scale == "bf16" else "fp8"
    sm = "none" if scale == "bf16" else scale
    seed = hash((page, vt, scale, sinks)) & 0xFFFF
    for ql, w in itertools.product([1, 2, 3, 4], [0, 1, 2, 17]):
        inp = W.make_dense_case(seed + 97 * ql + w, LENS, query_len=ql, num_q_heads=4, num_kv_heads=2, head_dim=32
                                if kv == "fp8" else 16, page_size=page, kv_dtype=kv, v_transposed=vt, scale_mode=sm,
                                sliding_window=w, has_sinks=sinks, poison=False, fill="context")
        got = O.attend(inp, nthreads=2).astype(np.float64)
        ref = bruteforce.attend(inp)
        np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7, err_msg=f"ql={ql} w={w}")


def test_oracle_vs_bruteforce_token_table():
    inp = W.config_sparse(num_rows=3, selected=40, pool_pages=8)
    got = O.attend(inp).astype(np.float64)
    ref = bruteforce.attend(inp)
    np.testing.assert_allclose(got, ref, rtol=1e-6, atol=1e-7)


def test_oracle_ignores_poison():
    """Poisoned (NaN) tails, windows and stale table entries never reach it."""
    inp = W.make_dense_case(5, [17, 40, 3], query_len=2, num_q_heads=4, num_kv_heads=1, head_dim=32, page_size=16,
                            scale_mode="token", sliding_window=9, poison=True)
    out = O.attend(inp)
    assert np.isfinite(out).all()
    clean = W.make_dense_case(5, [17, 40, 3], query_len=2, num_q_heads=4, num_kv_heads=1, head_dim=32, page_size=16,
                              scale_mode="token", sliding_window=9, poison=False)
    np.testing.assert_array_equal(out, O.attend(clean))


def _case(**kw):
    base = dict(query_len=1, num_q_heads=4, num_kv_heads=2, head_dim=32, page_size=16, poison=False, fill="context")
    base.update(kw)
    return base


def _logical_v(inp, s, t, g):
    K, V = bruteforce.logical_caches(inp)
    p = inp.problem
    page = int(inp.block_tables[s, t // p.page_size])
    return V[page, g, t % p.page_size]


def test_invariant_single_token():
    inp = W.make_dense_case(11, [1, 1], **_case(scale_mode="token"))
    out = O.attend(inp)
    for s in range(2):
        for h in range(4):
            np.testing.assert_array_equal(out[s, h], _logical_v(inp, s, 0, h // 2).astype(np.float32))


def test_invariant_window_one():
    ql = 3
    inp = W.make_dense_case(12, [9, 40], **_case(query_len=ql, sliding_window=1, scale_mode="tensor"))
    out = O.attend(inp)
    for s, L in enumerate([9, 40]):
        for i in range(ql):
            pos = L - ql + i
            for h in range(4):
                np.testing.assert_array_equal(out[s * ql + i, h], _logical_v(inp, s, pos, h // 2).astype(np.float32))


def test_invariant_uniform_keys_and_zero_query():
    inp = W.make_dense_case(13, [37, 5], **_case(scale_mode="tensor"))
    inp.q.zero_()
    out = O.attend(inp)
    assert np.isfinite(out).all()
    for s, L in enumerate([37, 5]):
        for h in range(4):
            mean = np.mean([_logical_v(inp, s, t, h // 2) for t in range(L)], axis=0)
            np.testing.assert_allclose(out[s, h], mean, rtol=1e-6, atol=1e-7)


@pytest.mark.parametrize("window", [0, 7])
def test_invariant_split_merge(window):
    inp = W.make_dense_case(14, [70], **_case(query_len=2, sliding_window=window, scale_mode="token", has_sinks=True))
    full = O.attend(inp)
    rng = np.random.default_rng(0)
    for i in range(2):
        for h in range(4):
            cuts = np.sort(rng.choice(np.arange(1, 70), size=3, replace=False))
            bounds = [0, *cuts.tolist(), 70]
            parts = [O.partial(inp, 0, i, h, a, b) for a, b in zip(bounds[:-1], bounds[1:])]
            merged = O.merge([p[0] for p in parts], [p[1] for p in parts], np.stack([p[2] for p in parts]),
                             sink=float(inp.sinks[h]))
            np.testing.assert_allclose(merged, full[i, h], rtol=1e-6, atol=1e-7)


def test_invariant_page_permutation():
    inp = W.make_dense_case(15, [50, 33], **_case(page_size=16, scale_mode="token", extra_pages=0))
    out = O.attend(inp)
    p = inp.problem
    perm = torch.randperm(p.num_pages, generator=torch.Generator().manual_seed(3))
    inv = torch.argsort(perm)
    # new physical page j holds old page perm[j]; tables map old id -> new id
    inp.k_cache = inp.k_cache[perm].contiguous()
    inp.v_cache = inp.v_cache[perm].contiguous()
    inp.k_scale = inp.k_scale[perm].contiguous()
    inp.v_scale = inp.v_scale[perm].contiguous()
    inp.block_tables = inv[inp.block_tables.long()].to(torch.int32)
    np.testing.assert_array_equal(O.attend(inp), out)


def test_invariant_sinks():
    base = W.make_dense_case(16, [30], **_case(scale_mode="tensor", has_sinks=True))
    nos = W.make_dense_case(16, [30], **_case(scale_mode="tensor", has_sinks=False))
    out_nos = O.attend(nos).astype(np.float64)
    base.sinks.fill_(-1e30)
    np.testing.assert_allclose(O.attend(base), out_nos, rtol=1e-6, atol=1e-7)
    for sink in [-3.0, 0.5, 4.0, 40.0]:
        base.sinks.fill_(sink)
        out = O.attend(base).astype(np.float64)
        for h in range(4):
            m, l, _ = O.partial(nos, 0, 0, h, 0, 1 << 30)
            M = max(m, sink)
            frac = l * math.exp(m - M) / (l * math.exp(m - M) + math.exp(sink - M))
            np.testing.assert_allclose(out[0, h], out_nos[0, h] * frac, rtol=1e-5, atol=1e-7)


def test_invariant_pow2_vscale():
    inp = W.make_dense_case(17, [45, 3], **_case(scale_mode="token"))
    out = O.attend(inp)
    inp.v_scale.mul_(8.0)
    np.testing.assert_array_equal(O.attend(inp), out * 8.0)


def test_empty_and_negative_rows_are_zero():
    inp = W.make_dense_case(18, [0, 2, 1], **_case(query_len=4))
    out = O.attend(inp)
    assert (out[0:4] == 0).all()  # empty sequence
    assert (out[4:6] == 0).all()  # L=2, rows 0,1 have pos < 0
    assert (out[6:8] != 0).any(axis=-1).all()
    assert (out[8:11] == 0).all() and (out[11] != 0).any()


def test_single_row_matches_sdpa():
    inp = W.make_dense_case(19, [77, 20], **_case(kv_dtype="bf16", scale_mode="none", num_q_heads=2, num_kv_heads=2))
    out = O.attend(inp).astype(np.float64)
    K, V = bruteforce.logical_caches(inp)
    for s, L in enumerate([77, 20]):
        pages = inp.block_tables[s, np.arange(L) // 16].long().numpy()
        offs = np.arange(L) % 16
        for h in range(2):
            k = torch.from_numpy(K[pages, h, offs])[None, None]
            v = torch.from_numpy(V[pages, h, offs])[None, None]
            q = inp.q[s, h].double()[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[0, 0, 0].numpy()
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-6, atol=1e-7)


def test_planted_token_digits():
    """A token whose key dominates by a wide margin: the output is exactly its
    (integer-valued) V row."""
    inp = W.make_dense_case(20, [100], **_case(kv_dtype="bf16", scale_mode="none", num_q_heads=1, num_kv_heads=1,
                                               head_dim=16))
    p = inp.problem
    target = 57
    qv = torch.ones(16)
    inp.q[0, 0] = qv.to(torch.bfloat16)
    x = 8
    kc = inp.k_cache.view(p.num_pages, 1, 16 // x, 16, x)
    vc = inp.v_cache.view(p.num_pages, 1, 16, 16)
    for t in range(100):
        page = int(inp.block_tables[0, t // 16])
        slot = t % 16
        val = 64.0 if t == target else -64.0
        kc[page, 0, :, slot, :] = val
        vc[page, 0, :, slot] = torch.tensor([(page + d) % 16 for d in range(16)], dtype=torch.bfloat16)
    out = O.attend(inp)
    page = int(inp.block_tables[0, target // 16])
    np.testing.assert_array_equal(out[0, 0], np.array([(page + d) % 16 for d in range(16)], np.float32))


@pytest.mark.parametrize("page", [16, 64])
def test_oracle_vs_bruteforce_non_causal(page):
    """Multi-token rows without the causal mask (every row at position L - 1)."""
    for ql, w in itertools.product([2, 4], [0, 1, 17]):
        inp = W.make_dense_case(700 + 13 * ql + w + page, LENS, query_len=ql, num_q_heads=4, num_kv_heads=2,
                                head_dim=32, page_size=page, scale_mode="token", sliding_window=w, causal=False,
                                poison=False, fill="context")
        got = O.attend(inp, nthreads=2).astype(np.float64)
        np.testing.assert_allclose(got, bruteforce.attend(inp), rtol=1e-6, atol=1e-7, err_msg=f"ql={ql} w={w}")
        # all rows of one (sequence, head) see the same tokens: equal queries give equal outputs
        p = inp.problem
        q = inp.q.view(p.num_seqs, ql, p.num_q_heads, p.head_dim)
        q[:, 1:] = q[:, :1]
        out = O.attend(inp, nthreads=2).reshape(p.num_seqs, ql, p.num_q_heads, p.head_dim)
        np.testing.assert_array_equal(out[:, 1:], np.broadcast_to(out[:, :1], out[:, 1:].shape))


@pytest.mark.parametrize("page", [16, 64])
def test_oracle_vs_bruteforce_fp16_queries(page):
    """FP16 queries (decoded exactly by both sides) over the same sweep of
    lengths, query lengths and windows, with per-token and per-tensor FP8
    caches and sinks."""
    for (ql, w), scale in itertools.product(itertools.product([1, 2, 4], [0, 1, 17]), ["tensor", "token"]):
        inp = W.make_dense_case(800 + 7 * ql + w + page + (scale == "token"), LENS, query_len=ql, num_q_heads=4,
                                num_kv_heads=2, head_dim=32, page_size=page, q_dtype="fp16", scale_mode=scale,
                                sliding_window=w, has_sinks=True, poison=False, fill="context")
        assert inp.q.dtype == torch.float16
        got = O.attend(inp, nthreads=2).astype(np.float64)
        np.testing.assert_allclose(got, bruteforce.attend(inp), rtol=1e-6, atol=1e-7, err_msg=f"ql={ql} w={w}")


@pytest.mark.parametrize("token_table", [False, True])
def test_clamped_lengths(token_table):
    """Context lengths below 0 count as 0 and lengths past the table's
    capacity (table_stride pages, or table_stride slots for token tables)
    count as that capacity: against the brute force, and identical to the
    oracle on the clamped lengths."""
    if token_table:
        inp = W.config_sparse(num_rows=4, selected=40, pool_pages=8)
        cap = inp.problem.table_stride
    else:
        inp = W.make_dense_case(21, [40, 17, 5, 33], **_case(query_len=2, scale_mode="token", table_slack=0))
        cap = inp.problem.table_stride * inp.problem.page_size
        assert cap < 100
    lens = torch.tensor([-7, cap + 1, -1, 1 << 30], dtype=torch.int32)
    wild = dataclasses.replace(inp, context_lens=lens)
    tame = dataclasses.replace(inp, context_lens=torch.tensor([0, cap, 0, cap], dtype=torch.int32))
    got = O.attend(wild, nthreads=2)
    np.testing.assert_allclose(got.astype(np.float64), bruteforce.attend(wild), rtol=1e-6, atol=1e-7)
    np.testing.assert_array_equal(got, O.attend(tame, nthreads=2))
    ql = inp.problem.query_len
    assert (got[0:ql] == 0).all() and (got[2 * ql:3 * ql] == 0).all()
    assert np.isfinite(got).all() and (got[ql:2 * ql] != 0).any()


def _mutants(inp):
    """The oracle's output with one plausible mistake planted: (name, output)."""
    p = inp.problem
    out = []
    out.append(("causal bound + 1", bruteforce.attend(inp, pos_shift=1)))
    if p.sliding_window > 0:
        out.append(("window + 1", bruteforce.attend(inp, window_shift=1)))
    if p.scale_mode == "token":
        for name in ("k_scale", "v_scale"):
            m = dataclasses.replace(inp, **{name: torch.roll(getattr(inp, name), 1, dims=2).contiguous()})
            out.append((f"{name} one slot off", O.attend(m, nthreads=2)))
    bt = inp.block_tables.clone()
    bt[:, 0] = inp.block_tables[:, 1]  # every sequence's first page replaced by its second
    out.append(("first page id", O.attend(dataclasses.replace(inp, block_tables=bt), nthreads=2)))
    return out


@pytest.mark.parametrize("scale,window", [("token", 0), ("token", 17), ("tensor", 257)])
def test_tolerance_detects_planted_mistakes(scale, window):
    """On inputs of the GPU parity matrix's kind (the same lengths, MTP rows,
    GQA and N(0,1) data), each planted mistake -- a causal bound shifted by
    one, a window one token longer, per-token K or V scales misplaced by one
    slot, a wrong page id -- moves some output by at least ten times the
    parity tolerance and puts at least 16 outputs outside it, so atol = rtol
    = 0.005 cannot hide them (the pages report differences of 0.13 or more
    for such mistakes in their cases, aiter PR #7079 test list; here a
    window one token longer than 257 moves outputs by about 0.1)."""
    inp = W.make_dense_case(900 + window, [0, 1, 2, 15, 17, 150, 300, 1000], query_len=4, num_q_heads=16,
                            num_kv_heads=1, head_dim=128, page_size=16, scale_mode=scale, sliding_window=window,
                            poison=False, fill="context")
    ref = O.attend(inp, nthreads=4).astype(np.float64)
    for name, got in _mutants(inp):
        err = np.abs(np.asarray(got, np.float64) - ref)
        excess = err - (0.005 + 0.005 * np.abs(ref))
        assert err.max() >= 0.05, (name, float(err.max()))
        assert (excess > 0).sum() >= 16, (name, int((excess > 0).sum()))


def test_oracle_two_level_topk():
    """Top-k logical positions through the block table (token_table 2):
    against the brute force on a small case (positions past the table's
    extent and below 0 clamp to it), and bit-identical to the same call with
    the positions resolved to physical slots on the host."""
    small = W.config_sparse_topk(num_rows=3, selected=40, pool_pages=8)
    np.testing.assert_allclose(O.attend(small).astype(np.float64), bruteforce.attend(small), rtol=1e-6, atol=1e-7)
    wild = dataclasses.replace(small, topk_indices=small.topk_indices.clone())
    wild.topk_indices[0, :3] = torch.tensor([-5, 1 << 20, 8 * 16], dtype=torch.int32)
    np.testing.assert_allclose(O.attend(wild).astype(np.float64), bruteforce.attend(wild), rtol=1e-6, atol=1e-7)
    full = W.config_sparse_topk()
    sel = [(r, h) for r in range(0, 64, 9) for h in (0, 7, 15)]
    np.testing.assert_array_equal(O.attend(full, sel=sel), O.attend(W.resolve_topk(full), sel=sel))
