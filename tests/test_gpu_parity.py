"""GPU parity: libpa.so against the CPU oracle, element by element, within
atol = rtol = 0.005 (the FP32-reference tolerance of the FlyDSL D256 decode
page, aiter PR #6617, Validation), on seeded inputs with NaN-poisoned output
and workspace before every call."""

from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run, to_device
from oracle import oracle as O
from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

LENS = [0, 1, 2, 15, 17, 150, 300, 1000]


def _parity(inp, sel=None, **plan_kw):
    got, plan = run(inp, **plan_kw)
    if sel is None:
        ref = O.attend(inp)
        return compare(got, ref, inp.name), plan
    ref = O.attend(inp, sel=sel)
    g = np.stack([got[r, h] for r, h in sel])
    return compare(g, ref, inp.name), plan


@pytest.mark.parametrize("vt", [False, True])
@pytest.mark.parametrize("maxp", [1, 0])
def test_tiny(vt, maxp):
    inp = W.config_tiny(v_transposed=vt)
    announce(f"tiny vt={vt} maxp={maxp}")
    err, plan = _parity(inp, max_partitions=maxp)
    if maxp == 1:
        assert plan.info().num_slots == 0


@pytest.mark.parametrize("page", [16, 32, 64, 128])
@pytest.mark.parametrize("vt", [False, True])
@pytest.mark.parametrize("scale", ["tensor", "token"])
def test_matrix_fp8(page, vt, scale):
    seed = 1000 + page * 4 + vt * 2 + (scale == "token")
    for ql, window, sinks, (hq, hkv) in itertools.product([1, 2, 3, 4], [0, 1, 17, 257], [False, True],
                                                          [(8, 1), (16, 1), (8, 2)]):
        if (ql + window + hq) % 3 != seed % 3 and not (ql == 4 and hq == 16):
            continue  # a deterministic third of the product, plus every 64-row case
        inp = W.make_dense_case(seed, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                page_size=page, v_transposed=vt, scale_mode=scale, sliding_window=window,
                                has_sinks=sinks)
        announce(f"fp8 page={page} vt={vt} scale={scale} ql={ql} w={window} sinks={sinks} hq={hq} hkv={hkv}")
        _parity(inp, cu_count=64)
        seed += 1


@pytest.mark.parametrize("page", [16, 32, 64, 128])
def test_matrix_bf16(page):
    seed = 2000 + page
    for ql, window, sinks, vt, (hq, hkv) in itertools.product([1, 4], [0, 17], [False, True], [False, True],
                                                              [(8, 1), (16, 1)]):
        inp = W.make_dense_case(seed, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=128,
                                page_size=page, kv_dtype="bf16", v_transposed=vt, sliding_window=window,
                                has_sinks=sinks)
        announce(f"bf16 page={page} vt={vt} ql={ql} w={window} sinks={sinks} hq={hq}")
        _parity(inp, cu_count=64)
        seed += 1


@pytest.mark.parametrize("kv,scale", [("fp8", "tensor"), ("fp8", "token"), ("bf16", "none")])
@pytest.mark.parametrize("page", [16, 32, 64, 128])
def test_d64(kv, scale, page):
    """Head dim 64 in every scale mode (FP8 caches with per-tensor and
    per-token scales, BF16 caches): 8 to 64 rows per KV head, windows,
    sinks, plain and transposed V, BF16 and FP16 queries."""
    seed = 4000 + page + 7 * (scale == "token") + 13 * (kv == "bf16")
    cases = [(1, 8, 1, 0, False, False, "bf16"), (2, 16, 2, 17, True, True, "fp16"), (4, 16, 2, 0, False, True, "bf16"),
             (4, 16, 1, 257, True, False, "bf16"), (3, 8, 1, 1, False, False, "fp16")]
    for ql, hq, hkv, window, sinks, vt, qd in cases:
        if kv == "bf16":
            qd = "bf16"  # BF16 caches take BF16 queries
        inp = W.make_dense_case(seed, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=64,
                                page_size=page, kv_dtype=kv, q_dtype=qd, v_transposed=vt, scale_mode=scale,
                                sliding_window=window, has_sinks=sinks)
        announce(f"d64 {kv} {scale} page={page} ql={ql} hq={hq} hkv={hkv} w={window} sinks={sinks} vt={vt} q={qd}")
        _parity(inp, cu_count=64)
        seed += 1


@pytest.mark.parametrize("scale", ["tensor", "token"])
@pytest.mark.parametrize("page", [16, 64, 128, 256])
def test_d512(scale, page):
    """Head dim 512 (FP8 caches: the one-stage tile pipeline): 8 to 64 rows
    per KV head, windows, sinks, plain and transposed V, BF16 and FP16
    queries, one and several partitions (the reducer at 512 dims)."""
    seed = 4500 + page + 7 * (scale == "token")
    lens = [0, 1, 127, 129, 700, 3000]
    cases = [(1, 8, 1, 0, False, False, "bf16"), (2, 16, 2, 17, True, True, "fp16"), (4, 16, 2, 0, False, True, "bf16"),
             (4, 16, 1, 257, True, False, "bf16")]
    for ql, hq, hkv, window, sinks, vt, qd in cases:
        inp = W.make_dense_case(seed, lens, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=512,
                                page_size=page, q_dtype=qd, v_transposed=vt, scale_mode=scale,
                                sliding_window=window, has_sinks=sinks)
        announce(f"d512 {scale} page={page} ql={ql} hq={hq} hkv={hkv} w={window} sinks={sinks} vt={vt} q={qd}")
        _parity(inp, cu_count=64)
        _parity(inp, cu_count=4, max_partitions=1, stage_limit=3)
        seed += 1


LARGE_PAGE_CASES = [
    # name, query_len, Hq, Hkv, D, kv dtype, scale mode, window, sinks, transposed V
    ("tile16-fp8", 1, 16, 4, 128, "fp8", "token", 257, True, False),
    ("stream64-fp8", 4, 16, 1, 128, "fp8", "token", 0, False, False),
    ("stream32-fp8", 2, 16, 1, 128, "fp8", "tensor", 300, True, True),
    ("d256-stream", 4, 16, 2, 256, "fp8", "tensor", 8193, False, True),
    ("d256-tile", 2, 16, 2, 256, "fp8", "token", 0, True, False),
    ("d64-tile", 4, 16, 1, 64, "fp8", "token", 17, False, True),
    ("bf16-64rows", 4, 16, 1, 128, "bf16", "none", 0, False, False),
]


@pytest.mark.parametrize("page", [256, 512, 1024])
@pytest.mark.parametrize("case", LARGE_PAGE_CASES, ids=[c[0] for c in LARGE_PAGE_CASES])
def test_large_pages(page, case):
    """Pages above 128 tokens (taken as 128-token sub-pages: the page's
    block-table entry plus the sub-page's offset in K, V and the scales) in
    every decode path, both V layouts and both scale modes, with lengths
    that end inside, at and past sub-page and page edges."""
    name, ql, hq, hkv, d, kv, scale, window, sinks, vt = case
    lens = [0, 1, 127, 128, 129, page - 1, page, page + 1, 3 * page + 77, 9000]
    inp = W.make_dense_case(5000 + page + len(name), lens, query_len=ql, num_q_heads=hq, num_kv_heads=hkv,
                            head_dim=d, page_size=page, kv_dtype=kv, v_transposed=vt, scale_mode=scale,
                            sliding_window=window, has_sinks=sinks)
    announce(f"large pages {name} page={page}")
    _parity(inp, cu_count=64)
    _parity(inp, cu_count=4, max_partitions=1, stage_limit=3)


@pytest.mark.parametrize("ql,hq,hkv", [(1, 8, 1), (4, 16, 2), (4, 16, 1)])
def test_d256(ql, hq, hkv):
    seed = 3000 + ql * 10 + hq
    for page, vt, window in itertools.product([16, 64], [False, True], [0, 257]):
        inp = W.make_dense_case(seed, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=256,
                                page_size=page, v_transposed=vt, scale_mode="tensor", sliding_window=window)
        announce(f"d256 page={page} vt={vt} ql={ql} w={window} hq={hq} hkv={hkv}")
        _parity(inp, cu_count=64)
        seed += 1


@pytest.mark.parametrize("ql,hq,hkv,d,page,scale", [(2, 16, 2, 128, 16, "token"), (4, 16, 1, 128, 128, "token"),
                                                    (2, 16, 1, 128, 64, "token"), (3, 8, 1, 128, 16, "tensor"),
                                                    (4, 16, 2, 256, 64, "tensor")])
def test_fp16_queries(ql, hq, hkv, d, page, scale):
    """FP16 queries in every decode path: the 16-row tile kernel, the
    streaming kernel with two row blocks (64 rows) and one (32 and 24 rows,
    pages of 64 and 16), and the D256 tile kernel."""
    inp = W.make_dense_case(41 + ql + d + page, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                            page_size=page, q_dtype="fp16", scale_mode=scale, sliding_window=17, has_sinks=True)
    announce(f"fp16 queries ql={ql} hq={hq} hkv={hkv} d={d} page={page} scale={scale}")
    _parity(inp, cu_count=64)


def test_many_partitions_and_fixed_partition_length():
    inp = W.make_dense_case(42, [5000, 7000, 3], query_len=4, num_q_heads=16, num_kv_heads=1, page_size=64,
                            scale_mode="token")
    announce("partition_tokens=128")
    _, plan = _parity(inp, cu_count=256, partition_tokens=128)
    assert plan.info().max_parts > 20
    announce("max_partitions=2")
    _parity(inp, cu_count=256, max_partitions=2)


def test_staging_fallback():
    """Page ids past a tiny staging bound come straight from the block table."""
    inp = W.make_dense_case(43, [3000, 900], query_len=1, num_q_heads=8, num_kv_heads=1, page_size=16,
                            scale_mode="tensor")
    for lim in [1, 7, 64]:
        announce(f"stage_limit={lim}")
        _parity(inp, cu_count=4, max_partitions=1, stage_limit=lim)


def test_device_context_longer_than_plan():
    """A plan made for shorter lengths still covers the device lengths."""
    inp = W.make_dense_case(44, [2000, 700], query_len=2, num_q_heads=8, num_kv_heads=1, page_size=16,
                            scale_mode="token", sliding_window=0)
    announce("plan lengths below device lengths")
    got, _ = run(inp, lens_for_plan=[1000, 300], cu_count=16)
    compare(got, O.attend(inp), "longer device context")


def test_run_to_run_bit_exact():
    inp = W.config_ragged()
    dev = to_device(inp)
    announce("ragged twice")
    a, plan = run(inp, dev=dev)
    b, _ = run(inp, dev=dev, plan=plan)
    assert np.array_equal(a, b)


def test_planted_token_digits_exact():
    """One token's key dominates; the output must equal its integer V digits
    exactly, wherever the token sits (page / tile / partition / staged-bound /
    window edges).  4, 16, 32 and 64 rows: the tile kernel and both row-block
    counts of the streaming kernel, where a token after the first step of a
    wave exceeds its reference by 522 (base 2) and forces a restart."""
    page, L = 16, 700
    for ql, window, target_off in [(1, 0, None), (4, 0, None), (1, 33, None), (8, 0, None), (16, 0, None)]:
        base = W.make_dense_case(45, [L], query_len=ql, num_q_heads=4, num_kv_heads=1, head_dim=128, page_size=page,
                                 scale_mode="tensor", sliding_window=window, poison=True, fill="context")
        p = base.problem
        base.k_scale.fill_(1.0)
        base.v_scale.fill_(1.0)
        base.q.fill_(1.0)
        kc = base.k_cache.view(p.num_pages, 1, 128 // 16, page, 16)
        vc = base.v_cache.view(p.num_pages, 1, 128, page)
        lo = max(0, L - ql - window + 1) if window else 0
        targets = sorted({lo, lo + 1, 127, 128, 129, 255, 256, 511, 512, L - ql, L - ql - 1} & set(range(lo, L - ql + 1)))
        for tgt in targets:
            pos_code = 0x58  # +16.0 in e4m3fn
            neg_code = 0xD8  # -16.0
            for t in range(lo, L):
                pid = int(base.block_tables[0, t // page])
                kc[pid, 0, :, t % page, :] = pos_code if t == tgt else neg_code
                digits = torch.tensor([((pid * 7 + d) % 16) for d in range(128)], dtype=torch.float32)
                vc[pid, 0, :, t % page] = W.to_fp8_bytes(digits)
            announce(f"planted ql={ql} w={window} target={tgt}")
            for kw in [dict(cu_count=4, max_partitions=1, stage_limit=5), dict(cu_count=256, partition_tokens=128)]:
                got, _ = run(base, **kw)
                pid = int(base.block_tables[0, tgt // page])
                want = np.array([((pid * 7 + d) % 16) for d in range(128)], np.float32)
                for i in range(ql):
                    pos = L - ql + i
                    vis_lo = max(0, pos - window + 1) if window else 0
                    if vis_lo <= tgt <= pos:
                        for h in range(4):
                            assert np.array_equal(got[i, h], want), (tgt, i, h, kw)


def test_uniform_attention_census():
    """K = 0 and one-hot V rows: out[d] * |visible| counts visible t with t mod D == d."""
    L, page = 333, 64
    inp = W.make_dense_case(46, [L], query_len=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=page,
                            kv_dtype="bf16", poison=True, fill="context")
    p = inp.problem
    kc = inp.k_cache.view(torch.int16).view(p.num_pages, 1, 16, page, 8)
    vc = inp.v_cache.view(torch.int16).view(p.num_pages, 1, 128, page)
    one = torch.tensor([1.0], dtype=torch.bfloat16).view(torch.int16)[0]
    for t in range(L):
        pid = int(inp.block_tables[0, t // page])
        kc[pid, 0, :, t % page, :] = 0
        vc[pid, 0, :, t % page] = 0
        vc[pid, 0, t % 128, t % page] = one
    announce("census")
    got, _ = run(inp, cu_count=16, partition_tokens=128)
    counts = np.bincount(np.arange(L) % 128, minlength=128)
    np.testing.assert_allclose(got[0] * L, np.broadcast_to(counts, (8, 128)), rtol=0.004, atol=0.0)


@pytest.mark.parametrize("page", [64, 128])
@pytest.mark.parametrize("ql", [4, 2])
def test_wide_scales_stream_rows(page, ql):
    """FP8 items of 64 and 32 rows (the streaming kernel): queries of magnitude 2^24 with per-token k scales
    2^24 smaller (the whole-item power-of-two rescaling of the query, folded
    back into the logits), and V scales 2^30 larger (the clamped V exponent
    and its overflow restart), against the oracle.  The output is linear in
    the V scales, so the second case is compared after dividing both sides
    by 2^30: the absolute part of the tolerance keeps its meaning."""
    for name, qmul, kmul, vmul in [("q x 2^24, k scales x 2^-24", 2.0**24, 2.0**-24, 1.0),
                                   ("v scales x 2^30", 1.0, 1.0, 2.0**30)]:
        inp = W.make_dense_case(48 + page + ql, LENS, query_len=ql, num_q_heads=16, num_kv_heads=1, head_dim=128,
                                page_size=page, scale_mode="token")
        inp.q.mul_(qmul)
        real = inp.k_scale < 1e29  # poisoned slots keep their poison
        inp.k_scale[real] *= kmul
        real = inp.v_scale < 1e29
        inp.v_scale[real] *= vmul
        announce(f"wide scales page={page} rows={16 * ql}: {name}")
        got, _ = run(inp, cu_count=64)
        compare(got / vmul, O.attend(inp) / vmul, name)


@pytest.mark.parametrize("page", [16, 64, 128])
@pytest.mark.parametrize("ql,hq", [(4, 16), (3, 8)])
def test_stream_kernel_run_to_run_bit_exact(page, ql, hq):
    """FP8 items of 64 rows (the streaming kernel's two row blocks) and of 24
    rows (one row block, 8 padding rows), several partitions per sequence
    merged in partition order: against the oracle, and two calls with one
    plan give identical bytes."""
    inp = W.make_dense_case(60 + page + ql, [5000, 3, 0, 1, 2600, 700], query_len=ql, num_q_heads=hq,
                            num_kv_heads=1, head_dim=128, page_size=page, scale_mode="token", sliding_window=0,
                            has_sinks=True)
    dev = to_device(inp)
    announce(f"stream kernel twice page={page} rows={ql * hq}")
    a, plan = run(inp, dev=dev, cu_count=64)
    assert plan.info().num_reduce > 0
    compare(a, O.attend(inp), "stream kernel")
    b, _ = run(inp, dev=dev, plan=plan)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("ql,hq,page", [(4, 16, 128), (2, 16, 64), (1, 8, 16)])
def test_multi_wave_plans(ql, hq, page):
    """Plans with more items than resident workgroups (long sequences on a
    small CU count, so several waves of items run through each slot), in
    the streaming kernel (64 and 32 rows) and the tile kernel (8 rows):
    against the oracle."""
    inp = W.make_dense_case(130 + ql + page, [12000, 11800, 12100, 12050, 11900], query_len=ql, num_q_heads=hq,
                            num_kv_heads=1, head_dim=128, page_size=page, scale_mode="token", sliding_window=0,
                            has_sinks=True, fill="context")
    announce(f"multi-wave plan ql={ql} hq={hq} page={page}")
    _, plan = _parity(inp, cu_count=3)
    slots = 3 * (1 if ql * hq > 16 else 2)  # resident workgroups on three CUs
    assert plan.info().num_items > slots


@pytest.mark.parametrize("ql,hq,page", [(4, 16, 128), (1, 8, 16)])
def test_pages_past_4gib(ql, hq, page):
    """Caches of more than 4 GiB (the pages' 200 000-token MI355 shape needs
    64-bit page offsets): the sequences' pages are moved to page ids whose
    byte offset in K and V is past 2^32, in the streaming (64-row) and the
    tile (8-row) kernels, against the oracle on the compact original."""
    inp = W.make_dense_case(70 + page, [3000, 700, 1], query_len=ql, num_q_heads=hq, num_kv_heads=1, head_dim=128,
                            page_size=page, scale_mode="token", sliding_window=0)
    p = inp.problem
    page_bytes = 128 * page  # FP8, one KV head
    big = (4 << 30) // page_bytes + 4 * p.num_pages  # more than 4 GiB of K (and of V)
    rng = np.random.default_rng(71)
    remap = torch.as_tensor(rng.choice(np.arange(big - 4 * p.num_pages, big), size=p.num_pages, replace=False))
    assert int(remap.min()) * page_bytes >= 1 << 32
    dev = to_device(inp)
    kb = torch.zeros((big,) + tuple(dev["k_cache"].shape[1:]), dtype=dev["k_cache"].dtype, device="cuda")
    vb = torch.zeros((big,) + tuple(dev["v_cache"].shape[1:]), dtype=dev["v_cache"].dtype, device="cuda")
    ksb = torch.ones((big,) + tuple(dev["k_scale"].shape[1:]), dtype=torch.float32, device="cuda")
    vsb = torch.ones_like(ksb)
    rd = remap.to("cuda")
    kb[rd] = dev["k_cache"]
    vb[rd] = dev["v_cache"]
    ksb[rd] = dev["k_scale"]
    vsb[rd] = dev["v_scale"]
    bt = remap[inp.block_tables.long()].to(torch.int32).to("cuda")
    prob = B.problem_of(p)
    prob.num_pages = big
    announce(f"pages past 4 GiB ql={ql} hq={hq} page={page} ({big} pages)")
    plan = B.Plan(prob, inp.context_lens, cu_count=64).allocate("cuda")
    plan.workspace.fill_(float("nan"))
    out = torch.full_like(dev["q"], float("nan"))
    B.attend(plan, out, dev["q"], kb, vb, bt, dev["context_lens"], ksb, vsb, None)
    torch.cuda.synchronize()
    compare(out.float().cpu().numpy(), O.attend(inp), "pages past 4 GiB")
    del kb, vb, ksb, vsb
    torch.cuda.empty_cache()


@pytest.mark.parametrize("page", [64, 128])
@pytest.mark.parametrize("ql", [4, 2])
def test_stream_kernel_device_context_longer_than_plan(page, ql):
    """FP8 items of 64 and 32 rows (the streaming kernel, two and one row
    blocks) with device lengths beyond the planned ones: the open-ended last
    partition reads the page ids past the staged range from the block table."""
    inp = W.make_dense_case(80 + page + ql, [9000, 2500, 300], query_len=ql, num_q_heads=16, num_kv_heads=1,
                            head_dim=128, page_size=page, scale_mode="token", sliding_window=0)
    announce(f"stream kernel, plan lengths below device lengths page={page} rows={16 * ql}")
    got, _ = run(inp, lens_for_plan=[1000, 300, 1], cu_count=16)
    compare(got, O.attend(inp), "stream kernel, longer device context")


@pytest.mark.parametrize("kind", ["stream", "stream32", "tile"])
def test_graph_replay_with_changing_lengths(kind):
    """One pa_decode + pa_reduce captured in a HIP graph and replayed while the
    device context lengths change between replays (growing past the planned
    lengths, and shrinking): every replay against the oracle and against an
    eager call with the same lengths (bit-identical).  Works because the
    plan's last partition of every row is open-ended and nothing in a call
    allocates, uploads or clears memory once the metadata is on the device."""
    import dataclasses

    if kind == "stream":
        cfg = dict(query_len=4, num_q_heads=16, page_size=128)
    elif kind == "stream32":  # one row block
        cfg = dict(query_len=2, num_q_heads=16, page_size=64)
    else:
        cfg = dict(query_len=1, num_q_heads=8, page_size=16)
    lens_max = [6000, 2500, 900]
    inp = W.make_dense_case(90 + len(kind), lens_max, num_kv_heads=1, head_dim=128, scale_mode="token",
                            sliding_window=0, fill="context", **cfg)
    dev = to_device(inp)
    planned = [3000, 1000, 500]
    plan = B.Plan(B.problem_of(inp.problem), planned, cu_count=64).allocate("cuda")
    cl = dev["context_lens"]
    out = torch.empty_like(dev["q"])
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], cl, dev["k_scale"], dev["v_scale"], None)
    cl.copy_(torch.tensor(planned, dtype=torch.int32))
    B.attend(plan, out, *args)  # an eager call before the capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.attend(plan, out, *args)
    torch.cuda.synchronize()
    for lens in ([3000, 1000, 500], [6000, 2500, 900], [4100, 1, 0], [5000, 2000, 700]):
        announce(f"graph replay {kind} lens={lens}")
        cl.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        ref = O.attend(dataclasses.replace(inp, context_lens=torch.tensor(lens, dtype=torch.int32)))
        compare(got, ref, f"graph replay {lens}")
        eager = torch.full_like(out, float("nan"))
        B.attend(plan, eager, *args)
        torch.cuda.synchronize()
        assert np.array_equal(got, eager.float().cpu().numpy())


def _check_device_work_list(plan, inp, lens, host_max_len):
    """Structure of a device-refreshed work list: every unit's visible tiles
    covered once, in partition order, by an even split; unused items do
    nothing; partial slots distinct and inside the budget; the longest item
    no longer than the host planner's for the same lengths."""
    p = inp.problem
    n = plan.info().num_items
    items = plan.work_list_device().cpu().numpy()
    used = items[items[:, 0] >= 0]
    slots = used[used[:, 5] >= 0, 5]
    assert len(set(slots.tolist())) == len(slots) and (slots < plan.info().num_slots).all()
    longest = 0
    for s in range(p.num_seqs):
        lo, hi = W.visible_span(int(lens[s]), p.query_len, p.sliding_window, p.causal)
        t0 = (lo // p.page_size) * p.page_size
        T = -(-(hi - t0) // 128) if hi > lo else 0
        mine = used[used[:, 0] == s]
        assert len(mine) >= 1
        parts = mine[:, 7]
        assert (parts == parts[0]).all() and len(mine) == parts[0] * p.num_kv_heads
        mine = mine[np.argsort(mine[:, 6], kind="stable")]
        ends = [e if e >= 0 else T for e in mine[:, 4]]
        assert mine[0, 3] == 0 and ends[-1] == T and mine[-1, 4] == -1
        assert all(mine[i + 1, 3] == ends[i] for i in range(len(mine) - 1))
        lengths = [e - b for b, e in zip(mine[:, 3], ends)]
        assert max(lengths) - min(lengths) <= 1
        longest = max(longest, max(lengths))
    assert longest <= host_max_len


@pytest.mark.parametrize("kind", ["stream", "stream32", "tile"])
def test_device_refresh_in_graph(kind):
    """Row f2: pa_plan_refresh re-partitions a refreshable plan on the device
    from the device lengths; a graph of refresh + decode + reduce is replayed
    as the lengths change, every replay against the oracle and an eager call,
    and the refreshed work list is checked structurally."""
    import dataclasses

    if kind == "stream":
        cfg = dict(query_len=4, num_q_heads=16, page_size=128)
    elif kind == "stream32":  # one row block
        cfg = dict(query_len=2, num_q_heads=16, page_size=64)
    else:
        cfg = dict(query_len=1, num_q_heads=8, page_size=16)
    lens_max = [6000, 2500, 900, 40]
    inp = W.make_dense_case(95 + len(kind), lens_max, num_kv_heads=1, head_dim=128, scale_mode="token",
                            sliding_window=0, has_sinks=True, fill="context", **cfg)
    dev = to_device(inp)
    planned = [3000, 1000, 500, 40]
    plan = B.Plan(B.problem_of(inp.problem), planned, cu_count=64, refreshable=1).allocate("cuda")
    cl = dev["context_lens"]
    out = torch.empty_like(dev["q"])
    args = (dev["q"], dev["k_cache"], dev["v_cache"], dev["block_tables"], cl, dev["k_scale"], dev["v_scale"],
            dev["sinks"])
    cl.copy_(torch.tensor(planned, dtype=torch.int32))
    B.pa_plan_refresh(plan, cl)
    B.attend(plan, out, *args)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        B.pa_plan_refresh(plan, cl)
        B.attend(plan, out, *args)
    torch.cuda.synchronize()
    for lens in ([6000, 2500, 900, 40], [3000, 1, 0, 17], [5900, 2400, 100, 40], [200, 2500, 900, 0]):
        announce(f"device refresh {kind} lens={lens}")
        cl.copy_(torch.tensor(lens, dtype=torch.int32))
        out.fill_(float("nan"))
        plan.workspace.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        got = out.float().cpu().numpy()
        ref = O.attend(dataclasses.replace(inp, context_lens=torch.tensor(lens, dtype=torch.int32)))
        compare(got, ref, f"device refresh {lens}")
        host = B.Plan(B.problem_of(inp.problem), lens, cu_count=64)
        hw = host.work().numpy()
        host_len = 0
        for row in hw:
            s_ = int(row[0])
            lo, hi = W.visible_span(lens[s_], inp.problem.query_len, 0, True)
            t0 = (lo // inp.problem.page_size) * inp.problem.page_size
            T = -(-(hi - t0) // 128) if hi > lo else 0
            host_len = max(host_len, (row[4] if row[4] >= 0 else T) - row[3])
        _check_device_work_list(plan, inp, lens, host_len)
        eager = torch.full_like(out, float("nan"))
        B.pa_plan_refresh(plan, cl)
        B.attend(plan, eager, *args)
        torch.cuda.synchronize()
        assert np.array_equal(got, eager.float().cpu().numpy())


@pytest.mark.parametrize("kv,hq,hkv,d,page", [("fp8", 16, 1, 128, 128), ("fp8", 16, 2, 256, 64),
                                              ("bf16", 8, 1, 128, 16)])
def test_non_causal_multi_token(kv, hq, hkv, d, page):
    """Multi-token rows without the causal mask (row f3): the streaming kernel
    (32 and 64 rows), the D256 and the BF16 tile kernels, with and without a window."""
    for ql, window in [(2, 0), (4, 0), (4, 33)]:
        inp = W.make_dense_case(110 + ql + window + d, LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv,
                                head_dim=d, page_size=page, kv_dtype=kv, scale_mode="token" if kv == "fp8" else "none",
                                sliding_window=window, causal=False)
        announce(f"non-causal kv={kv} d={d} page={page} ql={ql} w={window}")
        _parity(inp, cu_count=64)


ZERO_Q_PATHS = [
    # name, query_len, Hq, Hkv, D, page, kv, scale
    ("tile16", 1, 16, 1, 128, 16, "fp8", "token"),
    ("tile8-tensor", 1, 8, 1, 128, 64, "fp8", "tensor"),
    ("stream32", 2, 16, 1, 128, 64, "fp8", "token"),
    ("stream64", 4, 16, 1, 128, 128, "fp8", "token"),
    ("stream64-p16-tensor", 4, 16, 1, 128, 16, "fp8", "tensor"),
    ("d256", 4, 16, 2, 256, 64, "fp8", "tensor"),
    ("d256-token", 1, 8, 1, 256, 16, "fp8", "token"),
    ("bf16", 4, 16, 1, 128, 128, "bf16", "none"),
]


@pytest.mark.parametrize("case", ZERO_Q_PATHS, ids=[c[0] for c in ZERO_Q_PATHS])
def test_zero_query_rows(case):
    """All-zero query rows (every head of every third row, and head 5 of every
    row): the FP8 query split meets amax = 0, and the output must be the mean
    of the visible V rows with no NaN (aiter PR #4332, follow-up commit: an
    all-zero query row quantised to scale 0 turned the output into NaN)."""
    name, ql, hq, hkv, d, page, kv, scale = case
    inp = W.make_dense_case(150 + len(name), LENS, query_len=ql, num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
                            page_size=page, kv_dtype=kv, scale_mode=scale, sliding_window=17 if ql == 2 else 0,
                            has_sinks=ql == 4)
    inp.q[::3] = 0
    inp.q[:, 5] = 0
    announce(f"zero query rows {name}")
    _parity(inp, cu_count=64)
    _parity(inp, cu_count=4, max_partitions=1)


def test_zero_query_rows_token_table():
    inp = W.config_sparse(num_rows=6, selected=700, pool_pages=64)
    inp.q[::2] = 0
    inp.q[:, 3] = 0
    announce("zero query rows, token table")
    _parity(inp, cu_count=64, partition_tokens=256)


@pytest.mark.parametrize("scale", ["tensor", "token"])
@pytest.mark.parametrize("window", [0, 1, 17, 8193])
def test_d256_breadth(scale, window):
    """Head dim 256 across the pages' D256 validation axes (aiter PR #6617,
    Validation): per-tensor and per-token scales, 1-4 causal rows, windows
    0 / 1 / 17 / 8193, sinks, BF16 and FP16 queries, pages of 16 and 64,
    plain and transposed V, on lengths from 0 to past the largest window."""
    lens = [0, 1, 2, 17, 300, 9000]
    seed = 3100 + window + (scale == "token")
    for ql, page, vt in [(1, 16, True), (2, 64, False), (4, 64, True), (3, 16, False)]:
        sinks = (ql + window) % 2 == 0
        qd = "fp16" if ql % 2 == 1 else "bf16"
        inp = W.make_dense_case(seed, lens, query_len=ql, num_q_heads=16, num_kv_heads=2, head_dim=256,
                                page_size=page, q_dtype=qd, v_transposed=vt, scale_mode=scale, sliding_window=window,
                                has_sinks=sinks)
        announce(f"d256 scale={scale} w={window} ql={ql} page={page} vt={vt} sinks={sinks} q={qd}")
        _parity(inp, cu_count=64)
        seed += 1


@pytest.mark.parametrize("kind", ["tile", "stream64", "stream32", "token_table"])
def test_clamped_lengths(kind):
    """Device and planned context lengths below 0 (count as 0) and past the
    table's capacity (count as table_stride pages, or table_stride slots for
    token tables) in every kernel, against the oracle on the same lengths."""
    import dataclasses

    if kind == "token_table":
        inp = W.config_sparse(num_rows=4, selected=300, pool_pages=32)
        cap = inp.problem.table_stride
    else:
        ql = {"tile": 1, "stream64": 4, "stream32": 2}[kind]
        inp = W.make_dense_case(170 + ql, [2000, 40, 1000, 700], query_len=ql, num_q_heads=16, num_kv_heads=1,
                                page_size=64, scale_mode="token", fill="context", table_slack=0,
                                poison=False)  # the clamp makes stale table entries visible
        cap = inp.problem.table_stride * inp.problem.page_size
    lens = torch.tensor([cap + 5, -3, 1 << 30, -(1 << 30)], dtype=torch.int32)
    wild = dataclasses.replace(inp, context_lens=lens)
    announce(f"clamped lengths {kind} cap={cap}")
    got, _ = run(wild, cu_count=64)
    compare(got, O.attend(wild), f"clamped lengths {kind}")


def test_shared_meta_buffer():
    """Two plans sharing one metadata buffer: after plan B's upload, plan A is
    refused (its list is no longer there) until it uploads again; a buffer
    whose header no longer holds the plan's serial (reallocated or
    overwritten) makes the kernels do nothing, so the NaN-poisoned output
    stays untouched instead of following a foreign list."""
    inp_a = W.make_dense_case(181, [700, 300], query_len=4, num_q_heads=16, num_kv_heads=1, page_size=64,
                              scale_mode="token")
    inp_b = W.make_dense_case(182, [3000, 20, 900], query_len=1, num_q_heads=8, num_kv_heads=1, page_size=16,
                              scale_mode="tensor")
    da, db = to_device(inp_a), to_device(inp_b)
    pa = B.Plan(B.problem_of(inp_a.problem), inp_a.context_lens, cu_count=64)
    pb = B.Plan(B.problem_of(inp_b.problem), inp_b.context_lens, cu_count=64)
    buf = torch.empty(max(pa.meta_bytes, pb.meta_bytes), dtype=torch.uint8, device="cuda")
    for p_ in (pa, pb):
        p_.meta = buf
        p_.workspace = torch.full((max(p_.workspace_bytes // 4, 4),), float("nan"), device="cuda")

    def call(plan, inp, d):
        out = torch.full_like(d["q"], float("nan"))
        B.attend(plan, out, d["q"], d["k_cache"], d["v_cache"], d["block_tables"], d["context_lens"], d["k_scale"],
                 d["v_scale"], d["sinks"])
        torch.cuda.synchronize()
        return out.float().cpu().numpy()

    announce("shared meta buffer")
    pa.upload()
    compare(call(pa, inp_a, da), O.attend(inp_a), "plan A")
    pb.upload()
    compare(call(pb, inp_b, db), O.attend(inp_b), "plan B")
    with pytest.raises(ValueError, match="pa_plan_upload"):
        call(pa, inp_a, da)
    pa.upload()
    compare(call(pa, inp_a, da), O.attend(inp_a), "plan A again")
    buf[:32].zero_()  # the header no longer names plan A
    got = call(pa, inp_a, da)
    assert np.isnan(got).all(), "kernels followed a list whose header is not the plan's"
