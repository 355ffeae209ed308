"""GPU parity of the indexer (pa_mqa_logits, pa_topk) against the CPU
oracle (``oracle/indexer.py``).

Logits: within 2^-16 of their rounding scale sum_h |w| s sum_d |q k| (the
matrix cores add the 128 exact FP8 products of a dot in FP32, then at most
128 heads are summed in FP32: at most 256 roundings of at most 2^-24 of
that scale each), and exactly -inf outside every window under
clean_logits.  Top-k: bit-exact, the oracle's selection taken on the same FP32 logits the kernel read (the
selection is an integer decision made from floats, so both sides take it
on the same values).  The chained indexer -> two-level sparse decode is
checked for a valid selection against the oracle's logits and for the
decode's output against the oracle on the selected positions."""

from __future__ import annotations

import dataclasses

import numpy as np
import pytest
import torch

from gpu_helpers import announce, compare, run
from oracle import indexer as I
from oracle import oracle as O
from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W

pytestmark = pytest.mark.gpu

TOL = 2.0 ** -16


def _dev(x):
    return {k: getattr(x, k).cuda().contiguous() for k in ("q", "kv", "kv_scale", "weights", "ks", "ke")}


def _logits(x, clean=True, stride_pad=0, fill=float("nan")):
    d = _dev(x)
    out = torch.full((x.rows, x.num_kv + stride_pad), fill, dtype=torch.float32, device="cuda")
    B.pa_mqa_logits(out, d["q"], d["kv"], d["kv_scale"], d["weights"], d["ks"], d["ke"], clean=clean)
    torch.cuda.synchronize()
    return out[:, : x.num_kv].cpu().numpy()


def _check_logits(got, x, rows=None, clean=True):
    ref, mag = I.mqa_logits(x.q.numpy(), x.kv.numpy(), x.kv_scale.numpy(), x.weights.numpy(), x.ks.numpy(),
                            x.ke.numpy(), rows=rows)
    inside = np.isfinite(ref)
    if clean:
        assert (got[~inside] == -np.inf).all(), "outside the windows: not -inf"
    g, rf, m = got[inside].astype(np.float64), ref[inside], mag[inside]
    assert np.isfinite(g).all()
    err = np.abs(g - rf)
    bad = err > TOL * m + 1e-30
    worst = float((err / (m + 1e-30)).max()) if err.size else 0.0
    print(f"[logits] worst |error| / scale = {worst:.3g}", flush=True)
    assert not bad.any(), f"{bad.sum()} logits outside 2^-16 of their scale; worst {worst:.3g}"
    return ref


@pytest.mark.parametrize("heads", [16, 32, 64, 128])
@pytest.mark.parametrize("windows", ["full", "causal", "mixed"])
def test_logits_parity(heads, windows):
    x = W.make_indexer_case(700 + heads, 13, 1000, heads=heads, windows=windows)
    announce(f"mqa logits heads={heads} windows={windows}")
    _check_logits(_logits(x), x)


def test_logits_unclean_and_strided():
    """clean_logits off: every in-window value right (the rest unspecified);
    a row stride past num_kv leaves the padding columns untouched."""
    x = W.make_indexer_case(733, 9, 777, heads=64, windows="mixed")
    announce("mqa logits unclean, strided")
    d = _dev(x)
    out = torch.full((x.rows, 800), 7.0, dtype=torch.float32, device="cuda")
    B.pa_mqa_logits(out, d["q"], d["kv"], d["kv_scale"], d["weights"], d["ks"], d["ke"], clean=False)
    torch.cuda.synchronize()
    o = out.cpu().numpy()
    assert (o[:, 777:] == 7.0).all()
    _check_logits(o[:, :777], x, clean=False)


def test_logits_extreme_codes():
    """Queries and keys at the FP8 extremes (+-448, subnormals) and zero
    keys: exact products, no overflow of the FP32 accumulators."""
    x = W.make_indexer_case(734, 8, 300, heads=32)
    g = torch.Generator().manual_seed(5)
    pool = torch.tensor([0x7E, 0xFE, 0x01, 0x81, 0x00, 0x38, 0xB8], dtype=torch.uint8)  # 448, -448, tiny, 0, +-1
    x.q.copy_(pool[torch.randint(0, len(pool), x.q.shape, generator=g)])
    x.kv.copy_(pool[torch.randint(0, len(pool), x.kv.shape, generator=g)])
    x.kv[:20] = 0
    announce("mqa logits extreme codes")
    _check_logits(_logits(x), x)


def _topk_gpu(logits_np, ks, ke, k):
    lg = torch.from_numpy(np.ascontiguousarray(logits_np, dtype=np.float32)).cuda()
    rows = lg.shape[0]
    idx = torch.full((rows, k), 12345, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    B.pa_topk(idx, cnt, lg, ks.cuda().contiguous(), ke.cuda().contiguous())
    torch.cuda.synchronize()
    return idx.cpu().numpy(), cnt.cpu().numpy()


@pytest.mark.parametrize("k", [1, 7, 300, 2048])
def test_topk_bit_exact_on_kernel_logits(k):
    x = W.make_indexer_case(740 + k, 11, 3000, heads=64, windows="mixed")
    announce(f"top-k on kernel logits k={k}")
    lg = _logits(x)
    gi, gc = _topk_gpu(lg, x.ks, x.ke, k)
    oi, oc = I.topk(lg, x.ks.numpy(), x.ke.numpy(), k)
    assert np.array_equal(gc, oc) and np.array_equal(gi, oi)


@pytest.mark.parametrize("k", [1, 5, 64, 1000])
def test_topk_ties_and_specials(k):
    """Logits from a small pool (heavy ties, -inf, -0.0 and +0.0 equal):
    the tied keys taken are the lowest positions."""
    rng = np.random.default_rng(750 + k)
    pool = np.array([-np.inf, -3.0, -0.0, 0.0, 1.0, 1.0000001, 2.5], dtype=np.float32)
    lg = rng.choice(pool, size=(9, 5000)).astype(np.float32)
    ks = torch.tensor([0, 100, 4999, 3000, -10, 0, 2500, 0, 17], dtype=torch.int32)
    ke = torch.tensor([5000, 1100, 5000, 3000, 7000, 1, 2500 + k, 5000, 17 + k + 1], dtype=torch.int32)
    announce(f"top-k ties k={k}")
    gi, gc = _topk_gpu(lg, ks, ke, k)
    oi, oc = I.topk(lg, ks.numpy(), ke.numpy(), k)
    assert np.array_equal(gc, oc) and np.array_equal(gi, oi)


def test_indexer_full_size():
    """The sparse decode batch's indexer (64 rows x 65536 keys, 64 heads):
    logits of four sampled rows against the oracle, and the top-2048 of
    every row bit-exact against the oracle's selection on the same logits."""
    x = W.config_indexer_decode()
    announce("indexer full size")
    lg = _logits(x)
    rows = [0, 17, 40, 63]
    _check_logits(lg[rows], x, rows=rows)
    gi, gc = _topk_gpu(lg, x.ks, x.ke, 2048)
    oi, oc = I.topk(lg, x.ks.numpy(), x.ke.numpy(), 2048)
    assert np.array_equal(gc, oc) and np.array_equal(gi, oi)


def test_indexer_then_sparse_decode():
    """Indexer -> top-k -> two-level sparse decode: the selected positions
    are a valid top-k of the oracle's logits (every selected logit at least
    every unselected one, up to the logits tolerance), and the decode over
    them matches the oracle within atol = rtol = 0.005."""
    dec = W.config_sparse_topk(num_rows=6, selected=600, pool_pages=64)
    L = dec.problem.table_stride * dec.problem.page_size  # 1024 logical positions
    x = W.make_indexer_case(760, dec.problem.num_seqs, L, heads=64, windows="full")
    announce("indexer -> sparse decode")
    lg = _logits(x)
    k = dec.problem.index_stride
    gi, gc = _topk_gpu(lg, x.ks, x.ke, k)
    ref, mag = I.mqa_logits(x.q.numpy(), x.kv.numpy(), x.kv_scale.numpy(), x.weights.numpy(), x.ks.numpy(),
                            x.ke.numpy())
    for r in range(x.rows):
        sel = np.zeros(L, bool)
        sel[gi[r, : gc[r]]] = True
        tol = TOL * mag[r].max()
        assert ref[r, sel].min() >= ref[r, ~sel].max() - 2 * tol
    inp = dataclasses.replace(dec, topk_indices=torch.from_numpy(gi), context_lens=torch.from_numpy(gc))
    got, _ = run(inp, cu_count=64, partition_tokens=256)
    compare(got, O.attend(inp), "indexer -> sparse decode")
