"""Pins of the indexer oracle (``oracle/indexer.py``) against things other
than itself: pure-Python brute force over tiny shapes, closed forms
(one-hot queries and keys, opposed keys that ReLU zeroes, exact scaling),
window edges, and top-k against Python's sort and numpy's argmax.  A
dropped ReLU, a scale outside it, a weight paired with the wrong head or
row, an off-by-one window, or a tie broken the wrong way fails one of them
(the last test plants each of those mistakes and checks that)."""

from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import indexer as I
from oracle import oracle as O


def _rand_codes(rng, shape):
    """FP8 e4m3fn codes of finite values (the two NaN codes 0x7F/0xFF excluded)."""
    c = rng.integers(0, 256, size=shape).astype(np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x38  # 1.0
    return c


def _brute_logits(qc, kc, s, w, ks, ke):
    R, H, D = qc.shape
    N = kc.shape[0]
    out = [[-math.inf] * N for _ in range(R)]
    for r in range(R):
        lo = min(max(int(ks[r]), 0), N)
        hi = min(max(int(ke[r]), lo), N)
        for t in range(lo, hi):
            terms = []
            for h in range(H):
                dot = math.fsum(O.fp8_value(int(qc[r, h, d])) * O.fp8_value(int(kc[t, d])) for d in range(D))
                terms.append(float(w[r, h]) * max(float(s[t]) * dot, 0.0))
            out[r][t] = math.fsum(terms)
    return np.array(out)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_logits_brute_force(seed):
    rng = np.random.default_rng(seed)
    R, H, D, N = 4, 5, 8, 23
    qc, kc = _rand_codes(rng, (R, H, D)), _rand_codes(rng, (N, D))
    s = rng.uniform(0.01, 3.0, N)
    w = rng.standard_normal((R, H))
    ks = np.array([0, 5, -3, 20])
    ke = np.array([23, 5, 7, 40])  # full, empty, clamped below, clamped above
    got, mag = I.mqa_logits(qc, kc, s, w, ks, ke)
    want = _brute_logits(qc, kc, s, w, ks, ke)
    fin = np.isfinite(want)
    assert (np.isfinite(got) == fin).all()
    assert np.allclose(got[fin], want[fin], rtol=1e-12, atol=1e-12 * np.abs(want[fin]).max())
    assert (mag[fin] >= np.abs(got[fin]) - 1e-9).all() and (mag[~fin] == 0).all()


def test_logits_one_hot_closed_form():
    """q[r, h] = a_h e_(h mod D), k[t] = b_t e_(t mod D): the dot is a_h b_t
    when h = t (mod D), else 0."""
    rng = np.random.default_rng(7)
    R, H, D, N = 3, 6, 4, 11
    vals = [0.5, -1.0, 2.0, 3.0, -0.25, 448.0]
    code = {O.fp8_value(c): c for c in range(256) if (c & 0x7F) != 0x7F}
    qc = np.zeros((R, H, D), np.uint8)
    kc = np.zeros((N, D), np.uint8)
    a = rng.choice(vals, size=(R, H))
    b = rng.choice(vals, size=N)
    for r in range(R):
        for h in range(H):
            qc[r, h, h % D] = code[a[r, h]]
    for t in range(N):
        kc[t, t % D] = code[b[t]]
    s = rng.choice([0.5, 1.0, 4.0], size=N)
    w = rng.choice([-2.0, -0.5, 1.0, 3.0], size=(R, H))
    got, _ = I.mqa_logits(qc, kc, s, w, np.zeros(R, int), np.full(R, N))
    for r in range(R):
        for t in range(N):
            want = sum(w[r, h] * max(s[t] * a[r, h] * b[t], 0.0) for h in range(H) if h % D == t % D)
            assert got[r, t] == want, (r, t)


def test_logits_relu_and_scaling():
    """Keys opposed to a one-head query score exactly 0 whatever the weight;
    aligned keys score w s |q|^2; weights and scales scale the result
    exactly by powers of two."""
    rng = np.random.default_rng(11)
    D, N = 16, 6
    qc = _rand_codes(rng, (1, 1, D))
    kc = np.concatenate([np.repeat(qc[0], 3, axis=0), np.repeat(qc[0] ^ 0x80, 3, axis=0)])  # +q x3, -q x3
    s = np.array([1.0, 0.5, 2.0, 1.0, 0.5, 2.0])
    q2 = float(sum(O.fp8_value(int(c)) ** 2 for c in qc[0, 0]))
    for wv in (-3.0, 0.75):
        got, _ = I.mqa_logits(qc, kc, s, np.array([[wv]]), [0], [N])
        assert (got[0, 3:] == 0.0).all()
        assert np.array_equal(got[0, :3], wv * s[:3] * q2)
    R, H = 2, 3
    qc = _rand_codes(rng, (R, H, D))
    kc = _rand_codes(rng, (N, D))
    w = rng.standard_normal((R, H))
    base, _ = I.mqa_logits(qc, kc, np.ones(N), w, [0, 0], [N, N])
    scaled, _ = I.mqa_logits(qc, kc, np.full(N, 0.25), w * 8.0, [0, 0], [N, N])
    assert np.array_equal(scaled, base * 2.0)


def test_topk_brute_force_with_ties():
    rng = np.random.default_rng(5)
    R, N = 6, 50
    pool = np.array([-np.inf, -1.5, -0.0, 0.0, 0.5, 2.0, 7.25], dtype=np.float32)
    x = rng.choice(pool, size=(R, N)).astype(np.float32)
    ks = np.array([0, 10, 45, 30, -5, 0])
    ke = np.array([50, 40, 49, 30, 70, 3])
    for k in (1, 4, 17, 60):
        idx, cnt = I.topk(x, ks, ke, k)
        for r in range(R):
            lo, hi = min(max(ks[r], 0), N), min(max(ke[r], max(ks[r], 0)), N)
            order = sorted(range(lo, hi), key=lambda t: (-float(x[r, t]), t))
            want = sorted(t - lo for t in order[:k])
            assert cnt[r] == len(want) and list(idx[r, : cnt[r]]) == want and (idx[r, cnt[r]:] == -1).all()


def test_topk_special_cases():
    rng = np.random.default_rng(9)
    x = rng.standard_normal((5, 40)).astype(np.float32)
    x[:, 7] = x[:, 3] = x.max() + 1  # a tied maximum
    idx, cnt = I.topk(x, np.zeros(5, int), np.full(5, 40), 1)
    assert (idx[:, 0] == np.argmax(x, axis=1)).all() and (idx[:, 0] == 3).all()  # the lower tied position
    idx, cnt = I.topk(x, np.zeros(5, int), np.full(5, 40), 40)
    assert (cnt == 40).all() and (idx == np.arange(40)).all()
    y = rng.permutation(1000).astype(np.float32)[None, :]
    idx, _ = I.topk(y, [0], [1000], 100)
    assert np.array_equal(idx[0], np.sort(np.argpartition(-y[0], 100)[:100]))


def test_pins_catch_planted_mistakes():
    """Each plausible mistake, planted in a copy of the oracle's formula,
    moves a tiny case away from the brute force."""
    rng = np.random.default_rng(21)
    R, H, D, N = 3, 4, 8, 17
    qc, kc = _rand_codes(rng, (R, H, D)), _rand_codes(rng, (N, D))
    s = rng.uniform(0.1, 2.0, N)
    w = rng.standard_normal((R, H))
    ks, ke = np.array([0, 3, 5]), np.array([17, 12, 16])
    want = _brute_logits(qc, kc, s, w, ks, ke)
    T = I.fp8_table()

    def variant(kind):
        out = np.full((R, N), -np.inf)
        for r in range(R):
            lo, hi = ks[r] + (kind == "window"), ke[r]
            dots = T[qc[r]] @ T[kc[lo:hi]].T
            act = dots * s[lo:hi] if kind == "no_relu" else np.maximum(dots * s[lo:hi], 0.0)
            wr = np.roll(w[r], 1) if kind == "head" else (w[(r + 1) % R] if kind == "row" else w[r])
            out[r, lo:hi] = (wr[:, None] * act).sum(axis=0)
        return out

    for kind in ("no_relu", "head", "row", "window"):
        got = variant(kind)
        assert not np.allclose(np.nan_to_num(got, neginf=-1e30), np.nan_to_num(want, neginf=-1e30)), kind
    x = np.array([[1.0, 2.0, 2.0, 0.5]], np.float32)
    idx, _ = I.topk(x, [0], [4], 1)
    assert idx[0, 0] == 1  # the higher tied position would give 2
