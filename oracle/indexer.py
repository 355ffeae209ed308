"""CPU oracle of the sparse front end's indexer: FP8 MQA logits and top-k.

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg import this module; the product package never does.  It
shares no code with the GPU library: FP8 values come from the decode
oracle's own decoder (``pa_oracle.c``, pinned against the OCP OFP8 tables).

The operation (the fp8_mqa_logits indexer of the FlyDSL pages: aiter PR
"LDS-staged fp8_mqa_logits for gfx942", Summary and Changes — a ReLU times
weight epilogue, a reduction over heads, -inf outside each row's
[ks, ke) window under clean_logits).  The pages print no formula; the
reading taken here is the lightning-indexer score of DeepSeek-V3.2, which
those terms describe:

    logits[r, t] = sum_h  w[r, h] * relu(s[t] * (q[r, h, :] . k[t, :]))

for ks[r] <= t < ke[r] (both clamped into [0, N]), and -inf elsewhere;
q, k FP8 e4m3fn codes, s the per-token FP32 key scale, w FP32.  Every
product and sum is exact in float64 here (FP8 x FP8 products have at most 8
significant bits and D <= 256 of them fit in 53 bits; the head sum is
rounded once per term, far below any tolerance that matters).

Top-k (the selection the two-level sparse decode consumes, aiter PR #7079
Summary: a top-k index stage selects token positions): per row the k
largest logits of its window, ties by the lower position, returned as
positions relative to the window start (t - ks[r]) in ascending order,
with count = min(k, window length).  Values compare as IEEE floats
(-0.0 == +0.0); NaN logits are outside the contract.
"""

from __future__ import annotations

import numpy as np

from oracle import oracle as O

_FP8 = None


def fp8_table() -> np.ndarray:
    """float64 value of every e4m3fn code (NaN for the two NaN codes)."""
    global _FP8
    if _FP8 is None:
        _FP8 = np.array([O.fp8_value(c) for c in range(256)], dtype=np.float64)
    return _FP8


def window(ks: int, ke: int, n: int) -> tuple[int, int]:
    """A row's window [lo, hi) clamped into [0, n]; empty when ke <= ks."""
    lo = min(max(int(ks), 0), n)
    hi = min(max(int(ke), lo), n)
    return lo, hi


def mqa_logits(q_codes, kv_codes, kv_scale, weights, ks, ke, rows=None):
    """float64 logits [R, N] (or only the given rows) and their rounding
    scale sum_h |w| s sum_d |q k| (the sum of absolute products: the scale of
    the error of any float32 evaluation of the dot products, whatever their
    cancellation, and of the ReLU decision near 0), both -inf / 0 outside
    the windows.

    q_codes uint8 [R, H, D], kv_codes uint8 [N, D], kv_scale float [N],
    weights float [R, H], ks / ke int [R]."""
    T = fp8_table()
    q_codes = np.asarray(q_codes, dtype=np.uint8)
    kv_codes = np.asarray(kv_codes, dtype=np.uint8)
    s = np.asarray(kv_scale, dtype=np.float64)
    w = np.asarray(weights, dtype=np.float64)
    R, H, D = q_codes.shape
    N = kv_codes.shape[0]
    rows = range(R) if rows is None else rows
    K = T[kv_codes]  # [N, D]
    out = np.full((len(rows), N), -np.inf)
    mag = np.zeros((len(rows), N))
    for i, r in enumerate(rows):
        lo, hi = window(ks[r], ke[r], N)
        if hi <= lo:
            continue
        dots = T[q_codes[r]] @ K[lo:hi].T          # [H, n]: exact
        act = np.maximum(dots * s[lo:hi][None, :], 0.0)  # relu of the scaled score
        out[i, lo:hi] = (w[r][:, None] * act).sum(axis=0)
        absdots = np.abs(T[q_codes[r]]) @ np.abs(K[lo:hi]).T
        mag[i, lo:hi] = (np.abs(w[r])[:, None] * absdots * s[lo:hi][None, :]).sum(axis=0)
    return out, mag


def topk(logits, ks, ke, k):
    """Selected positions int32 [R, k] (relative to ks, ascending, -1 past
    the count) and counts int32 [R] from float logits [R, N]."""
    logits = np.asarray(logits)
    R, N = logits.shape
    idx = np.full((R, k), -1, dtype=np.int32)
    cnt = np.zeros(R, dtype=np.int32)
    for r in range(R):
        lo, hi = window(ks[r], ke[r], N)
        pos = np.arange(lo, hi)
        vals = logits[r, lo:hi].astype(np.float64) + 0.0  # -0.0 and +0.0 compare equal
        order = np.lexsort((pos, -vals))  # largest value first, then the lower position
        sel = np.sort(pos[order[:k]]) - lo
        cnt[r] = len(sel)
        idx[r, : len(sel)] = sel
    return idx, cnt
