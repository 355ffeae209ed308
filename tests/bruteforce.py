"""Dense brute-force attention used to pin the oracle on tiny inputs.

It takes a different route from the oracle on purpose: the caches are
unpacked to logical ``[page, Hkv, slot, D]`` arrays with tensor permutes, FP8
codes are decoded by torch's float8_e4m3fn conversion, every sequence's K/V
are materialised densely, an explicit boolean mask matrix is built, and the
softmax is evaluated in numpy long double.
"""

from __future__ import annotations

import numpy as np
import torch


def logical_caches(inp):
    """Return K, V as float64 numpy arrays [pages, Hkv, page, D] (dequantised)."""
    p = inp.problem
    P, H, ps, D = p.num_pages, p.num_kv_heads, p.page_size, p.head_dim
    if p.kv_dtype == "fp8":
        kf = inp.k_cache.view(torch.float8_e4m3fn).float()
        vf = inp.v_cache.view(torch.float8_e4m3fn).float()
        x = 16
    else:
        kf = inp.k_cache.float()
        vf = inp.v_cache.float()
        x = 8
    K = kf.reshape(P, H, D // x, ps, x).permute(0, 1, 3, 2, 4).reshape(P, H, ps, D)
    if p.v_transposed:
        V = vf.reshape(P, H, ps // x, D, x).permute(0, 1, 2, 4, 3).reshape(P, H, ps, D)
    else:
        V = vf.reshape(P, H, D, ps).permute(0, 1, 3, 2)
    K = K.double().numpy()
    V = V.double().numpy()
    if p.kv_dtype == "fp8":
        if p.scale_mode == "tensor":
            K = K * float(inp.k_scale[0])
            V = V * float(inp.v_scale[0])
        elif p.scale_mode == "token":
            K = K * inp.k_scale.double().numpy()[..., None]
            V = V * inp.v_scale.double().numpy()[..., None]
    return K, V


def attend(inp, pos_shift: int = 0, window_shift: int = 0) -> np.ndarray:
    """Dense masked softmax attention.  ``pos_shift`` / ``window_shift`` move
    the causal bound and the window length (mutations for the sensitivity
    test; 0 for the definition)."""
    p = inp.problem
    K, V = logical_caches(inp)
    q = inp.q.double().numpy()  # exact for bf16 / fp16
    bt = inp.block_tables.numpy()
    lens = inp.context_lens.numpy()
    G = p.num_q_heads // p.num_kv_heads
    out = np.zeros((p.rows, p.num_q_heads, p.head_dim), np.float64)
    cap = (p.index_stride if p.token_table == 2 else p.table_stride) if p.token_table else p.table_stride * p.page_size
    for s in range(p.num_seqs):
        L = int(min(max(int(lens[s]), 0), cap))
        if L == 0:
            continue
        t = np.arange(L)
        if p.token_table == 2:
            pos = np.clip(inp.topk_indices.numpy()[s, :L].astype(np.int64), 0, p.table_stride * p.page_size - 1)
            pages, offs = bt[s][pos // p.page_size].astype(np.int64), pos % p.page_size
        elif p.token_table:
            slots = bt[s, :L].astype(np.int64)
            pages, offs = slots // p.page_size, slots % p.page_size
        else:
            pages, offs = bt[s, t // p.page_size].astype(np.int64), t % p.page_size
        Kd = K[pages, :, offs, :]  # [L, Hkv, D]
        Vd = V[pages, :, offs, :]
        # explicit mask matrix [QL, L]
        i = np.arange(p.query_len)[:, None]
        pos = (L - p.query_len + i) if p.causal else np.full_like(i, L - 1)
        mask = (t[None, :] <= pos + pos_shift) & (t[None, :] < L)
        if p.sliding_window > 0:
            mask &= t[None, :] > pos - (p.sliding_window + window_shift)
        for ii in range(p.query_len):
            row = s * p.query_len + ii
            for h in range(p.num_q_heads):
                g = h // G
                vis = mask[ii]
                if not vis.any():
                    continue
                x = (Kd[vis, g, :].astype(np.longdouble) @ q[row, h].astype(np.longdouble)) * np.longdouble(p.scale)
                m = x.max()
                if p.has_sinks:
                    m = max(m, np.longdouble(float(inp.sinks[h])))
                w = np.exp(x - m)
                den = w.sum()
                if p.has_sinks:
                    den += np.exp(np.longdouble(float(inp.sinks[h])) - m)
                out[row, h] = (w[:, None] * Vd[vis, g, :].astype(np.longdouble)).sum(0) / den
    return out
