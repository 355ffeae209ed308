"""Pins of the oracle's MXFP4 cache path (``oracle/pa_oracle.c``) against
things other than itself: the OCP microscaling format's E2M1 value table and
E8M0 definition, and the oracle's own BF16 path (already pinned by the
brute force) on the same K/V values laid out as BF16 caches.  The values of
those caches come from codes and scale bytes drawn here and decoded with the
format table below, not through the oracle, so a wrong nibble order, block
index, scale index or row stride in the oracle's MXFP4 addressing moves its
output away from the BF16 path's (the last test checks that each such
mistake would be seen)."""

from __future__ import annotations

import math

import numpy as np
import pytest
import torch

from oracle import oracle as O
from paged_attention_decode_plan_amd import workloads as W

# OCP MX E2M1: (exponent, mantissa) -> magnitude; bias 1, subnormal at exponent 0
E2M1 = {(0, 0): 0.0, (0, 1): 0.5, (1, 0): 1.0, (1, 1): 1.5, (2, 0): 2.0, (2, 1): 3.0, (3, 0): 4.0, (3, 1): 6.0}


def _fp4(code: int) -> float:
    mag = E2M1[((code >> 1) & 3, code & 1)]
    return -mag if code & 8 else mag


def test_fp4_table():
    for c in range(16):
        assert O.fp4_value(c) == _fp4(c), c
    assert math.copysign(1.0, O.fp4_value(8)) == -1.0  # negative zero


def test_e8m0():
    for e in (0, 1, 64, 126, 127, 128, 200, 254):
        assert O.e8m0_value(e) == 2.0 ** (e - 127), e
    assert math.isnan(O.e8m0_value(255))


def _mx_and_bf16(seed, lens, page=32, D=128, H=1, G=4, QL=2, window=0, sinks=False, pack=None):
    """One MXFP4 case and the BF16 case holding the same K/V values."""
    rng = np.random.default_rng(seed)
    base = W.make_dense_case(seed, lens, query_len=QL, num_q_heads=H * G, num_kv_heads=H, head_dim=D,
                             page_size=page, kv_dtype="mxfp4", sliding_window=window, has_sinks=sinks,
                             poison=False)
    P = base.problem.num_pages
    kc = rng.integers(0, 16, size=(P, H, page, D), dtype=np.uint8)
    vc = rng.integers(0, 16, size=(P, H, page, D), dtype=np.uint8)
    ks = rng.integers(120, 131, size=(P, H, page, D // 32), dtype=np.uint8)
    vs = rng.integers(120, 131, size=(P, H, page, D // 32), dtype=np.uint8)
    table = np.array([_fp4(c) for c in range(16)], np.float64)
    kval = table[kc] * np.exp2(np.repeat(ks.astype(np.float64) - 127, 32, axis=-1))
    vval = table[vc] * np.exp2(np.repeat(vs.astype(np.float64) - 127, 32, axis=-1))
    pk = (pack or {}).get("k", W._layout_k_mx)
    pv = (pack or {}).get("v", W._layout_v_mx)
    mx = W.Inputs(problem=base.problem, q=base.q, k_cache=pk(torch.from_numpy(kc)), v_cache=pv(torch.from_numpy(vc)),
                  block_tables=base.block_tables, context_lens=base.context_lens,
                  k_scale=torch.from_numpy(ks), v_scale=torch.from_numpy(vs), sinks=base.sinks)
    pb = W.Problem(**{**base.problem.__dict__, "kv_dtype": "bf16", "scale_mode": "none"})
    kb = torch.from_numpy(kval.astype(np.float32)).to(torch.bfloat16)  # exact: 2 significant bits
    vb = torch.from_numpy(vval.astype(np.float32)).to(torch.bfloat16)
    assert torch.equal(kb.float().double(), torch.from_numpy(kval)) and torch.equal(vb.float().double(), torch.from_numpy(vval))
    bf = W.Inputs(problem=pb, q=base.q, k_cache=W._layout_k(kb.view(torch.int16), 2).view(torch.bfloat16),
                  v_cache=W._layout_v(vb.view(torch.int16), 2, False).view(torch.bfloat16),
                  block_tables=base.block_tables, context_lens=base.context_lens, k_scale=None, v_scale=None,
                  sinks=base.sinks)
    return mx, bf


@pytest.mark.parametrize("page,window,sinks", [(32, 0, False), (64, 17, True), (128, 0, True)])
def test_mx_path_equals_bf16_path(page, window, sinks):
    mx, bf = _mx_and_bf16(31 + page, [1, 70, 200, 0, 333], page=page, window=window, sinks=sinks)
    a, b = O.attend(mx), O.attend(bf)
    assert np.array_equal(a, b)
    assert np.abs(a).max() > 0


def test_one_token_context_returns_its_v_row():
    mx, _ = _mx_and_bf16(77, [1], page=32, QL=1)
    p = mx.problem
    page = int(mx.block_tables[0, 0])
    vbytes = mx.v_cache[page, 0, :, 0].numpy()  # row d, byte 0 holds token 0 in its low nibble
    vs = mx.v_scale[page, 0, 0].numpy()
    want = np.array([_fp4(int(vbytes[d]) & 15) * 2.0 ** (int(vs[d // 32]) - 127) for d in range(p.head_dim)])
    got = O.attend(mx)
    for h in range(p.num_q_heads):
        assert np.array_equal(got[0, h], want.astype(np.float32))


def test_planted_layout_mistakes_are_seen():
    """Packings with the nibbles swapped, the K blocks in token-major order or
    V in token-major rows: the oracle (reading the documented layout) no
    longer matches the BF16 path."""
    def k_swapped(codes):
        P, H, page, D = codes.shape
        c = codes.reshape(P, H, page, D // 32, 16, 2)
        return (c[..., 1] | (c[..., 0] << 4)).permute(0, 1, 3, 2, 4).contiguous()

    def k_token_major(codes):
        P, H, page, D = codes.shape
        c = codes.reshape(P, H, page, D // 32, 16, 2)
        b = c[..., 0] | (c[..., 1] << 4)
        return b.contiguous().reshape(P, H, D // 32, page, 16)

    def v_token_major(codes):
        P, H, page, D = codes.shape
        c = codes.reshape(P, H, page, D // 2, 2)
        return (c[..., 0] | (c[..., 1] << 4)).reshape(P, H, D, page // 2).contiguous()

    for pack in ({"k": k_swapped}, {"k": k_token_major}, {"v": v_token_major}):
        mx, bf = _mx_and_bf16(91, [40, 90], page=32, pack=pack)
        assert not np.allclose(O.attend(mx), O.attend(bf), atol=1e-3), pack
