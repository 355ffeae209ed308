"""Seeded synthetic inputs for paged-attention decode.

This module builds host-side input tensors only: queries, paged K/V caches in
the packed/plain/transposed layouts, block tables, context lengths, dequant
scales and sink logits.  It holds none of the attention arithmetic; both the
GPU path and the CPU oracle consume what it produces.

Shapes follow the problem statement of the FlyDSL paged-attention decode pages
(aiter PR #4332 "Add paged-attention Tile kernel", host wrapper fragments;
aiter PR #6617 "Extend packed D256 PA decode pipe", summary):

* query ``[rows, Hq, D]`` with ``rows = num_seqs * query_len`` (BF16/FP16);
* packed K ``[pages, Hkv, D/x, page, x]`` with ``x = 16 / elem_bytes``;
* plain V ``[pages, Hkv, D, page]``; transposed V ``[pages, Hkv, page/x, D, x]``;
* int32 ``block_tables [num_seqs, table_stride]`` and ``context_lens [num_seqs]``;
* FP32 scales: one per tensor, or per token ``[pages, Hkv, page]``;
* FP32 sink logits ``[Hq]``;
* MXFP4 caches (OCP microscaling FP4: 32-dim blocks of E2M1 codes, two per
  byte with the lower index in the low nibble, one E8M0 scale byte per
  block): K ``[pages, Hkv, D/32, page, 16]``, V ``[pages, Hkv, D, page/2]``
  (row d holds the page's tokens in order), scales uint8
  ``[pages, Hkv, page, D/32]``.

Quantisation to FP8 e4m3fn uses torch's round-to-nearest-even cast after
clamping to +-448 (the format's largest finite value).  BF16 rounding is
torch's round-to-nearest-even.

Positions that no query row can see (tail slots of a sequence's last page,
slots before a sliding window, pages that are never referenced) are filled
with poison when ``poison=True``: FP8 byte 0x7F and BF16 0x7FC0 (both NaN),
and per-token scales of 1e30; MXFP4 poison is the scale byte 0xFF (NaN).
A correct decode never lets them reach the output.

MXFP4 quantisation of a 32-dim block: shared exponent e = floor(log2 amax) -
2 (the largest E2M1 power), clamped into E8M0's range, then each element
x / 2^e rounded to the nearest E2M1 value (ties to the even code),
saturating at +-6; an all-zero block takes the scale byte 0.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

FP8_MAX = 448.0
FP8_POISON = 0x7F
BF16_POISON = 0x7FC0
SCALE_POISON = 1.0e30

KV_FP8 = "fp8"
KV_BF16 = "bf16"
KV_MXFP4 = "mxfp4"
SCALE_NONE = "none"
SCALE_TENSOR = "tensor"
SCALE_TOKEN = "token"
SCALE_MX = "mx"
FP4_GRID = (0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0)  # E2M1 magnitudes of codes 0-7
MX_POISON = 0xFF  # E8M0 NaN


@dataclasses.dataclass
class Problem:
    num_seqs: int
    query_len: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    table_stride: int
    q_dtype: str = "bf16"  # "bf16" | "fp16"
    kv_dtype: str = KV_FP8  # "fp8" | "bf16" | "mxfp4"
    v_transposed: bool = False
    scale_mode: str = SCALE_TENSOR  # "none" | "tensor" | "token" | "mx"
    causal: bool = True
    sliding_window: int = 0
    has_sinks: bool = False
    token_table: int = 0  # 0: page tables; 1: physical token slots; 2: top-k logical positions
    softmax_scale: float = 0.0  # <= 0 means 1/sqrt(head_dim)
    index_stride: int = 0  # top-k index tables: row stride of topk_indices

    @property
    def rows(self) -> int:
        return self.num_seqs * self.query_len

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)


@dataclasses.dataclass
class Inputs:
    problem: Problem
    q: torch.Tensor  # [rows, Hq, D] bf16/fp16
    k_cache: torch.Tensor  # uint8 (fp8) or bf16, packed layout
    v_cache: torch.Tensor  # uint8 (fp8) or bf16, plain or transposed layout
    block_tables: torch.Tensor  # int32 [num_seqs, table_stride]
    context_lens: torch.Tensor  # int32 [num_seqs]
    k_scale: Optional[torch.Tensor]  # float32 [1] or [pages, Hkv, page]
    v_scale: Optional[torch.Tensor]
    sinks: Optional[torch.Tensor]  # float32 [Hq]
    name: str = ""
    # top-k index tables (token_table 2): int32 [num_seqs, index_stride]
    # logical positions; context_lens then counts each row's selected tokens
    topk_indices: Optional[torch.Tensor] = None


def _streams(seed: int, n: int):
    return [np.random.Generator(np.random.PCG64(s)) for s in np.random.SeedSequence(seed).spawn(n)]


def config_seed(config_id: int) -> int:
    return 0x5EED0000 + config_id


def to_bf16(x: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)


def to_fp8_bytes(x: torch.Tensor) -> torch.Tensor:
    """float32 tensor -> uint8 e4m3fn codes (RNE, saturating at +-448)."""
    return x.clamp(-FP8_MAX, FP8_MAX).to(torch.float8_e4m3fn).view(torch.uint8)


def to_mxfp4(x: torch.Tensor):
    """float32 [..., D] -> (E2M1 codes uint8 [..., D] in 0..15, E8M0 scale
    bytes uint8 [..., D/32])."""
    *lead, D = x.shape
    xb = x.reshape(*lead, D // 32, 32)
    amax = xb.abs().amax(-1)
    e = torch.where(amax > 0, torch.floor(torch.log2(amax)) - 2, torch.full_like(amax, -127.0)).clamp(-127, 127)
    scaled = xb / torch.exp2(e)[..., None]
    mag = scaled.abs()
    # nearest magnitude: count the midpoints below; a tie goes to the even code
    code = torch.zeros(mag.shape, dtype=torch.uint8)
    for c in range(7):
        mid = 0.5 * (FP4_GRID[c] + FP4_GRID[c + 1])
        code += (mag > mid if c % 2 == 0 else mag >= mid).to(torch.uint8)
    code = torch.where((scaled < 0) & (code > 0), code | 8, code)
    return code.reshape(*lead, D), (e + 127).to(torch.uint8)


def _layout_k_mx(codes: torch.Tensor) -> torch.Tensor:
    """E2M1 codes [P, H, page, D] -> packed K [P, H, D/32, page, 16] bytes."""
    P, H, page, D = codes.shape
    c = codes.reshape(P, H, page, D // 32, 16, 2)
    b = c[..., 0] | (c[..., 1] << 4)
    return b.permute(0, 1, 3, 2, 4).contiguous()


def _layout_v_mx(codes: torch.Tensor) -> torch.Tensor:
    """E2M1 codes [P, H, page, D] -> V [P, H, D, page/2] bytes."""
    P, H, page, D = codes.shape
    c = codes.permute(0, 1, 3, 2).reshape(P, H, D, page // 2, 2)
    return (c[..., 0] | (c[..., 1] << 4)).contiguous()


def visible_span(L: int, query_len: int, window: int, causal: bool):
    """Token range [lo, hi) that at least one query row of a sequence can see."""
    if L <= 0:
        return 0, 0
    last = L - 1
    first_pos = L - query_len if causal else L - 1
    if window > 0:
        lo = max(0, first_pos - window + 1)
    else:
        lo = 0
    return lo, last + 1


def _layout_k(kl: torch.Tensor, elem_bytes: int) -> torch.Tensor:
    """[P, H, page, D] -> packed [P, H, D/x, page, x]."""
    P, H, page, D = kl.shape
    x = 16 // elem_bytes
    return kl.reshape(P, H, page, D // x, x).permute(0, 1, 3, 2, 4).contiguous()


def _layout_v(vl: torch.Tensor, elem_bytes: int, transposed: bool) -> torch.Tensor:
    """[P, H, page, D] -> plain [P, H, D, page] or transposed [P, H, page/x, D, x]."""
    P, H, page, D = vl.shape
    if not transposed:
        return vl.permute(0, 1, 3, 2).contiguous()
    x = 16 // elem_bytes
    return vl.reshape(P, H, page // x, x, D).permute(0, 1, 2, 4, 3).contiguous()


def build_dense(
    prob: Problem,
    context_lens: np.ndarray,
    block_tables: np.ndarray,
    seed: int,
    fill: str = "visible",
    poison: bool = True,
    kv_amplitude: float = 1.0,
    name: str = "",
) -> Inputs:
    """Dense (block-table) workload.

    ``fill``: "visible" gives real data only to pages holding visible tokens,
    "context" to every page a sequence references up to its length.
    """
    rq, rkv, rs = _streams(seed, 3)
    P, H, page, D = prob.num_pages, prob.num_kv_heads, prob.page_size, prob.head_dim
    fp8 = prob.kv_dtype == KV_FP8
    q = rq.standard_normal((prob.rows, prob.num_q_heads, D), dtype=np.float32)
    qt = to_bf16(q) if prob.q_dtype == "bf16" else torch.from_numpy(q).to(torch.float16)

    # Which (physical page) holds real data, and which slots of it.
    real_pages = []
    valid_lo = np.zeros(P, np.int64)  # first slot with real data (per page)
    valid_hi = np.zeros(P, np.int64)  # one past last slot with real data
    for s in range(prob.num_seqs):
        L = int(min(max(int(context_lens[s]), 0), prob.table_stride * page))
        lo, hi = visible_span(L, prob.query_len, prob.sliding_window, prob.causal)
        if fill == "context":
            lo = 0 if L > 0 else 0
        if hi <= lo:
            continue
        for j in range(lo // page, (hi + page - 1) // page):
            pid = int(block_tables[s, j])
            real_pages.append(pid)
            valid_lo[pid] = max(lo - j * page, 0)
            valid_hi[pid] = min(hi - j * page, page)
    real_pages = np.asarray(real_pages, dtype=np.int64)
    nreal = len(real_pages)

    vals_k = torch.from_numpy(rkv.standard_normal((nreal, H, page, D), dtype=np.float32)) * kv_amplitude
    vals_v = torch.from_numpy(rkv.standard_normal((nreal, H, page, D), dtype=np.float32)) * kv_amplitude

    k_scale = v_scale = None
    if prob.kv_dtype == KV_MXFP4:
        qk, ksr = to_mxfp4(vals_k)
        qv, vsr = to_mxfp4(vals_v)
        kl = torch.zeros((P, H, page, D), dtype=torch.uint8)
        vl = torch.zeros((P, H, page, D), dtype=torch.uint8)
        k_scale = torch.full((P, H, page, D // 32), MX_POISON if poison else 127, dtype=torch.uint8)
        v_scale = torch.full((P, H, page, D // 32), MX_POISON if poison else 127, dtype=torch.uint8)
        if nreal:
            idx = torch.from_numpy(real_pages)
            kl[idx] = qk
            vl[idx] = qv
            k_scale[idx] = ksr
            v_scale[idx] = vsr
            if poison:
                # slots of a real page outside the visible span: NaN scales
                for pid in real_pages.tolist():
                    lo_s, hi_s = int(valid_lo[pid]), int(valid_hi[pid])
                    k_scale[pid, :, :lo_s] = MX_POISON
                    v_scale[pid, :, :lo_s] = MX_POISON
                    k_scale[pid, :, hi_s:] = MX_POISON
                    v_scale[pid, :, hi_s:] = MX_POISON
        sinks = None
        if prob.has_sinks:
            sinks = torch.from_numpy(rs.standard_normal(prob.num_q_heads, dtype=np.float32))
        return Inputs(
            problem=prob, q=qt.contiguous(), k_cache=_layout_k_mx(kl), v_cache=_layout_v_mx(vl),
            block_tables=torch.from_numpy(np.ascontiguousarray(block_tables, dtype=np.int32)),
            context_lens=torch.from_numpy(np.ascontiguousarray(context_lens, dtype=np.int32)),
            k_scale=k_scale, v_scale=v_scale, sinks=sinks, name=name)
    if fp8:
        if prob.scale_mode == SCALE_TOKEN:
            ks_real = vals_k.abs().amax(dim=3) / FP8_MAX  # [nreal, H, page]
            vs_real = vals_v.abs().amax(dim=3) / FP8_MAX
            ks_real = torch.where(ks_real == 0, torch.ones_like(ks_real), ks_real)
            vs_real = torch.where(vs_real == 0, torch.ones_like(vs_real), vs_real)
            qk = to_fp8_bytes(vals_k / ks_real[..., None])
            qv = to_fp8_bytes(vals_v / vs_real[..., None])
            k_scale = torch.full((P, H, page), SCALE_POISON if poison else 1.0, dtype=torch.float32)
            v_scale = torch.full((P, H, page), SCALE_POISON if poison else 1.0, dtype=torch.float32)
            if nreal:
                k_scale[torch.from_numpy(real_pages)] = ks_real
                v_scale[torch.from_numpy(real_pages)] = vs_real
        elif prob.scale_mode == SCALE_TENSOR:
            ka = float(vals_k.abs().max()) if nreal else 0.0
            va = float(vals_v.abs().max()) if nreal else 0.0
            ks = ka / FP8_MAX if ka > 0 else 1.0
            vs = va / FP8_MAX if va > 0 else 1.0
            qk = to_fp8_bytes(vals_k / ks)
            qv = to_fp8_bytes(vals_v / vs)
            k_scale = torch.tensor([ks], dtype=torch.float32)
            v_scale = torch.tensor([vs], dtype=torch.float32)
        else:
            raise ValueError("FP8 caches need a scale mode")
        kl = torch.full((P, H, page, D), FP8_POISON if poison else 0, dtype=torch.uint8)
        vl = torch.full((P, H, page, D), FP8_POISON if poison else 0, dtype=torch.uint8)
        elem = 1
    else:
        qk = vals_k.to(torch.bfloat16).view(torch.int16)
        qv = vals_v.to(torch.bfloat16).view(torch.int16)
        pv = np.int16(BF16_POISON).item() if poison else 0
        kl = torch.full((P, H, page, D), pv, dtype=torch.int16)
        vl = torch.full((P, H, page, D), pv, dtype=torch.int16)
        elem = 2
    if nreal:
        idx = torch.from_numpy(real_pages)
        kl[idx] = qk
        vl[idx] = qv
        if poison:
            # Slots of a real page outside the visible span become poison again.
            pz = kl.new_full((D,), FP8_POISON if fp8 else np.int16(BF16_POISON).item())
            for pid in real_pages.tolist():
                lo_s, hi_s = int(valid_lo[pid]), int(valid_hi[pid])
                if lo_s > 0:
                    kl[pid, :, :lo_s] = pz
                    vl[pid, :, :lo_s] = pz
                    if k_scale is not None and k_scale.numel() > 1:
                        k_scale[pid, :, :lo_s] = SCALE_POISON
                        v_scale[pid, :, :lo_s] = SCALE_POISON
                if hi_s < page:
                    kl[pid, :, hi_s:] = pz
                    vl[pid, :, hi_s:] = pz
                    if k_scale is not None and k_scale.numel() > 1:
                        k_scale[pid, :, hi_s:] = SCALE_POISON
                        v_scale[pid, :, hi_s:] = SCALE_POISON
    kc = _layout_k(kl, elem)
    vc = _layout_v(vl, elem, prob.v_transposed)
    if not fp8:
        kc = kc.view(torch.bfloat16)
        vc = vc.view(torch.bfloat16)
    sinks = None
    if prob.has_sinks:
        sinks = torch.from_numpy(rs.standard_normal(prob.num_q_heads, dtype=np.float32))
    return Inputs(
        problem=prob,
        q=qt.contiguous(),
        k_cache=kc,
        v_cache=vc,
        block_tables=torch.from_numpy(np.ascontiguousarray(block_tables, dtype=np.int32)),
        context_lens=torch.from_numpy(np.ascontiguousarray(context_lens, dtype=np.int32)),
        k_scale=k_scale,
        v_scale=v_scale,
        sinks=sinks,
        name=name,
    )


def disjoint_tables(rng: np.random.Generator, lens_pages: np.ndarray, num_pages: int, stride: int) -> np.ndarray:
    """Give each sequence a disjoint slice of a random page permutation; fill
    entries past a sequence's extent with other sequences' page ids (stale)."""
    perm = rng.permutation(num_pages).astype(np.int32)
    bt = np.empty((len(lens_pages), stride), np.int32)
    off = 0
    for s, n in enumerate(lens_pages):
        n = int(n)
        bt[s, :n] = perm[off : off + n]
        off += n
        if n < stride:
            bt[s, n:] = rng.choice(perm, size=stride - n) if num_pages > 0 else 0
    return bt


def make_dense_case(
    seed: int,
    context_lens,
    query_len: int = 1,
    num_q_heads: int = 8,
    num_kv_heads: int = 1,
    head_dim: int = 128,
    page_size: int = 16,
    kv_dtype: str = KV_FP8,
    q_dtype: str = "bf16",
    v_transposed: bool = False,
    scale_mode: str = SCALE_TENSOR,
    sliding_window: int = 0,
    has_sinks: bool = False,
    causal: bool = True,
    extra_pages: int = 3,
    table_slack: int = 2,
    poison: bool = True,
    fill: str = "visible",
    kv_amplitude: float = 1.0,
    name: str = "",
) -> Inputs:
    """A general dense case; used by the parity matrix."""
    lens = np.asarray(context_lens, dtype=np.int64)
    rng = _streams(seed ^ 0xB10C, 1)[0]
    lens_pages = (lens + page_size - 1) // page_size
    num_pages = int(lens_pages.sum()) + extra_pages
    stride = int(max(1, lens_pages.max(initial=0) + table_slack))
    bt = disjoint_tables(rng, lens_pages, num_pages, stride)
    prob = Problem(
        num_seqs=len(lens), query_len=query_len, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, page_size=page_size, num_pages=num_pages, table_stride=stride,
        q_dtype=q_dtype, kv_dtype=kv_dtype, v_transposed=v_transposed,
        scale_mode=scale_mode if kv_dtype == KV_FP8 else (SCALE_MX if kv_dtype == KV_MXFP4 else SCALE_NONE),
        causal=causal,
        sliding_window=sliding_window, has_sinks=has_sinks,
    )
    return build_dense(prob, lens.astype(np.int32), bt, seed, fill=fill, poison=poison,
                       kv_amplitude=kv_amplitude, name=name)


# ----------------------------------------------------------------------------
# The five named workloads.
# ----------------------------------------------------------------------------

def config_tiny(v_transposed: bool = False, poison: bool = True) -> Inputs:
    """C1: batch 2, Hq 8 / Hkv 1, D 128, QL 1, page 16, lengths 37 and 100,
    tables a permutation of 16 pages, FP8 per-tensor amax/448, one partition."""
    seed = config_seed(1)
    rng = _streams(seed ^ 0xB10C, 1)[0]
    bt = rng.permutation(16).astype(np.int32).reshape(2, 8)
    prob = Problem(num_seqs=2, query_len=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16,
                   num_pages=16, table_stride=8, v_transposed=v_transposed, scale_mode=SCALE_TENSOR)
    return build_dense(prob, np.array([37, 100], np.int32), bt, seed, fill="context", poison=poison, name="tiny")


def config_long_d256(poison: bool = True, window: int = 8193) -> Inputs:
    """C3: batch 4, Hkv 2, GQA 8, QL 4 causal, D 256, page 64, context 131072,
    packed K, transposed V, per-tensor scales, window 8193."""
    seed = config_seed(3)
    rng = _streams(seed ^ 0xB10C, 1)[0]
    L = 131072
    pages_per = L // 64
    num_pages = 4 * pages_per
    bt = rng.permutation(num_pages).astype(np.int32).reshape(4, pages_per)
    prob = Problem(num_seqs=4, query_len=4, num_q_heads=16, num_kv_heads=2, head_dim=256, page_size=64,
                   num_pages=num_pages, table_stride=pages_per, v_transposed=True, scale_mode=SCALE_TENSOR,
                   sliding_window=window)
    return build_dense(prob, np.full(4, L, np.int32), bt, seed, fill="visible", poison=poison, name="long_d256")


def dense_mtp4_lengths(rng: np.random.Generator, n: int = 32) -> np.ndarray:
    return rng.integers(16384, 32768, size=n, endpoint=True).astype(np.int32)


def config_dense_mtp4(kv_dtype: str = KV_FP8, poison: bool = True, num_seqs: int = 32, query_len: int = 4) -> Inputs:
    """C4: batch 32, Hq 16 / Hkv 1, D 128, QL 4 causal, page 128, lengths
    uniform in [16384, 32768]; FP8 with per-token scales, or BF16 unscaled.
    Another query_len gives the same caches and tables with that many
    causal rows per sequence (QL 2: 32 rows per KV head)."""
    seed = config_seed(4)
    rng = _streams(seed ^ 0xB10C, 2)
    lens = dense_mtp4_lengths(rng[1], 32)[:num_seqs]
    lens_pages = (lens.astype(np.int64) + 127) // 128
    num_pages = int(lens_pages.sum())
    stride = 256
    bt = disjoint_tables(rng[0], lens_pages, num_pages, stride)
    prob = Problem(num_seqs=num_seqs, query_len=query_len, num_q_heads=16, num_kv_heads=1, head_dim=128,
                   page_size=128, num_pages=num_pages, table_stride=stride, kv_dtype=kv_dtype,
                   scale_mode={KV_FP8: SCALE_TOKEN, KV_MXFP4: SCALE_MX}.get(kv_dtype, SCALE_NONE))
    return build_dense(prob, lens, bt, seed, fill="context", poison=poison, name=f"dense_mtp{query_len}_{kv_dtype}")


def ragged_lengths(rng: np.random.Generator, n: int = 128) -> np.ndarray:
    u = rng.uniform(0.0, math.log(65537.0), size=n)
    L = np.floor(np.exp(u)).astype(np.int64) - 1
    L = np.clip(L, 0, 65536)
    L[:8] = 0
    L[8:16] = 1
    rng.shuffle(L)
    return L.astype(np.int32)


def config_ragged(poison: bool = True) -> Inputs:
    """C5: 128 sequences, lengths log-uniform in [0, 65536] with 8 empty and 8
    of length 1, Hkv 4 / GQA 4, D 128, QL 1, page 16, FP8 per-token scales,
    window 257, sink logits ~N(0,1)."""
    seed = config_seed(5)
    rng = _streams(seed ^ 0xB10C, 2)
    lens = ragged_lengths(rng[1], 128)
    lens_pages = (lens.astype(np.int64) + 15) // 16
    num_pages = int(lens_pages.sum())
    stride = int(max(1, lens_pages.max()))
    bt = disjoint_tables(rng[0], lens_pages, num_pages, stride)
    prob = Problem(num_seqs=128, query_len=1, num_q_heads=16, num_kv_heads=4, head_dim=128, page_size=16,
                   num_pages=num_pages, table_stride=stride, scale_mode=SCALE_TOKEN, sliding_window=257,
                   has_sinks=True)
    return build_dense(prob, lens, bt, seed, fill="visible", poison=poison, name="ragged")


def config_sparse(num_rows: int = 64, selected: int = 2048, pool_pages: int = 4096) -> Inputs:
    """C2: 64 rows, Hq 16 / Hkv 1, D 128, page 16 FP8 with per-token scales;
    each row attends `selected` distinct token slots drawn uniformly from a
    65536-token pool.  ``block_tables[r][j]`` holds a physical token slot
    (page * 16 + offset), ascending; ``context_lens[r]`` is the count."""
    seed = config_seed(2)
    rq, rkv, rsel = _streams(seed, 3)
    page, H, D = 16, 1, 128
    P = pool_pages
    perm = rsel.permutation(P).astype(np.int64)
    bt = np.empty((num_rows, selected), np.int32)
    for r in range(num_rows):
        logical = rsel.choice(P * page, size=selected, replace=False)
        phys = perm[logical // page] * page + logical % page
        bt[r] = np.sort(phys).astype(np.int32)
    q = rq.standard_normal((num_rows, 16, D), dtype=np.float32)
    vals_k = torch.from_numpy(rkv.standard_normal((P, H, page, D), dtype=np.float32))
    vals_v = torch.from_numpy(rkv.standard_normal((P, H, page, D), dtype=np.float32))
    ks = vals_k.abs().amax(dim=3) / FP8_MAX
    vs = vals_v.abs().amax(dim=3) / FP8_MAX
    ks = torch.where(ks == 0, torch.ones_like(ks), ks)
    vs = torch.where(vs == 0, torch.ones_like(vs), vs)
    kl = to_fp8_bytes(vals_k / ks[..., None])
    vl = to_fp8_bytes(vals_v / vs[..., None])
    prob = Problem(num_seqs=num_rows, query_len=1, num_q_heads=16, num_kv_heads=1, head_dim=D, page_size=page,
                   num_pages=P, table_stride=selected, scale_mode=SCALE_TOKEN, token_table=True)
    return Inputs(
        problem=prob, q=to_bf16(q), k_cache=_layout_k(kl, 1), v_cache=_layout_v(vl, 1, False),
        block_tables=torch.from_numpy(bt), context_lens=torch.full((num_rows,), selected, dtype=torch.int32),
        k_scale=ks.contiguous(), v_scale=vs.contiguous(), sinks=None, name="sparse",
    )


def config_sparse_topk(num_rows: int = 64, selected: int = 2048, pool_pages: int = 4096) -> Inputs:
    """The sparse decode batch of config_sparse with two-level indices: every
    row's context is the same 65536-token paged sequence (block table: a
    random permutation of the 4096-page pool), and the row attends
    ``selected`` distinct logical positions of it, drawn uniformly and
    sorted (the output of a top-k indexer), resolved through the block
    table by the decode.  The caches, scales and queries are those of
    config_sparse (same seed), and so are the physical tokens each row
    selects: the two calls give the same result."""
    base = config_sparse(num_rows, selected, pool_pages)
    seed = config_seed(2)
    rq, rkv, rsel = _streams(seed, 3)
    page = 16
    perm = rsel.permutation(pool_pages).astype(np.int64)
    logical = np.empty((num_rows, selected), np.int32)
    for r in range(num_rows):
        sel = rsel.choice(pool_pages * page, size=selected, replace=False)
        phys = perm[sel // page] * page + sel % page
        order = np.argsort(phys)  # the token order config_sparse uses (ascending physical slot)
        logical[r] = sel[order].astype(np.int32)
    bt = np.broadcast_to(perm.astype(np.int32), (num_rows, pool_pages)).copy()
    prob = dataclasses.replace(base.problem, table_stride=pool_pages, token_table=2, index_stride=selected)
    return dataclasses.replace(base, problem=prob, block_tables=torch.from_numpy(bt),
                               topk_indices=torch.from_numpy(logical), name="sparse_topk")


def resolve_topk(inp: Inputs) -> Inputs:
    """The same call with physical token slots (token_table 1): each top-k
    logical position resolved through the block table on the host."""
    p = inp.problem
    assert p.token_table == 2
    idx = inp.topk_indices.long().clamp(0, p.table_stride * p.page_size - 1)
    pages = torch.gather(inp.block_tables.long(), 1, idx // p.page_size)
    slots = (pages * p.page_size + idx % p.page_size).to(torch.int32)
    prob = dataclasses.replace(p, token_table=1, table_stride=p.index_stride, index_stride=0)
    return dataclasses.replace(inp, problem=prob, block_tables=slots.contiguous(), topk_indices=None)


@dataclasses.dataclass
class IndexerInputs:
    """Inputs of the indexer (FP8 MQA logits, then top-k): FP8 e4m3fn codes
    of the query rows [rows, heads, 128] and of the KV tokens' index keys
    [num_kv, 128], the keys' FP32 scales [num_kv], FP32 head weights
    [rows, heads], and each row's window [ks, ke)."""
    q: torch.Tensor
    kv: torch.Tensor
    kv_scale: torch.Tensor
    weights: torch.Tensor
    ks: torch.Tensor
    ke: torch.Tensor
    name: str = ""

    @property
    def rows(self) -> int:
        return self.q.shape[0]

    @property
    def num_kv(self) -> int:
        return self.kv.shape[0]


def make_indexer_case(seed: int, rows: int, num_kv: int, heads: int = 64, windows: str = "full",
                      name: str = "indexer") -> IndexerInputs:
    """Seeded indexer inputs: queries and keys drawn N(0, 1) and quantised to
    FP8 (keys with a per-token scale amax / 448, queries at a fixed scale of
    32 so that they use the FP8 range), head weights N(0, 1 / heads).
    windows: "full" (every row sees [0, num_kv)), "causal" (row r of a
    prefill chunk ending at num_kv sees [0, num_kv - rows + r + 1)), or
    "mixed" (a random window per row, including empty, clamped and
    out-of-range bounds)."""
    rq, rk, rw, rs = _streams(seed, 4)
    D = 128
    q = torch.from_numpy(rq.standard_normal((rows, heads, D), dtype=np.float32))
    k = torch.from_numpy(rk.standard_normal((num_kv, D), dtype=np.float32))
    ks = k.abs().amax(dim=1) / FP8_MAX
    ks = torch.where(ks == 0, torch.ones_like(ks), ks)
    w = torch.from_numpy((rw.standard_normal((rows, heads), dtype=np.float32) / np.sqrt(heads)).astype(np.float32))
    if windows == "full":
        lo = np.zeros(rows, np.int64)
        hi = np.full(rows, num_kv, np.int64)
    elif windows == "causal":
        lo = np.zeros(rows, np.int64)
        hi = num_kv - rows + np.arange(rows) + 1
    else:
        lo = rs.integers(-50, num_kv, size=rows)
        hi = lo + rs.integers(-10, num_kv + 50, size=rows)
        lo[:3], hi[:3] = [0, 5, num_kv - 1], [num_kv, 5, num_kv + 100]
    return IndexerInputs(q=to_fp8_bytes(q * 32.0).contiguous(), kv=to_fp8_bytes(k / ks[:, None]).contiguous(),
                         kv_scale=ks.contiguous(), weights=w.contiguous(),
                         ks=torch.from_numpy(lo.astype(np.int32)), ke=torch.from_numpy(hi.astype(np.int32)),
                         name=name)


def config_indexer_decode() -> IndexerInputs:
    """The indexer of the sparse decode batch (config_sparse_topk): 64 decode
    rows, each scoring every one of its sequence's 65536 tokens with 64 FP8
    index heads of dim 128 (the heads of the pages' indexer model shapes),
    before the top-2048 selection."""
    return make_indexer_case(config_seed(7), 64, 65536, heads=64, windows="full", name="indexer_decode")


CONFIGS = {
    "tiny": config_tiny,
    "sparse": config_sparse,
    "long_d256": config_long_d256,
    "dense_mtp4_fp8": lambda **kw: config_dense_mtp4(KV_FP8, **kw),
    "dense_mtp4_bf16": lambda **kw: config_dense_mtp4(KV_BF16, **kw),
    "ragged": config_ragged,
}


def kv_bytes_visible(inp: Inputs) -> int:
    """Algorithmic KV bytes of one call: K + V (+ per-token K and V scales) of
    the visible-token union of every (sequence, KV head), counted once."""
    p = inp.problem
    if p.kv_dtype == KV_MXFP4:  # half a byte per element, one scale byte per 32-dim block, K and V
        per_tok = 2 * (p.head_dim // 2 + p.head_dim // 32)
    else:
        elem = 1 if p.kv_dtype == KV_FP8 else 2
        per_tok = 2 * p.head_dim * elem + (8 if (p.kv_dtype == KV_FP8 and p.scale_mode == SCALE_TOKEN) else 0)
    lens = inp.context_lens.numpy().astype(np.int64)
    tot = 0
    for s in range(p.num_seqs):
        if p.token_table:
            n = int(min(max(lens[s], 0), p.index_stride if p.token_table == 2 else p.table_stride))
        else:
            L = int(min(max(lens[s], 0), p.table_stride * p.page_size))
            lo, hi = visible_span(L, p.query_len, p.sliding_window, p.causal)
            n = hi - lo
        tot += n
    return tot * p.num_kv_heads * per_tok


def config_long_mtp4_device(device, num_seqs: int = 200, context: int = 200_000, seed: int = 0x5EED0200) -> Inputs:
    """The pages' own MI355X decode shape (aiter PR #4332, the MI355 BS=200,
    MTP4, C=200k measurement): batch 200, every context 200 000 tokens, QL 4
    causal, Hq 16 / Hkv 1, D 128, page 128, FP8 e4m3fn K/V with per-token
    scales, plain V, no window.  10.56 GB of KV per call, so the caches are
    drawn on the device (torch's generator, seeded): K/V ~ N(0, 1) rounded
    to FP8, per-token scales uniform in [0.005, 0.015), Q ~ N(0, 1) in BF16,
    each sequence's pages a disjoint slice of one random permutation.  Every
    tensor but context_lens lives on ``device``; use host_subset() to give
    the oracle a few of the sequences."""
    D, page, H = 128, 128, 1
    pages_per_seq = (context + page - 1) // page
    num_pages = num_seqs * pages_per_seq
    prob = Problem(num_seqs=num_seqs, query_len=4, num_q_heads=16, num_kv_heads=H, head_dim=D, page_size=page,
                   num_pages=num_pages, table_stride=pages_per_seq, kv_dtype=KV_FP8, scale_mode=SCALE_TOKEN)
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def fp8_normal(shape):
        out = torch.empty(shape, dtype=torch.uint8, device=device)
        flat = out.view(-1)
        step = 1 << 28  # bounded temporaries
        for i in range(0, flat.numel(), step):
            n = min(step, flat.numel() - i)
            x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
            flat[i:i + n] = x.to(torch.float8_e4m3fn).view(torch.uint8)
        return out

    kc = fp8_normal((num_pages, H, D // 16, page, 16))
    vc = fp8_normal((num_pages, H, D, page))
    ks = 0.005 + 0.01 * torch.rand((num_pages, H, page), generator=g, device=device, dtype=torch.float32)
    vs = 0.005 + 0.01 * torch.rand((num_pages, H, page), generator=g, device=device, dtype=torch.float32)
    q = torch.randn((prob.rows, prob.num_q_heads, D), generator=g, device=device, dtype=torch.float32)
    perm = torch.randperm(num_pages, generator=g, device=device).to(torch.int32)
    return Inputs(problem=prob, q=q.to(torch.bfloat16).contiguous(), k_cache=kc, v_cache=vc,
                  block_tables=perm.view(num_seqs, pages_per_seq).contiguous(),
                  context_lens=torch.full((num_seqs,), context, dtype=torch.int32), k_scale=ks, v_scale=vs,
                  sinks=None, name="long_mtp4_c200k")


def host_subset(inp: Inputs, seqs) -> Inputs:
    """A host copy of some sequences of a block-table workload whose tensors
    may live on a device: their query rows, lengths and the pages their
    tables name (renumbered in order), the rest of the problem unchanged.
    The oracle's result for sequence seqs[i] of the subset is the original
    sequence's."""
    p = inp.problem
    assert not p.token_table
    seqs = list(seqs)
    bt = inp.block_tables[seqs].cpu().long()  # [n, stride]
    ids = bt.reshape(-1)
    dev_ids = ids.to(inp.k_cache.device)
    sub = dataclasses.replace(p, num_seqs=len(seqs), num_pages=int(ids.numel()))
    rows = torch.cat([torch.arange(s * p.query_len, (s + 1) * p.query_len) for s in seqs])
    per_token = inp.k_scale is not None and inp.k_scale.numel() > 1
    return Inputs(
        problem=sub,
        q=inp.q[rows.to(inp.q.device)].cpu().contiguous(),
        k_cache=inp.k_cache[dev_ids].cpu().contiguous(),
        v_cache=inp.v_cache[dev_ids].cpu().contiguous(),
        block_tables=torch.arange(ids.numel(), dtype=torch.int32).view(len(seqs), -1).contiguous(),
        context_lens=inp.context_lens[seqs].cpu().contiguous(),
        k_scale=None if inp.k_scale is None else (inp.k_scale[dev_ids] if per_token else inp.k_scale).cpu().contiguous(),
        v_scale=None if inp.v_scale is None else (inp.v_scale[dev_ids] if per_token else inp.v_scale).cpu().contiguous(),
        sinks=None if inp.sinks is None else inp.sinks.cpu(),
        name=inp.name + "_subset",
    )
