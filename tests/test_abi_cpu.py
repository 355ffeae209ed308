"""C-ABI and host-planner tests that need no GPU: the library loads, exports
every function include/pa_decode.h declares, rejects bad problems with the
documented status codes, and plans cover every visible tile exactly once."""

from __future__ import annotations

import ctypes
import os
import re

import numpy as np
import pytest

from paged_attention_decode_plan_amd import binding as B
from paged_attention_decode_plan_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _header_functions():
    import glob

    text = "".join(open(f).read() for f in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = B.load_library()
    names = _header_functions()
    assert set(names) == set(B.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def _prob(**kw):
    base = dict(num_seqs=2, query_len=1, num_q_heads=8, num_kv_heads=1, head_dim=128, page_size=16, num_pages=16,
                table_stride=8)
    base.update(kw)
    return B.make_problem(**base)


@pytest.mark.parametrize("kw,exc", [
    (dict(query_len=0), ValueError),
    (dict(num_q_heads=6, num_kv_heads=4), ValueError),
    (dict(sliding_window=-1), ValueError),
    (dict(head_dim=96), NotImplementedError),
    (dict(page_size=48), NotImplementedError),
    (dict(page_size=2048), NotImplementedError),
    (dict(token_table=True, page_size=256), NotImplementedError),
    (dict(scale_mode="none"), NotImplementedError),
    (dict(kv_dtype="bf16"), NotImplementedError),  # BF16 with a scale
    (dict(kv_dtype="bf16", scale_mode="none", head_dim=256), NotImplementedError),
    (dict(kv_dtype="bf16", scale_mode="none", head_dim=512), NotImplementedError),
    (dict(head_dim=1024), NotImplementedError),
    (dict(head_dim=512, token_table=True), NotImplementedError),
    (dict(token_table=True, sliding_window=4), NotImplementedError),
    (dict(token_table=True, query_len=2), NotImplementedError),
    (dict(num_pages=1 << 30, head_dim=256, page_size=128, num_kv_heads=8, num_q_heads=8), ValueError),
])
def test_plan_rejects(kw, exc):
    with pytest.raises(exc):
        B.Plan(_prob(**kw), [37, 100], cu_count=256)


def test_plan_negative_options():
    with pytest.raises(ValueError):
        B.Plan(_prob(), [37, 100], cu_count=-1)


def test_decode_error_paths_without_launch():
    L = B.load_library()
    plan = B.Plan(_prob(), [37, 100], cu_count=256)
    z = [None] * 12
    assert L.pa_decode(None, *z) == B.PA_ERR_INVALID
    assert L.pa_decode(plan.handle, *z) == B.PA_ERR_INVALID  # null device pointers
    bad = 0x1008  # not 16-byte aligned
    args = [bad, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000, None, 0x9000, 0xA000, None]
    assert L.pa_decode(plan.handle, *args) == B.PA_ERR_INVALID
    assert b"aligned" in L.pa_last_error()
    args[0] = 0x1000
    args[6] = None  # k_scale missing for FP8
    assert L.pa_decode(plan.handle, *args) == B.PA_ERR_INVALID
    args[6] = 0x7000
    args[9] = None  # meta_dev
    assert L.pa_decode(plan.handle, *args) == B.PA_ERR_WORKSPACE
    args[9] = 0x9000  # never filled by pa_plan_upload for this plan
    assert L.pa_decode(plan.handle, *args) == B.PA_ERR_WORKSPACE
    assert b"pa_plan_upload" in L.pa_last_error()
    assert L.pa_reduce(plan.handle, 0x1000, None, 0x9000, 0xA000, None) in (B.PA_OK, B.PA_ERR_WORKSPACE)
    assert L.pa_plan_upload(None, 0x9000, None) == B.PA_ERR_INVALID
    assert L.pa_plan_upload(plan.handle, None, None) == B.PA_ERR_WORKSPACE
    assert L.pa_plan_upload(plan.handle, 0x9008, None) == B.PA_ERR_INVALID  # misaligned
    assert L.pa_reduce(None, None, None, None, None, None) == B.PA_ERR_INVALID
    assert L.pa_plan_sizes(None, None, None) == B.PA_ERR_INVALID


def _coverage(plan, lens, prob, ql, window, page):
    """Every (seq, kv head, row group) tile range is covered exactly once."""
    work = plan.work().numpy()
    info = plan.info()
    tiles = {}
    for s, L in enumerate(lens):
        L = min(max(int(L), 0), prob.table_stride * page)
        lo, hi = W.visible_span(L, ql, window, True)
        t0 = (lo // page) * page
        tiles[s] = (hi - t0 + 127) // 128 if hi > lo else 0
    seen = {}
    slots = []
    for (s, g, rg, b, e, slot, part, nparts) in work.tolist():
        e = tiles[s] if e < 0 else e
        key = (s, g, rg)
        seen.setdefault(key, []).append((part, b, e, slot, nparts))
        if slot >= 0:
            slots.append(slot)
    assert len(slots) == len(set(slots)) == info.num_slots
    for s in range(prob.num_seqs):
        for g in range(prob.num_kv_heads):
            for rg in range(info.row_groups):
                parts = sorted(seen[(s, g, rg)])
                n = len(parts)
                assert all(p[4] == n for p in parts)
                assert [p[0] for p in parts] == list(range(n))
                assert parts[0][1] == 0 and parts[-1][2] == tiles[s]
                for a, b in zip(parts[:-1], parts[1:]):
                    assert a[2] == b[1] and a[1] <= a[2]
                if n > 1:
                    assert all(p[3] >= 0 for p in parts)
                    assert [p[3] for p in parts] == list(range(parts[0][3], parts[0][3] + n))
                else:
                    assert parts[0][3] == -1
    return work


@pytest.mark.parametrize("cu", [8, 80, 256, 304])
@pytest.mark.parametrize("ql,window,page", [(1, 0, 16), (4, 0, 128), (4, 8193, 64), (1, 257, 16), (3, 17, 64)])
def test_plan_covers_tiles_exactly_once(cu, ql, window, page):
    rng = np.random.default_rng(cu * 7 + ql)
    lens = rng.integers(0, 40000, size=23)
    lens[:3] = [0, 1, 2]
    stride = int((lens.max() + page - 1) // page) + 1
    prob = _prob(num_seqs=len(lens), query_len=ql, num_q_heads=16, num_kv_heads=2, page_size=page,
                 num_pages=stride * len(lens), table_stride=stride, sliding_window=window)
    plan = B.Plan(prob, lens, cu_count=cu)
    work = _coverage(plan, lens, prob, ql, window, page)
    info = plan.info()
    assert info.max_parts <= min(cu, 256)
    units = len(lens) * 2 * info.row_groups
    assert info.num_items <= max(units, 8 * 2 * cu)  # at most 8 items per resident workgroup slot
    # longest items first
    lens_tiles = []
    for (s, g, rg, b, e, slot, part, np_) in work.tolist():
        lens_tiles.append(b)
    # determinism
    again = B.Plan(prob, lens, cu_count=cu).work()
    assert (again.numpy() == work).all()


def test_plan_multi_wave_for_long_batches():
    """Long contexts on fewer units than resident slots: the planner takes
    more items than slots when that balances the slots (the pages' MI355X
    shape gets about five partitions per sequence), and keeps to one item
    per slot for the dense MTP4 batch; refreshable plans keep the budget."""
    prob = _prob(num_seqs=200, query_len=4, num_q_heads=16, num_kv_heads=1, page_size=128,
                 num_pages=200 * 1563, table_stride=1563)
    lens = [200000] * 200
    plan = B.Plan(prob, lens, cu_count=256)
    info = plan.info()
    assert 4 * 256 <= info.num_items <= 8 * 256 and 5 <= info.max_parts <= 6
    _coverage(plan, np.array(lens), prob, 4, 0, 128)
    refresh = B.Plan(prob, lens, cu_count=256, refreshable=1)
    assert refresh.info().num_items == 256
    c4 = W.config_dense_mtp4("fp8", poison=False)
    assert B.Plan(B.problem_of(c4.problem), c4.context_lens, cu_count=256).info().num_items == 256


def test_plan_empty_sequences_get_clearing_items():
    prob = _prob(num_seqs=3, num_q_heads=8, num_kv_heads=2)
    plan = B.Plan(prob, [0, 0, 5], cu_count=16)
    work = plan.work().numpy()
    assert len(work) == 6  # one direct item per (seq, kv head)
    assert (work[:, 5] == -1).all()


def test_plan_caps_and_fixed_partitions():
    prob = _prob(num_seqs=2, table_stride=4096)
    plan = B.Plan(prob, [65536, 3000], cu_count=256, max_partitions=3)
    assert plan.info().max_parts <= 3
    plan = B.Plan(prob, [2048, 2048], cu_count=256, partition_tokens=512)
    assert plan.info().max_parts == 4 and plan.info().num_reduce == 2
    plan = B.Plan(prob, [65536, 65536], cu_count=256, max_partitions=1)
    assert plan.info().num_slots == 0


def test_plan_row_groups():
    prob = _prob(num_seqs=1, query_len=4, num_q_heads=32, num_kv_heads=1)  # 128 rows -> 2 groups
    plan = B.Plan(prob, [1000], cu_count=64)
    info = plan.info()
    assert info.row_groups == 2 and info.rows_per_group == 64


def test_plan_zero_sequences():
    prob = _prob(num_seqs=0)
    plan = B.Plan(prob, [], cu_count=8)
    assert plan.info().num_items == 0 and plan.meta_bytes == 32  # the header only


def test_refreshable_plan_layout():
    """A refreshable plan: a fixed item budget (cu_count x resident
    workgroups) padded with unused items (seq -1), one reduce entry per
    (sequence, KV head, row group), at least one partial slot per item; a
    plan made without the option refuses pa_plan_refresh."""
    lens = [5000, 0, 1, 700]
    prob = B.make_problem(4, 4, 16, 1, 128, 128, 64, 16, "bf16", "fp8", False, "token", 1, 0, 0, 0, 0.0)
    plan = B.Plan(prob, lens, cu_count=32, refreshable=1)
    info = plan.info()
    work = plan.work().numpy()
    assert info.num_items == 32 and work.shape[0] == 32
    used = work[:, 0] >= 0
    assert used.sum() >= 4 and (work[~used, 0] == -1).all()
    assert info.num_reduce == 4  # one entry per unit (Hkv 1, one row group)
    assert info.num_slots >= info.num_items
    plain = B.Plan(prob, lens, cu_count=32)
    with pytest.raises(ValueError):
        B._check(B.load_library().pa_plan_refresh(plain.handle, None, None, None))


def test_shared_meta_buffer_is_refused_without_upload():
    """Two plans and one meta_dev on a host without a GPU: the upload fails
    with PA_ERR_DEVICE and registers nothing, so both plans are refused with
    PA_ERR_WORKSPACE before any launch (the GPU test of the same name covers
    a successful upload followed by the other plan's)."""
    L = B.load_library()
    a = B.Plan(_prob(), [37, 100], cu_count=256)
    b = B.Plan(_prob(), [100, 37], cu_count=256)
    buf = 0x10000
    st = L.pa_plan_upload(a.handle, buf, None)
    assert st == B.PA_ERR_DEVICE  # no device here: nothing was copied, nothing registered
    args = [0x1000, 0x2000, 0x3000, 0x4000, 0x5000, 0x6000, 0x7000, 0x8000, None, buf, 0xA000, None]
    for plan in (a, b):
        assert L.pa_decode(plan.handle, *args) == B.PA_ERR_WORKSPACE


def test_in_kernel_merge_plan_layout():
    """The in-kernel merge: the same work list and partial slots as the
    reducer plan, plus one zeroed 128-byte arrival counter per slot after
    the reduce table (128-byte aligned); pa_reduce then has nothing to
    launch; merge values outside 0..2 are refused."""
    lens = [5000, 0, 1, 700]
    prob = B.make_problem(4, 4, 16, 1, 128, 128, 64, 16, "bf16", "fp8", False, "token", 1, 0, 0, 0, 0.0)
    red = B.Plan(prob, lens, cu_count=32, merge=B.MERGE_REDUCER)
    ikm = B.Plan(prob, lens, cu_count=32, merge=B.MERGE_IN_KERNEL)
    auto = B.Plan(prob, lens, cu_count=32)
    assert (red.work().numpy() == ikm.work().numpy()).all()
    ri, ii = red.info(), ikm.info()
    assert ri.num_slots == ii.num_slots > 0 and ri.num_reduce == ii.num_reduce
    base = 32 + 32 * ri.num_items + 32 * ri.num_reduce
    assert red.meta_bytes == base == auto.meta_bytes
    assert ikm.meta_bytes == ((base + 127) // 128) * 128 + 128 * ii.num_slots
    # pa_reduce of an in-kernel-merge plan returns before any argument check or launch
    L = B.load_library()
    assert L.pa_reduce(ikm.handle, None, None, None, None, None) == B.PA_OK
    for bad in (-1, 3):
        with pytest.raises(ValueError):
            B.Plan(prob, lens, cu_count=32, merge=bad)
