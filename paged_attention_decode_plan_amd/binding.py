"""ctypes binding of libpa.so (argument marshalling only).

Every step of the decode runs in the library's HIP kernels; this module only
checks tensors, fills the C structs and maps status codes to exceptions
(PA_ERR_INVALID / PA_ERR_WORKSPACE -> ValueError, PA_ERR_UNSUPPORTED ->
NotImplementedError, PA_ERR_DEVICE -> RuntimeError).  Importing it fails
loudly when libpa.so has not been built; there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libpa.so")

PA_OK, PA_ERR_INVALID, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE, PA_ERR_DEVICE = range(5)
PA_BF16, PA_FP16, PA_FP8_E4M3FN, PA_MXFP4 = range(4)
PA_V_PLAIN, PA_V_TRANSPOSED = range(2)
PA_SCALE_NONE, PA_SCALE_PER_TENSOR, PA_SCALE_PER_TOKEN, PA_SCALE_MX = range(4)

EXPORTS = ["pa_plan", "pa_plan_sizes", "pa_plan_info", "pa_plan_work", "pa_plan_upload", "pa_plan_free", "pa_decode",
           "pa_reduce", "pa_plan_refresh", "pa_attend_static", "pa_decode_sparse", "pa_mqa_logits", "pa_topk",
           "pa_topk_workspace_size", "pa_last_error"]
STATIC_SCRATCH_BYTES = 32 << 20  # PA_STATIC_SCRATCH_BYTES of include/pa_decode.h
META_HEADER_BYTES = 32  # meta_dev starts with the plan's header; the work list follows


class PaProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_seqs", "query_len", "num_q_heads", "num_kv_heads", "head_dim", "page_size", "num_pages",
        "table_stride", "q_dtype", "kv_dtype", "v_layout", "scale_mode", "causal", "sliding_window",
        "has_sinks", "token_table")] + [("softmax_scale", ctypes.c_float), ("index_stride", ctypes.c_int32)]


class PaPlanOpts(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("cu_count", "max_partitions", "partition_tokens", "stage_limit",
                                              "refreshable", "merge")]

MERGE_AUTO, MERGE_REDUCER, MERGE_IN_KERNEL = 0, 1, 2


class PaPlanInfo(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "num_items", "num_slots", "num_reduce", "rows_per_group", "row_groups", "max_parts", "total_tiles",
        "cu_count")]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libpa.so; raises ImportError if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libpa.so not found at {path}: build it with paged_attention_decode_plan_amd.build")
    L = ctypes.CDLL(path)
    vp = ctypes.c_void_p
    L.pa_plan.restype = ctypes.c_int
    L.pa_plan.argtypes = [ctypes.POINTER(PaProblem), vp, ctypes.POINTER(PaPlanOpts), ctypes.POINTER(vp)]
    L.pa_plan_sizes.restype = ctypes.c_int
    L.pa_plan_sizes.argtypes = [vp, ctypes.POINTER(ctypes.c_size_t), ctypes.POINTER(ctypes.c_size_t)]
    L.pa_plan_info.restype = ctypes.c_int
    L.pa_plan_info.argtypes = [vp, ctypes.POINTER(PaPlanInfo)]
    L.pa_plan_work.restype = ctypes.c_int
    L.pa_plan_work.argtypes = [vp, vp, ctypes.c_int32]
    L.pa_plan_upload.restype = ctypes.c_int
    L.pa_plan_upload.argtypes = [vp, vp, vp]
    L.pa_plan_free.restype = None
    L.pa_plan_free.argtypes = [vp]
    L.pa_decode.restype = ctypes.c_int
    L.pa_decode.argtypes = [vp] * 13
    L.pa_reduce.restype = ctypes.c_int
    L.pa_reduce.argtypes = [vp] * 6
    L.pa_plan_refresh.restype = ctypes.c_int
    L.pa_plan_refresh.argtypes = [vp] * 4
    L.pa_decode_sparse.restype = ctypes.c_int
    L.pa_decode_sparse.argtypes = [vp] * 14
    L.pa_mqa_logits.restype = ctypes.c_int
    L.pa_mqa_logits.argtypes = [vp] * 7 + [ctypes.c_int32] * 4 + [ctypes.c_int64, ctypes.c_int32, vp]
    L.pa_topk.restype = ctypes.c_int
    L.pa_topk.argtypes = [vp] * 5 + [ctypes.c_int32] * 2 + [ctypes.c_int64, ctypes.c_int32, vp, ctypes.c_size_t, vp]
    L.pa_topk_workspace_size.restype = ctypes.c_int
    L.pa_topk_workspace_size.argtypes = [ctypes.c_int32] * 3 + [ctypes.POINTER(ctypes.c_size_t)]
    L.pa_attend_static.restype = ctypes.c_int
    L.pa_attend_static.argtypes = [vp] * 11
    L.pa_last_error.restype = ctypes.c_char_p
    L.pa_last_error.argtypes = []
    _lib = L
    return L


def _check(st: int):
    if st == PA_OK:
        return
    msg = load_library().pa_last_error().decode()
    if st == PA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if st in (PA_ERR_INVALID, PA_ERR_WORKSPACE):
        raise ValueError(msg)
    raise RuntimeError(f"status {st}: {msg}")


def make_problem(num_seqs, query_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, table_stride,
                 q_dtype="bf16", kv_dtype="fp8", v_transposed=False, scale_mode="tensor", causal=True,
                 sliding_window=0, has_sinks=False, token_table=0, softmax_scale=0.0, index_stride=0) -> PaProblem:
    dt = {"bf16": PA_BF16, "fp16": PA_FP16, "fp8": PA_FP8_E4M3FN, "mxfp4": PA_MXFP4}
    sm = {"none": PA_SCALE_NONE, "tensor": PA_SCALE_PER_TENSOR, "token": PA_SCALE_PER_TOKEN, "mx": PA_SCALE_MX}
    return PaProblem(num_seqs, query_len, num_q_heads, num_kv_heads, head_dim, page_size, num_pages, table_stride,
                     dt[q_dtype], dt[kv_dtype], PA_V_TRANSPOSED if v_transposed else PA_V_PLAIN, sm[scale_mode],
                     int(causal), int(sliding_window), int(has_sinks), int(token_table), float(softmax_scale),
                     int(index_stride))


def problem_of(p) -> PaProblem:
    """PaProblem from any object with the problem's attribute names."""
    return make_problem(p.num_seqs, p.query_len, p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size,
                        p.num_pages, p.table_stride, p.q_dtype, p.kv_dtype, p.v_transposed, p.scale_mode, p.causal,
                        p.sliding_window, p.has_sinks, p.token_table, p.softmax_scale,
                        getattr(p, "index_stride", 0))


class Plan:
    """Owns a pa_plan_t plus the device metadata and workspace it needs."""

    def __init__(self, problem: PaProblem, context_lens_host, cu_count=0, max_partitions=0, partition_tokens=0,
                 stage_limit=0, refreshable=0, merge=MERGE_AUTO):
        L = load_library()
        self.problem = problem
        lens = torch.as_tensor(context_lens_host, dtype=torch.int32).contiguous().cpu()
        self._lens = lens
        opts = PaPlanOpts(cu_count, max_partitions, partition_tokens, stage_limit, refreshable, merge)
        h = ctypes.c_void_p()
        _check(L.pa_plan(ctypes.byref(problem), lens.data_ptr() if lens.numel() else None, ctypes.byref(opts),
                         ctypes.byref(h)))
        self.handle = h
        mb, wb = ctypes.c_size_t(), ctypes.c_size_t()
        _check(L.pa_plan_sizes(h, ctypes.byref(mb), ctypes.byref(wb)))
        self.meta_bytes, self.workspace_bytes = mb.value, wb.value
        self.meta = None
        self.workspace = None

    def info(self) -> PaPlanInfo:
        inf = PaPlanInfo()
        _check(load_library().pa_plan_info(self.handle, ctypes.byref(inf)))
        return inf

    def work(self) -> torch.Tensor:
        n = self.info().num_items
        out = torch.zeros((max(n, 1), 8), dtype=torch.int32)
        _check(load_library().pa_plan_work(self.handle, out.data_ptr(), n))
        return out[:n]

    def allocate(self, device="cuda", stream=None):
        """Device metadata and workspace (16-byte aligned torch allocations),
        and the metadata upload (pa_plan_upload) on `stream`."""
        self.meta = torch.empty(max(self.meta_bytes, 16), dtype=torch.uint8, device=device)
        self.workspace = torch.empty(max(self.workspace_bytes // 4, 4), dtype=torch.float32, device=device)
        self.upload(stream)
        return self

    def upload(self, stream=None):
        """Copy the plan's metadata into self.meta (needed again only if the
        buffer has since held another plan's list)."""
        _check(load_library().pa_plan_upload(self.handle, _ptr(self.meta), _stream_ptr(stream)))

    def work_list_device(self) -> torch.Tensor:
        """The work list as it is in self.meta (int32 [num_items, 8])."""
        n = self.info().num_items
        return self.meta[META_HEADER_BYTES: META_HEADER_BYTES + 32 * n].view(torch.int32).view(n, 8)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h is not None and h.value:
            try:
                load_library().pa_plan_free(h)
            except Exception:
                pass
            self.handle = None


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream_ptr(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def pa_decode(plan: Plan, out, q, k_cache, v_cache, block_tables, context_lens, k_scale=None, v_scale=None,
              sinks=None, stream=None):
    _check_decode_args(out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, sinks)
    if plan.meta is None:
        plan.allocate(q.device)
    _check(load_library().pa_decode(plan.handle, _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                    _ptr(block_tables), _ptr(context_lens), _ptr(k_scale), _ptr(v_scale),
                                    _ptr(sinks), _ptr(plan.meta), _ptr(plan.workspace), _stream_ptr(stream)))


def pa_decode_sparse(plan: Plan, out, q, k_cache, v_cache, block_tables, topk_indices, topk_counts, k_scale=None,
                     v_scale=None, sinks=None, stream=None):
    """Two-level sparse decode: rows attend their top-k logical positions
    (int32 [rows, index_stride], the first topk_counts[r] valid), resolved
    through block_tables."""
    _check_decode_args(out, q, k_cache, v_cache, block_tables, topk_counts, k_scale, v_scale, sinks)
    if not topk_indices.is_cuda or not topk_indices.is_contiguous() or topk_indices.dtype != torch.int32:
        raise ValueError("topk_indices must be a contiguous int32 device tensor")
    if plan.meta is None:
        plan.allocate(q.device)
    _check(load_library().pa_decode_sparse(plan.handle, _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_tables), _ptr(topk_indices), _ptr(topk_counts), _ptr(k_scale),
                                           _ptr(v_scale), _ptr(sinks), _ptr(plan.meta), _ptr(plan.workspace),
                                           _stream_ptr(stream)))


def pa_reduce(plan: Plan, out, sinks=None, stream=None):
    _check(load_library().pa_reduce(plan.handle, _ptr(out), _ptr(sinks), _ptr(plan.meta), _ptr(plan.workspace),
                                    _stream_ptr(stream)))


def pa_plan_refresh(plan: Plan, context_lens, stream=None):
    """Re-partition a refreshable plan on the device from device lengths."""
    if not context_lens.is_cuda or context_lens.dtype != torch.int32:
        raise ValueError("context_lens must be an int32 device tensor")
    if plan.meta is None:
        plan.allocate(context_lens.device)
    _check(load_library().pa_plan_refresh(plan.handle, _ptr(context_lens), _ptr(plan.meta), _stream_ptr(stream)))


def _check_decode_args(out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, sinks):
    for name, t in (("out", out), ("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                    ("block_tables", block_tables), ("context_lens", context_lens)):
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if block_tables.dtype != torch.int32 or context_lens.dtype != torch.int32:
        raise ValueError("block_tables and context_lens must be int32")
    if out.shape != q.shape or out.dtype != q.dtype:
        raise ValueError("out must match q in shape and dtype")
    for name, t in (("k_scale", k_scale), ("v_scale", v_scale)):
        # float32 scales, or the E8M0 bytes of MXFP4 caches
        if t is not None and (t.dtype not in (torch.float32, torch.uint8) or not t.is_contiguous() or not t.is_cuda):
            raise ValueError(f"{name} must be a contiguous float32 (uint8 for MXFP4) device tensor")
    if sinks is not None and (sinks.dtype != torch.float32 or not sinks.is_contiguous() or not sinks.is_cuda):
        raise ValueError("sinks must be a contiguous float32 device tensor")


def pa_attend_static(plan: Plan, out, q, k_cache, v_cache, block_tables, context_lens, k_scale=None, v_scale=None,
                     sinks=None, stream=None):
    """pa_decode + pa_reduce with the metadata and partials in the library's
    static device array (no device allocation; plan.meta / plan.workspace
    are not used)."""
    _check_decode_args(out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, sinks)
    _check(load_library().pa_attend_static(plan.handle, _ptr(out), _ptr(q), _ptr(k_cache), _ptr(v_cache),
                                           _ptr(block_tables), _ptr(context_lens), _ptr(k_scale), _ptr(v_scale),
                                           _ptr(sinks), _stream_ptr(stream)))
    return out


def attend(plan: Plan, out, q, k_cache, v_cache, block_tables, context_lens, k_scale=None, v_scale=None, sinks=None,
           stream=None):
    """pa_decode followed by pa_reduce on the same stream."""
    pa_decode(plan, out, q, k_cache, v_cache, block_tables, context_lens, k_scale, v_scale, sinks, stream)
    pa_reduce(plan, out, sinks, stream)
    return out


def _dev_i32(t, name):
    if not t.is_cuda or not t.is_contiguous() or t.dtype != torch.int32:
        raise ValueError(f"{name} must be a contiguous int32 device tensor")


def pa_mqa_logits(logits, q, kv, kv_scale, weights, ks, ke, clean=True, stream=None):
    """FP8 MQA logits (pa_indexer.h): logits float32 [rows, >= num_kv] (row
    stride = its second dim), q uint8 FP8 codes [rows, heads, 128], kv uint8
    [num_kv, 128], kv_scale float32 [num_kv], weights float32 [rows, heads],
    ks / ke int32 [rows]."""
    rows, heads, dim = q.shape
    num_kv = kv.shape[0]
    for t, name, dt in ((q, "q", torch.uint8), (kv, "kv", torch.uint8), (kv_scale, "kv_scale", torch.float32),
                        (weights, "weights", torch.float32), (logits, "logits", torch.float32)):
        if not t.is_cuda or t.dtype != dt:
            raise ValueError(f"{name} must be a {dt} device tensor")
        if t is not logits and not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    _dev_i32(ks, "ks")
    _dev_i32(ke, "ke")
    if kv.shape[1] != dim or weights.shape != (rows, heads) or kv_scale.shape != (num_kv,):
        raise ValueError("q, kv, kv_scale and weights shapes disagree")
    if ks.shape != (rows,) or ke.shape != (rows,):
        raise ValueError("ks and ke must be [rows]")
    if logits.dim() != 2 or logits.shape[0] != rows or logits.shape[1] < num_kv or logits.stride(1) != 1:
        raise ValueError("logits must be [rows, >= num_kv] with unit column stride")
    _check(load_library().pa_mqa_logits(_ptr(logits), _ptr(q), _ptr(kv), _ptr(kv_scale), _ptr(weights), _ptr(ks),
                                        _ptr(ke), rows, num_kv, heads, dim, logits.stride(0), int(bool(clean)),
                                        _stream_ptr(stream)))


def topk_workspace_bytes(rows: int, num_kv: int, k: int) -> int:
    n = ctypes.c_size_t()
    _check(load_library().pa_topk_workspace_size(rows, num_kv, k, ctypes.byref(n)))
    return n.value


def pa_topk(indices, counts, logits, ks, ke, num_kv=None, stream=None, workspace=None):
    """Top-k of each row's window (pa_indexer.h): indices int32 [rows, k],
    counts int32 [rows], logits float32 [rows, >= num_kv]; workspace: a
    device tensor of at least topk_workspace_bytes (allocated here if
    None)."""
    rows, k = indices.shape
    num_kv = logits.shape[1] if num_kv is None else num_kv
    need = topk_workspace_bytes(rows, num_kv, k)
    if workspace is None and need > 0:
        workspace = torch.empty(need, dtype=torch.uint8, device=indices.device)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _dev_i32(indices, "indices")
    _dev_i32(counts, "counts")
    _dev_i32(ks, "ks")
    _dev_i32(ke, "ke")
    if not logits.is_cuda or logits.dtype != torch.float32 or logits.stride(1) != 1 or logits.shape[0] != rows:
        raise ValueError("logits must be a float32 device tensor [rows, >= num_kv] with unit column stride")
    if counts.shape != (rows,) or ks.shape != (rows,) or ke.shape != (rows,) or num_kv > logits.shape[1]:
        raise ValueError("counts, ks and ke must be [rows]; num_kv at most logits.shape[1]")
    _check(load_library().pa_topk(_ptr(indices), _ptr(counts), _ptr(logits), _ptr(ks), _ptr(ke), rows, num_kv,
                                  logits.stride(0), k, _ptr(workspace), wbytes, _stream_ptr(stream)))
