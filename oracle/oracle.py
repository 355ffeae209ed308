"""Python binding of the CPU decode oracle (``pa_oracle.c``).

TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the benchmark's
CPU-baseline leg import this module; the product package never does.  It is
independent of the GPU library: it builds its own shared object from plain C
with gcc and shares no header, table or helper with it.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "pa_oracle.c")
_LIB = os.path.join(_HERE, "libpa_oracle.so")
_lock = threading.Lock()
_lib = None


class OrcProblem(ctypes.Structure):
    _fields_ = [
        ("num_seqs", ctypes.c_int), ("query_len", ctypes.c_int), ("num_q_heads", ctypes.c_int),
        ("num_kv_heads", ctypes.c_int), ("head_dim", ctypes.c_int), ("page_size", ctypes.c_int),
        ("num_pages", ctypes.c_int), ("table_stride", ctypes.c_int),
        ("q_kind", ctypes.c_int), ("kv_kind", ctypes.c_int), ("v_transposed", ctypes.c_int),
        ("scale_mode", ctypes.c_int), ("causal", ctypes.c_int), ("window", ctypes.c_int),
        ("has_sinks", ctypes.c_int), ("token_table", ctypes.c_int), ("softmax_scale", ctypes.c_double),
        ("index_stride", ctypes.c_int), ("topk", ctypes.c_void_p),
    ]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain C, -O2, pthreads)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            L.orc_fp8_e4m3fn.restype = ctypes.c_double
            L.orc_fp8_e4m3fn.argtypes = [ctypes.c_uint8]
            L.orc_bf16.restype = ctypes.c_double
            L.orc_bf16.argtypes = [ctypes.c_uint16]
            L.orc_fp16.restype = ctypes.c_double
            L.orc_fp16.argtypes = [ctypes.c_uint16]
            L.orc_fp4_e2m1.restype = ctypes.c_double
            L.orc_fp4_e2m1.argtypes = [ctypes.c_uint8]
            L.orc_e8m0.restype = ctypes.c_double
            L.orc_e8m0.argtypes = [ctypes.c_uint8]
            vp = ctypes.c_void_p
            L.orc_attend.restype = ctypes.c_int
            L.orc_attend.argtypes = [ctypes.POINTER(OrcProblem), vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                     ctypes.c_long, vp, ctypes.c_int]
            L.orc_partial.restype = None
            L.orc_partial.argtypes = [ctypes.POINTER(OrcProblem), vp, vp, vp, vp, vp, vp, vp] + [ctypes.c_int] * 5 + [
                vp, vp, vp]
            L.orc_merge.restype = None
            L.orc_merge.argtypes = [ctypes.c_int, vp, vp, vp, ctypes.c_int, ctypes.c_int, ctypes.c_double, vp]
            _lib = L
    return _lib


def fp8_value(code: int) -> float:
    return lib().orc_fp8_e4m3fn(code)


def fp4_value(code: int) -> float:
    return lib().orc_fp4_e2m1(code)


def e8m0_value(code: int) -> float:
    return lib().orc_e8m0(code)


def bf16_value(bits: int) -> float:
    return lib().orc_bf16(bits)


def fp16_value(bits: int) -> float:
    return lib().orc_fp16(bits)


def _problem(p, held=None) -> OrcProblem:
    return OrcProblem(
        p.num_seqs, p.query_len, p.num_q_heads, p.num_kv_heads, p.head_dim, p.page_size, p.num_pages,
        p.table_stride, 1 if p.q_dtype == "fp16" else 0, {"bf16": 0, "fp8": 2, "mxfp4": 3}[p.kv_dtype],
        int(p.v_transposed), {"none": 0, "tensor": 1, "token": 2, "mx": 3}[p.scale_mode], int(p.causal), int(p.sliding_window),
        int(p.has_sinks), int(p.token_table), float(p.scale), int(getattr(p, "index_stride", 0)),
        None if held is None else held.topk_ptr,
    )


class _Held:
    """Host views of an Inputs object that stay alive during a call."""

    def __init__(self, inp):
        def c(t):
            if t is None:
                return None
            t = t.contiguous()
            if t.dtype in (torch.bfloat16, torch.float16):
                t = t.view(torch.int16)
            return t.numpy()

        self.arrays = [c(inp.q), c(inp.k_cache), c(inp.v_cache), c(inp.block_tables), c(inp.context_lens),
                       c(inp.k_scale), c(inp.v_scale), c(inp.sinks)]
        self.ptrs = [None if a is None else a.ctypes.data for a in self.arrays]
        topk = getattr(inp, "topk_indices", None)
        self.topk = None if topk is None else np.ascontiguousarray(topk.cpu().numpy(), dtype=np.int32)
        self.topk_ptr = None if self.topk is None else self.topk.ctypes.data


def attend(inp, sel=None, nthreads: int | None = None, return_threads: bool = False):
    """Oracle output as float32: ``[rows, Hq, D]`` for sel None, else ``[n, D]``
    for ``sel`` an int array of (token_row, head) pairs."""
    L = lib()
    p = inp.problem
    held = _Held(inp)
    prob = _problem(p, held)
    if nthreads is None:
        nthreads = os.cpu_count() or 1
    if sel is None:
        out = np.zeros((p.rows, p.num_q_heads, p.head_dim), np.float32)
        sel_ptr, n = None, 0
    else:
        sel_a = np.ascontiguousarray(np.asarray(sel, dtype=np.int32).reshape(-1, 2))
        out = np.zeros((sel_a.shape[0], p.head_dim), np.float32)
        sel_ptr, n = sel_a.ctypes.data, sel_a.shape[0]
    used = L.orc_attend(ctypes.byref(prob), *held.ptrs, sel_ptr, n, out.ctypes.data, int(nthreads))
    return (out, used) if return_threads else out


def partial(inp, s: int, i: int, h: int, t_begin: int, t_end: int):
    """Unnormalised (m, l, o[D]) of one row over visible tokens in [t_begin, t_end)."""
    L = lib()
    p = inp.problem
    held = _Held(inp)
    prob = _problem(p, held)
    m = np.zeros(1, np.float64)
    l = np.zeros(1, np.float64)
    o = np.zeros(p.head_dim, np.float64)
    L.orc_partial(ctypes.byref(prob), *held.ptrs[:7], s, i, h, t_begin, t_end, m.ctypes.data, l.ctypes.data,
                  o.ctypes.data)
    return float(m[0]), float(l[0]), o


def merge(ms, ls, os_, sink=None):
    """Log-sum-exp merge of partial states in the given order."""
    L = lib()
    ms = np.ascontiguousarray(ms, dtype=np.float64)
    ls = np.ascontiguousarray(ls, dtype=np.float64)
    os_ = np.ascontiguousarray(os_, dtype=np.float64)
    D = os_.shape[-1]
    out = np.zeros(D, np.float64)
    L.orc_merge(len(ms), ms.ctypes.data, ls.ctypes.data, os_.ctypes.data, D, 0 if sink is None else 1,
                0.0 if sink is None else float(sink), out.ctypes.data)
    return out
