"""ctypes front end of the fp64 CPU oracle (oracle/ts_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the smoke check
and the benchmark's CPU-baseline leg may import this module.  It depends on
numpy only; it imports nothing from the HIP package and the HIP package never
imports it.

Inputs are numpy arrays: q, k, v as uint16 bf16 bit patterns in the packed
layout [T, heads, head_dim]; sinks as float32 [n_q_heads] or None; cu_seqlens
as int32 [n_seqs + 1].  The cache form (cache_attend) takes k_cache / v_cache
as uint16 [n_pages, page_size, n_kv_heads, head_dim], seqlens_k as int32
[n_seqs] and block_table as int32 [n_seqs, pages_per_seq].  Outputs are
float64.  The arithmetic lives in the C file; see its header for what is
computed and which pages it follows.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ts_oracle.c")
_LIB = os.path.join(_HERE, "libts_oracle.so")

_lib = None


def build(src: str = _SRC, out: str = _LIB, extra_flags: tuple = ()) -> str:
    """Compile the oracle with gcc (plain -O2, OpenMP, no fast-math)."""
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall", "-Wextra",
           *extra_flags, src, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def load(path: str = _LIB, build_if_missing: bool = True):
    """Load (building first if absent) and declare the oracle's C entry points."""
    global _lib
    if path == _LIB and _lib is not None:
        return _lib
    if not os.path.exists(path):
        if not build_if_missing:
            raise FileNotFoundError(path)
        build(out=path)
    lib = ctypes.CDLL(path)
    u16p = ctypes.POINTER(ctypes.c_uint16)
    f32p = ctypes.POINTER(ctypes.c_float)
    i32p = ctypes.POINTER(ctypes.c_int32)
    i64p = ctypes.POINTER(ctypes.c_int64)
    f64p = ctypes.POINTER(ctypes.c_double)
    common = [u16p, u16p, u16p, f32p, i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
              ctypes.c_int32, ctypes.c_int32, ctypes.c_double]
    lib.ts_oracle_prefill.argtypes = common + [f64p]
    lib.ts_oracle_prefill.restype = ctypes.c_int
    lib.ts_oracle_prefill_rows.argtypes = common + [i64p, i32p, ctypes.c_int64, f64p]
    lib.ts_oracle_prefill_rows.restype = ctypes.c_int
    lib.ts_oracle_row_probs.argtypes = common + [ctypes.c_int64, ctypes.c_int32, f64p, f64p]
    lib.ts_oracle_row_probs.restype = ctypes.c_int
    lib.ts_oracle_cache.argtypes = [u16p, u16p, u16p, f32p, i32p, i32p, i32p, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_double,
                                    i64p, i32p, ctypes.c_int64, f64p]
    lib.ts_oracle_cache.restype = ctypes.c_int
    if path == _LIB:
        _lib = lib
    return lib


def _ptr(a, ctype):
    return None if a is None else a.ctypes.data_as(ctypes.POINTER(ctype))


def _prep(q, k, v, sinks, cu_seqlens):
    q = np.ascontiguousarray(q, dtype=np.uint16)
    k = np.ascontiguousarray(k, dtype=np.uint16)
    v = np.ascontiguousarray(v, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int32)
    s = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3 or k.shape != v.shape:
        raise ValueError("q, k, v must be [T, heads, head_dim] with k.shape == v.shape")
    if q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q and k/v must share T and head_dim")
    if cu.ndim != 1 or cu.shape[0] < 1 or int(cu[-1]) != q.shape[0]:
        raise ValueError("cu_seqlens must be [n_seqs + 1] ending at T")
    if s is not None and s.shape != (q.shape[1],):
        raise ValueError("sinks must be [n_q_heads]")
    return q, k, v, s, cu


def _common_args(q, k, v, s, cu, window, scale):
    return (_ptr(q, ctypes.c_uint16), _ptr(k, ctypes.c_uint16), _ptr(v, ctypes.c_uint16),
            _ptr(s, ctypes.c_float), _ptr(cu, ctypes.c_int32), cu.shape[0] - 1,
            q.shape[1], k.shape[1], q.shape[2], int(window), float(scale))


def _check(rc, what):
    if rc != 0:
        raise ValueError(f"{what} rejected its arguments (code {rc})")


def prefill(q, k, v, sinks, cu_seqlens, window: int, scale: float, lib=None) -> np.ndarray:
    """Every output row, float64 [T, n_q_heads, head_dim]."""
    lib = lib or load()
    q, k, v, s, cu = _prep(q, k, v, sinks, cu_seqlens)
    out = np.zeros(q.shape, dtype=np.float64)
    _check(lib.ts_oracle_prefill(*_common_args(q, k, v, s, cu, window, scale),
                                 _ptr(out, ctypes.c_double)), "ts_oracle_prefill")
    return out


def prefill_rows(q, k, v, sinks, cu_seqlens, window: int, scale: float, rows, heads,
                 lib=None) -> np.ndarray:
    """Selected rows: float64 [n, head_dim] for (packed row rows[n], head heads[n])."""
    lib = lib or load()
    q, k, v, s, cu = _prep(q, k, v, sinks, cu_seqlens)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    heads = np.ascontiguousarray(heads, dtype=np.int32)
    if rows.shape != heads.shape or rows.ndim != 1:
        raise ValueError("rows and heads must be 1-D and of equal length")
    out = np.zeros((rows.shape[0], q.shape[2]), dtype=np.float64)
    _check(lib.ts_oracle_prefill_rows(*_common_args(q, k, v, s, cu, window, scale),
                                      _ptr(rows, ctypes.c_int64), _ptr(heads, ctypes.c_int32),
                                      rows.shape[0], _ptr(out, ctypes.c_double)),
           "ts_oracle_prefill_rows")
    return out


def row_probs(q, k, v, sinks, cu_seqlens, window: int, scale: float, row: int, head: int,
              lib=None):
    """(probs over key positions 0..i of the row's sequence, sink share)."""
    lib = lib or load()
    q, k, v, s, cu = _prep(q, k, v, sinks, cu_seqlens)
    b = int(np.searchsorted(cu, row, side="right")) - 1
    i = row - int(cu[b])
    probs = np.zeros(i + 1, dtype=np.float64)
    p_sink = ctypes.c_double(0.0)
    _check(lib.ts_oracle_row_probs(*_common_args(q, k, v, s, cu, window, scale), int(row),
                                   int(head), _ptr(probs, ctypes.c_double),
                                   ctypes.byref(p_sink)), "ts_oracle_row_probs")
    return probs, p_sink.value


def cache_attend(q, k_cache, v_cache, sinks, cu_seqlens_q, seqlens_k, block_table, window: int,
                 scale: float, rows=None, heads=None, lib=None) -> np.ndarray:
    """New query rows against a paged KV cache (prefill with a cache; decode is q_len = 1).

    Row i of sequence b's q_len rows sits at position seqlens_k[b] - q_len + i.
    Returns float64 [Tq, n_q_heads, head_dim], or [n, head_dim] for the selected
    (rows[n], heads[n]).
    """
    lib = lib or load()
    q = np.ascontiguousarray(q, dtype=np.uint16)
    kc = np.ascontiguousarray(k_cache, dtype=np.uint16)
    vc = np.ascontiguousarray(v_cache, dtype=np.uint16)
    cu = np.ascontiguousarray(cu_seqlens_q, dtype=np.int32)
    sk = np.ascontiguousarray(seqlens_k, dtype=np.int32)
    bt = np.ascontiguousarray(block_table, dtype=np.int32)
    s = None if sinks is None else np.ascontiguousarray(sinks, dtype=np.float32)
    if q.ndim != 3 or kc.ndim != 4 or kc.shape != vc.shape or kc.shape[3] != q.shape[2]:
        raise ValueError("q must be [Tq, Hq, D] and k/v caches [n_pages, page_size, Hkv, D]")
    if cu.ndim != 1 or cu.shape[0] < 1 or int(cu[-1]) != q.shape[0]:
        raise ValueError("cu_seqlens_q must be [n_seqs + 1] ending at Tq")
    n_seqs = cu.shape[0] - 1
    if sk.shape != (n_seqs,) or bt.ndim != 2 or bt.shape[0] != n_seqs:
        raise ValueError("seqlens_k must be [n_seqs] and block_table [n_seqs, pages_per_seq]")
    if s is not None and s.shape != (q.shape[1],):
        raise ValueError("sinks must be [n_q_heads]")
    hq, D = q.shape[1], q.shape[2]
    if rows is None:
        r = h = None
        out = np.zeros(q.shape, dtype=np.float64)
        n = 0
    else:
        r = np.ascontiguousarray(rows, dtype=np.int64)
        h = np.ascontiguousarray(heads, dtype=np.int32)
        if r.shape != h.shape or r.ndim != 1:
            raise ValueError("rows and heads must be 1-D and of equal length")
        out = np.zeros((r.shape[0], D), dtype=np.float64)
        n = r.shape[0]
    _check(lib.ts_oracle_cache(_ptr(q, ctypes.c_uint16), _ptr(kc, ctypes.c_uint16),
                               _ptr(vc, ctypes.c_uint16), _ptr(s, ctypes.c_float),
                               _ptr(cu, ctypes.c_int32), _ptr(sk, ctypes.c_int32),
                               _ptr(bt, ctypes.c_int32), n_seqs, kc.shape[0], kc.shape[1],
                               bt.shape[1], hq, kc.shape[2], D, int(window), float(scale),
                               _ptr(r, ctypes.c_int64), _ptr(h, ctypes.c_int32), n,
                               _ptr(out, ctypes.c_double)), "ts_oracle_cache")
    return out
