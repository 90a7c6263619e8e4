"""Thin ctypes binding over libts_mha.so (declared in include/ts_mha.h).

Argument marshalling only: shapes, dtypes and devices of torch tensors are
checked and turned into the C call's pointers and sizes; every step of the
attention runs in the library's HIP kernels.  There is no fallback: if the
library is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
# TS_MHA_LIBRARY names another build of the same library (the tests use it for a
# build whose host code carries the address and undefined-behaviour sanitizers).
LIB_PATH = os.environ.get("TS_MHA_LIBRARY") or os.path.join(_PKG, "libts_mha.so")

TS_MHA_OK = 0
ERROR_NAMES = {
    -1: "TS_MHA_ERR_NULL_ARG", -2: "TS_MHA_ERR_BAD_SHAPE", -3: "TS_MHA_ERR_UNSUPPORTED",
    -4: "TS_MHA_ERR_BAD_SCALE", -5: "TS_MHA_ERR_ALIGN", -6: "TS_MHA_ERR_NO_DEVICE",
    -7: "TS_MHA_ERR_ARCH", -8: "TS_MHA_ERR_LAUNCH", -9: "TS_MHA_ERR_SEQLENS",
    -10: "TS_MHA_ERR_WORKSPACE", -11: "TS_MHA_ERR_PAGES",
}

_lib = None


class TsMhaError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERROR_NAMES.get(code, code)}: {message}")
        self.code = code


def lib() -> ctypes.CDLL:
    """Load libts_mha.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m sinks_ts_mha_amd.build` (hipcc, gfx950)")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
        L.ts_mha_prefill.argtypes = [vp, vp, vp, vp, vp, i32, i32, i32, i32, ctypes.c_float,
                                     vp, i32, i32, vp]
        L.ts_mha_prefill.restype = ctypes.c_int
        L.ts_mha_strerror.argtypes = [ctypes.c_int]
        L.ts_mha_strerror.restype = ctypes.c_char_p
        L.ts_mha_unmasked_pairs.argtypes = [ctypes.POINTER(ctypes.c_int32), i32, i32]
        L.ts_mha_unmasked_pairs.restype = i64
        L.ts_mha_decode_with_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                 ctypes.c_float, vp, i32, i32, i32, i32, i32, vp,
                                                 i64, vp]
        L.ts_mha_decode_with_kvcache.restype = ctypes.c_int
        L.ts_mha_prefill_with_kvcache.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                  ctypes.c_float, vp, i32, i32, i32, i32, i32, i32,
                                                  vp]
        L.ts_mha_prefill_with_kvcache.restype = ctypes.c_int
        L.ts_mha_decode_with_kvcache_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32,
                                                         ctypes.c_float, vp, i32, i32, i32, i32, i32,
                                                         vp]
        L.ts_mha_decode_with_kvcache_noalloc.restype = ctypes.c_int
        L.ts_mha_decode_workspace_size.argtypes = [i32, i32, i32, i32, i32, i32]
        L.ts_mha_decode_workspace_size.restype = i64
        _lib = L
    return _lib


def ts_mha_strerror(code: int) -> str:
    return lib().ts_mha_strerror(int(code)).decode()


def ts_mha_unmasked_pairs(cu_seqlens, window: int = 0) -> int:
    """Visible (query, key) pairs per head for host cu_seqlens (sequence or CPU tensor)."""
    cu = torch.as_tensor(cu_seqlens, dtype=torch.int32).cpu().contiguous()
    n = int(cu.numel()) - 1
    r = lib().ts_mha_unmasked_pairs(ctypes.cast(cu.data_ptr(), ctypes.POINTER(ctypes.c_int32)),
                                    n, int(window))
    if r < 0:
        raise ValueError("ts_mha_unmasked_pairs rejected cu_seqlens")
    return int(r)


def _check_no_overlap(out: torch.Tensor, inputs) -> None:
    """Raise if out's bytes overlap those of any (name, tensor) in inputs (None skipped)."""
    o0 = out.data_ptr()
    o1 = o0 + out.numel() * out.element_size()
    if o1 == o0:
        return
    for name, t in inputs:
        if t is None:
            continue
        t0 = t.data_ptr()
        t1 = t0 + t.numel() * t.element_size()
        if t0 < o1 and o0 < t1 and t1 > t0:
            raise ValueError(f"out must not overlap {name}")


def ts_mha_prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, sinks, cu_seqlens,
                   window: int = 0, softmax_scale: float | None = None, out=None,
                   max_seqlen: int | None = None, stream=None) -> torch.Tensor:
    """Causal GQA prefill attention with optional sinks and sliding window.

    q [T, Hq, 64], k/v [T, Hkv, 64] bf16 CUDA tensors; sinks fp32 [Hq] or None;
    cu_seqlens int32 [n_seqs + 1] on the same device.  max_seqlen (the longest
    sequence) sizes the launch; if omitted it is read back from cu_seqlens,
    which synchronises.  softmax_scale defaults to 1/sqrt(head_dim).  Runs on
    `stream` (default: torch's current stream) and returns `out`.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 3:
            raise TypeError(f"{name} must be a 3-D bfloat16 tensor")
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("shapes must be q [T, Hq, D], k = v [T, Hkv, D]")
    dev = q.device
    if k.device != dev or v.device != dev:
        raise ValueError("q, k, v must be on one device")
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dtype != torch.int32 \
            or cu_seqlens.dim() != 1 or cu_seqlens.device != dev or not cu_seqlens.is_contiguous():
        raise TypeError("cu_seqlens must be a contiguous int32 1-D tensor on q's device")
    if sinks is not None:
        if not isinstance(sinks, torch.Tensor) or sinks.dtype != torch.float32 \
                or sinks.shape != (q.shape[1],) or sinks.device != dev or not sinks.is_contiguous():
            raise TypeError("sinks must be None or a contiguous float32 [Hq] tensor on q's device")
    T, hq, D = q.shape
    hkv = k.shape[1]
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != torch.bfloat16 or out.device != dev \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 tensor shaped like q on q's device")
    _check_no_overlap(out, (("q", q), ("k", k), ("v", v), ("cu_seqlens", cu_seqlens), ("sinks", sinks)))
    if softmax_scale is None:
        softmax_scale = 1.0 / (D ** 0.5)
    if T == 0:  # no rows: nothing to compute or write (torch gives empty tensors no address)
        return out
    n_seqs = cu_seqlens.numel() - 1
    if max_seqlen is None:
        cu = cu_seqlens.cpu()
        max_seqlen = int((cu[1:] - cu[:-1]).max()) if n_seqs > 0 else 0
    handle = _stream_handle(stream, dev)
    rc = lib().ts_mha_prefill(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                              None if sinks is None else sinks.data_ptr(),
                              cu_seqlens.data_ptr(), hq, hkv, D, int(window), float(softmax_scale),
                              out.data_ptr(), n_seqs, int(max_seqlen), handle)
    if rc != TS_MHA_OK:
        raise TsMhaError(rc, ts_mha_strerror(rc))
    return out


def _check_tensor(name, t, dtype, dim, dev):
    if not isinstance(t, torch.Tensor) or t.dtype != dtype or t.dim() != dim:
        raise TypeError(f"{name} must be a {dim}-D {dtype} tensor")
    if t.device != dev or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous tensor on {dev}")


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream_handle(stream, dev):
    if stream is None:
        if _raw_stream is not None:  # the current stream's handle without a Stream object (~2 us less)
            return _raw_stream(dev.index if dev.index is not None else torch.cuda.current_device())
        stream = torch.cuda.current_stream(dev)
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _check_cache(q, k_cache, v_cache, sinks, seqlens_k, block_table, n_seqs):
    dev = q.device
    _check_tensor("q", q, torch.bfloat16, 3, dev)
    _check_tensor("k_cache", k_cache, torch.bfloat16, 4, dev)
    _check_tensor("v_cache", v_cache, torch.bfloat16, 4, dev)
    _check_tensor("seqlens_k", seqlens_k, torch.int32, 1, dev)
    _check_tensor("block_table", block_table, torch.int32, 2, dev)
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    if v_cache.shape != k_cache.shape or k_cache.shape[3] != q.shape[2]:
        raise ValueError("k_cache and v_cache must both be [n_pages, page_size, Hkv, D]")
    if seqlens_k.shape != (n_seqs,) or block_table.shape[0] != n_seqs:
        raise ValueError("seqlens_k must be [n_seqs] and block_table [n_seqs, pages_per_seq]")
    if sinks is not None:
        _check_tensor("sinks", sinks, torch.float32, 1, dev)
        if sinks.shape != (q.shape[1],):
            raise ValueError("sinks must be [Hq]")


def _check_out(out, q, inputs):
    if out is None:
        out = torch.empty_like(q)
    else:
        _check_tensor("out", out, torch.bfloat16, 3, q.device)
        if out.shape != q.shape:
            raise ValueError("out must be shaped like q")
    _check_no_overlap(out, inputs)
    return out


def ts_mha_prefill_with_kvcache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                sinks, cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor,
                                block_table: torch.Tensor, window: int = 0,
                                softmax_scale: float | None = None, out=None,
                                max_seqlen_q: int | None = None, max_seqlen_k: int | None = None,
                                stream=None) -> torch.Tensor:
    """Prefill of new query rows against a paged KV cache (chunked prefill).

    q [Tq, Hq, 64] bf16 packed by cu_seqlens_q (int32 [n_seqs + 1]); the caches
    [n_pages, page_size, Hkv, 64] bf16 already hold the new rows' keys and values;
    seqlens_k int32 [n_seqs] counts every cached key; block_table int32
    [n_seqs, pages_per_seq].  Row i of a sequence with q_len new rows sits at
    position seqlens_k - q_len + i.  max_seqlen_q / max_seqlen_k size the launch;
    if omitted they are read back (synchronising).
    """
    dev = q.device
    _check_tensor("cu_seqlens_q", cu_seqlens_q, torch.int32, 1, dev)
    n_seqs = cu_seqlens_q.numel() - 1
    _check_cache(q, k_cache, v_cache, sinks, seqlens_k, block_table, n_seqs)
    out = _check_out(out, q, (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                              ("cu_seqlens_q", cu_seqlens_q), ("seqlens_k", seqlens_k),
                              ("block_table", block_table), ("sinks", sinks)))
    Tq, hq, D = q.shape
    n_pages, page_size, hkv, _ = k_cache.shape
    if softmax_scale is None:
        softmax_scale = 1.0 / (D ** 0.5)
    if Tq == 0:
        return out
    if max_seqlen_q is None:
        cu = cu_seqlens_q.cpu()
        max_seqlen_q = int((cu[1:] - cu[:-1]).max()) if n_seqs > 0 else 0
    if max_seqlen_k is None:
        max_seqlen_k = int(seqlens_k.max().cpu()) if n_seqs > 0 else 0
    rc = lib().ts_mha_prefill_with_kvcache(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if sinks is None else sinks.data_ptr(), cu_seqlens_q.data_ptr(), seqlens_k.data_ptr(),
        block_table.data_ptr(), hq, hkv, D, int(window), float(softmax_scale), out.data_ptr(),
        n_seqs, n_pages, page_size, block_table.shape[1], int(max_seqlen_q), int(max_seqlen_k),
        _stream_handle(stream, dev))
    if rc != TS_MHA_OK:
        raise TsMhaError(rc, ts_mha_strerror(rc))
    return out


def ts_mha_decode_workspace_size(n_seqs: int, n_q_heads: int, n_kv_heads: int, head_dim: int = 64,
                                 window: int = 0, max_seqlen_k: int = 0) -> int:
    """Workspace bytes a decode call with these arguments needs (0: none)."""
    r = lib().ts_mha_decode_workspace_size(int(n_seqs), int(n_q_heads), int(n_kv_heads),
                                           int(head_dim), int(window), int(max_seqlen_k))
    if r < 0:
        raise TsMhaError(int(r), ts_mha_strerror(int(r)))
    return int(r)


def ts_mha_decode_with_kvcache(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                               sinks, seqlens_k: torch.Tensor, block_table: torch.Tensor,
                               window: int = 0, softmax_scale: float | None = None, out=None,
                               max_seqlen_k: int | None = None, workspace=None,
                               stream=None) -> torch.Tensor:
    """Decode attention of one new query row per sequence against a paged KV cache.

    q [B, Hq, 64] bf16; k_cache / v_cache [n_pages, page_size, Hkv, 64] bf16;
    seqlens_k int32 [B] (cached keys, the new token's own included); block_table
    int32 [B, pages_per_seq]; sinks fp32 [Hq] or None.  max_seqlen_k sizes the
    launch; if omitted it is read back from seqlens_k (synchronising).  The
    workspace for long sequences is taken from `workspace` (a uint8 tensor) or
    allocated here.  Runs on `stream` (default: torch's current stream).
    """
    dev = q.device
    B, hq, D = q.shape
    _check_cache(q, k_cache, v_cache, sinks, seqlens_k, block_table, B)
    n_pages, page_size, hkv, _ = k_cache.shape
    out = _check_out(out, q, (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                              ("seqlens_k", seqlens_k), ("block_table", block_table),
                              ("sinks", sinks)))
    if softmax_scale is None:
        softmax_scale = 1.0 / (D ** 0.5)
    if B == 0:
        return out
    if max_seqlen_k is None:
        max_seqlen_k = int(seqlens_k.max().cpu())
    need = ts_mha_decode_workspace_size(B, hq, hkv, D, window, max_seqlen_k)
    if need > 0:
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=dev)
        elif not isinstance(workspace, torch.Tensor) or workspace.device != dev \
                or workspace.numel() * workspace.element_size() < need or not workspace.is_contiguous():
            raise ValueError(f"workspace must be a contiguous tensor of at least {need} bytes on {dev}")
    ws_ptr = workspace.data_ptr() if (workspace is not None and need > 0) else None
    ws_bytes = workspace.numel() * workspace.element_size() if ws_ptr else 0
    rc = lib().ts_mha_decode_with_kvcache(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if sinks is None else sinks.data_ptr(), seqlens_k.data_ptr(), block_table.data_ptr(),
        hq, hkv, D, int(window), float(softmax_scale), out.data_ptr(), B, n_pages, page_size,
        block_table.shape[1], int(max_seqlen_k), ws_ptr, ws_bytes, _stream_handle(stream, dev))
    if rc != TS_MHA_OK:
        raise TsMhaError(rc, ts_mha_strerror(rc))
    return out


NOALLOC_SCRATCH_BYTES = 16 * 1024 * 1024  # TS_MHA_NOALLOC_SCRATCH_BYTES


def ts_mha_decode_with_kvcache_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                                       sinks, seqlens_k: torch.Tensor, block_table: torch.Tensor,
                                       window: int = 0, softmax_scale: float | None = None, out=None,
                                       max_seqlen_k: int | None = None, stream=None) -> torch.Tensor:
    """ts_mha_decode_with_kvcache with the split partials in the library's own scratch
    (no workspace, no device allocation by the call; pass `out` to allocate nothing here
    either).  Calls that overlap on one GPU race on that scratch."""
    dev = q.device
    B, hq, D = q.shape
    _check_cache(q, k_cache, v_cache, sinks, seqlens_k, block_table, B)
    n_pages, page_size, hkv, _ = k_cache.shape
    out = _check_out(out, q, (("q", q), ("k_cache", k_cache), ("v_cache", v_cache),
                              ("seqlens_k", seqlens_k), ("block_table", block_table),
                              ("sinks", sinks)))
    if softmax_scale is None:
        softmax_scale = 1.0 / (D ** 0.5)
    if B == 0:
        return out
    if max_seqlen_k is None:
        max_seqlen_k = int(seqlens_k.max().cpu())
    rc = lib().ts_mha_decode_with_kvcache_noalloc(
        q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
        None if sinks is None else sinks.data_ptr(), seqlens_k.data_ptr(), block_table.data_ptr(),
        hq, hkv, D, int(window), float(softmax_scale), out.data_ptr(), B, n_pages, page_size,
        block_table.shape[1], int(max_seqlen_k), _stream_handle(stream, dev))
    if rc != TS_MHA_OK:
        raise TsMhaError(rc, ts_mha_strerror(rc))
    return out


# The operations' names in the public API the pages list.
mha_prefill = ts_mha_prefill
mha_decode_with_kvcache = ts_mha_decode_with_kvcache
mha_prefill_with_kvcache = ts_mha_prefill_with_kvcache
