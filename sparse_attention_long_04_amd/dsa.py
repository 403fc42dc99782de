"""Thin ctypes binding of ``libdsa.so`` (declared in ``include/dsa.h``).

Argument marshalling only: every function here has the name of a C entry point, turns
tensors into device pointers and a stream into a ``hipStream_t``, calls the library and
raises :class:`DSAError` on a non-zero status.  All computation happens in the HIP kernels;
there is no fallback path.  If the library has not been built, the first call raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libdsa.so")
_lib = None

IDX_BF16 = 0
IDX_FP8_E4M3 = 1
_DTYPES = {"bf16": IDX_BF16, "fp8_e4m3": IDX_FP8_E4M3}


class DSAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = lib().dsa_status_string(status).decode()
        if status == 4:
            msg += f" (hipError {lib().dsa_last_hip_error()})"
        super().__init__(f"{where}: {msg} [{status}]")


class PrefillShape(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("cu_seqlens", ctypes.c_void_p),
                ("total_tokens", ctypes.c_int64), ("max_seqlen", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("idx_dtype", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


class DecodeShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("cache_capacity", ctypes.c_int32),
                ("cache_lens", ctypes.c_void_p), ("max_cache_len", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("idx_heads", ctypes.c_int32), ("idx_dim", ctypes.c_int32),
                ("idx_dtype", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("softmax_scale", ctypes.c_float)]


EXPORTS = {
    # name: (argtypes after the shape pointer / full argtypes, restype)
    "dsa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "dsa_last_hip_error": ([], ctypes.c_int),
    "dsa_prefill_workspace_size": ([ctypes.POINTER(PrefillShape), ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dsa_index_scores": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_index_topk": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_sparse_attention": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 6, ctypes.c_int),
    "dsa_prefill": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dense_causal_attention": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_decode_workspace_size": ([ctypes.POINTER(DecodeShape), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dsa_kv_append": ([ctypes.POINTER(DecodeShape)] + [ctypes.c_void_p] * 8, ctypes.c_int),
    "dsa_decode": ([ctypes.POINTER(DecodeShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_decode_noalloc": ([ctypes.POINTER(DecodeShape)] + [ctypes.c_void_p] * 9, ctypes.c_int),
    "dense_decode_attention": ([ctypes.POINTER(DecodeShape)] + [ctypes.c_void_p] * 5 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_prefill_timing_events": ([ctypes.POINTER(PrefillShape), ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
    "dsa_prefill_timed": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "dsa_decode_timed": ([ctypes.POINTER(DecodeShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "dsa_dedup_workspace_size": ([ctypes.POINTER(PrefillShape), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dsa_sparse_attention_dedup": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_prefill_dedup": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_size_t, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
    "dsa_indexer_kl_workspace_size": ([ctypes.POINTER(PrefillShape), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dsa_indexer_kl": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 9 + [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_sparse_attention_fwd_lse": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 7, ctypes.c_int),
    "dsa_sparse_attention_bwd_workspace_size": ([ctypes.POINTER(PrefillShape), ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
    "dsa_sparse_attention_bwd": ([ctypes.POINTER(PrefillShape)] + [ctypes.c_void_p] * 11 + [ctypes.c_size_t, ctypes.c_void_p], ctypes.c_int),
    "dsa_topk": ([ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int64, ctypes.c_void_p, ctypes.c_int32,
                  ctypes.c_void_p, ctypes.c_void_p], ctypes.c_int),
}


def lib_path() -> str:
    return _LIB_PATH


def lib():
    """Load libdsa.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(f"{_LIB_PATH} is missing: build it with `python -m sparse_attention_long_04_amd.build`")
        import torch  # noqa: F401  -- load torch's HIP runtime first so the process has exactly one
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in EXPORTS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(x):
    """Tensor -> device pointer; ints are raw pointers; (pointer, nbytes) tuples are buffers."""
    if x is None:
        return None
    if isinstance(x, tuple):
        return x[0]
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(rc, where):
    if rc != 0:
        raise DSAError(rc, where)


def _nbytes(ws):
    if ws is None:
        return 0
    if isinstance(ws, tuple):
        return ws[1]
    if isinstance(ws, int):
        raise TypeError("pass a raw workspace as (pointer, nbytes)")
    return ws.numel() * ws.element_size()


def prefill_shape(cu_seqlens, total_tokens, max_seqlen, *, topk, idx_heads, idx_dim, idx_dtype,
                  q_heads=32, kv_heads=4, head_dim=128, softmax_scale=None, num_seqs=None) -> PrefillShape:
    """``cu_seqlens`` is a device int32 tensor (or a raw pointer with ``num_seqs`` given)."""
    if num_seqs is None:
        num_seqs = cu_seqlens.numel() - 1
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    return PrefillShape(num_seqs, _ptr(cu_seqlens), total_tokens, max_seqlen, topk, idx_heads, idx_dim,
                        _DTYPES.get(idx_dtype, idx_dtype), q_heads, kv_heads, head_dim, softmax_scale)


def decode_shape(cache_lens, cache_capacity, max_cache_len, *, topk, idx_heads, idx_dim, idx_dtype,
                 q_heads=32, kv_heads=4, head_dim=128, softmax_scale=None, batch=None) -> DecodeShape:
    if batch is None:
        batch = cache_lens.numel()
    if softmax_scale is None:
        softmax_scale = head_dim ** -0.5
    return DecodeShape(batch, cache_capacity, _ptr(cache_lens), max_cache_len, topk, idx_heads, idx_dim,
                       _DTYPES.get(idx_dtype, idx_dtype), q_heads, kv_heads, head_dim, softmax_scale)


def dsa_status_string(status: int) -> str:
    return lib().dsa_status_string(status).decode()


def dsa_prefill_workspace_size(shape: PrefillShape, cu_seqlens_host=None) -> int:
    n = ctypes.c_size_t(0)
    arr = None
    if cu_seqlens_host is not None:
        import numpy as np
        arr = np.ascontiguousarray(cu_seqlens_host, dtype=np.int32)
    _check(lib().dsa_prefill_workspace_size(ctypes.byref(shape), None if arr is None else arr.ctypes.data,
                                            ctypes.byref(n)), "dsa_prefill_workspace_size")
    return n.value


def dsa_index_scores(shape, q_idx, k_idx, w_idx, scores, workspace, stream=None):
    _check(lib().dsa_index_scores(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(scores),
                                  _ptr(workspace), _nbytes(workspace), _stream(stream)), "dsa_index_scores")


def dsa_index_topk(shape, q_idx, k_idx, w_idx, topk_idx, workspace, stream=None):
    _check(lib().dsa_index_topk(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(topk_idx),
                                _ptr(workspace), _nbytes(workspace), _stream(stream)), "dsa_index_topk")


def dsa_sparse_attention(shape, q, k, v, topk_idx, out, stream=None):
    _check(lib().dsa_sparse_attention(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(out),
                                      _stream(stream)), "dsa_sparse_attention")


def dsa_prefill(shape, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, workspace, stream=None):
    _check(lib().dsa_prefill(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(out), _ptr(topk_idx), _ptr(workspace), _nbytes(workspace),
                             _stream(stream)), "dsa_prefill")


def dense_causal_attention(shape, q, k, v, out, workspace, stream=None):
    _check(lib().dense_causal_attention(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                        _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "dense_causal_attention")


def dsa_decode_workspace_size(shape: DecodeShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_decode_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "dsa_decode_workspace_size")
    return n.value


def dsa_kv_append(shape, k_idx_new, k_new, v_new, cache_lens, k_idx_cache, k_cache, v_cache, stream=None):
    _check(lib().dsa_kv_append(ctypes.byref(shape), _ptr(k_idx_new), _ptr(k_new), _ptr(v_new), _ptr(cache_lens),
                               _ptr(k_idx_cache), _ptr(k_cache), _ptr(v_cache), _stream(stream)), "dsa_kv_append")


def dsa_decode(shape, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, workspace, stream=None):
    _check(lib().dsa_decode(ctypes.byref(shape), _ptr(q_idx), _ptr(w_idx), _ptr(q), _ptr(k_idx_cache),
                            _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(topk_idx), _ptr(workspace),
                            _nbytes(workspace), _stream(stream)), "dsa_decode")


def dsa_decode_noalloc(shape, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, stream=None):
    """dsa_decode on the library's static device scratch (no workspace argument)."""
    _check(lib().dsa_decode_noalloc(ctypes.byref(shape), _ptr(q_idx), _ptr(w_idx), _ptr(q), _ptr(k_idx_cache),
                                    _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(topk_idx), _stream(stream)),
           "dsa_decode_noalloc")


def dense_decode_attention(shape, q, k_cache, v_cache, out, workspace, stream=None):
    _check(lib().dense_decode_attention(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out),
                                        _ptr(workspace), _nbytes(workspace), _stream(stream)),
           "dense_decode_attention")


def _events(events):
    arr = (ctypes.c_void_p * len(events))(*[e if isinstance(e, int) else e.cuda_event for e in events])
    return arr


def dsa_prefill_timing_events(shape) -> int:
    """Events dsa_prefill_timed records: 3 + 2 x (indexer chunks)."""
    n = ctypes.c_int32(0)
    _check(lib().dsa_prefill_timing_events(ctypes.byref(shape), ctypes.byref(n)), "dsa_prefill_timing_events")
    return n.value


def _prefill_events(shape, events):
    need = dsa_prefill_timing_events(shape)
    if len(events) < need:
        raise ValueError(f"the prefill records {need} timing events; {len(events)} given")
    return _events(events)


def dsa_prefill_timed(shape, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, workspace, events, stream=None):
    """``events``: dsa_prefill_timing_events(shape) recorded-once torch.cuda.Event(enable_timing=True)
    (or raw hipEvent_t)."""
    ev = _prefill_events(shape, events)
    _check(lib().dsa_prefill_timed(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(out), _ptr(topk_idx), _ptr(workspace), _nbytes(workspace),
                                   _stream(stream), ev), "dsa_prefill_timed")


def dsa_decode_timed(shape, q_idx, w_idx, q, k_idx_cache, k_cache, v_cache, out, topk_idx, workspace, events,
                     stream=None):
    ev = _events(events)
    _check(lib().dsa_decode_timed(ctypes.byref(shape), _ptr(q_idx), _ptr(w_idx), _ptr(q), _ptr(k_idx_cache),
                                  _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(topk_idx), _ptr(workspace),
                                  _nbytes(workspace), _stream(stream), ev), "dsa_decode_timed")


def dsa_topk(scores, rows, n, ld, row_lens, k, out, stream=None):
    """Standalone deterministic top-k: scores fp32 rows (row r at scores + r*ld), out int32 [rows, k]."""
    _check(lib().dsa_topk(_ptr(scores), int(rows), int(n), int(ld), _ptr(row_lens), int(k), _ptr(out),
                          _stream(stream)), "dsa_topk")


def dsa_dedup_workspace_size(shape: PrefillShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_dedup_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "dsa_dedup_workspace_size")
    return n.value


def dsa_sparse_attention_dedup(shape, q, k, v, topk_idx, out, dedup_workspace, stream=None):
    _check(lib().dsa_sparse_attention_dedup(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(out),
                                            _ptr(dedup_workspace), _nbytes(dedup_workspace), _stream(stream)),
           "dsa_sparse_attention_dedup")


def dsa_prefill_dedup(shape, q_idx, k_idx, w_idx, q, k, v, out, topk_idx, workspace, dedup_workspace, events=None,
                      stream=None):
    """``events``: None, or dsa_prefill_timing_events(shape) recorded-once timing events (as
    dsa_prefill_timed)."""
    ev = None if events is None else _prefill_events(shape, events)
    _check(lib().dsa_prefill_dedup(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k),
                                   _ptr(v), _ptr(out), _ptr(topk_idx), _ptr(workspace), _nbytes(workspace),
                                   _ptr(dedup_workspace), _nbytes(dedup_workspace), _stream(stream), ev),
           "dsa_prefill_dedup")


def dsa_indexer_kl_workspace_size(shape: PrefillShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_indexer_kl_workspace_size(ctypes.byref(shape), ctypes.byref(n)), "dsa_indexer_kl_workspace_size")
    return n.value


def dsa_indexer_kl(shape, q_idx, k_idx, w_idx, q, k, kl, dq_idx, dk_idx, dw_idx, workspace, stream=None):
    _check(lib().dsa_indexer_kl(ctypes.byref(shape), _ptr(q_idx), _ptr(k_idx), _ptr(w_idx), _ptr(q), _ptr(k), _ptr(kl),
                                _ptr(dq_idx), _ptr(dk_idx), _ptr(dw_idx), _ptr(workspace), _nbytes(workspace),
                                _stream(stream)), "dsa_indexer_kl")


def dsa_sparse_attention_fwd_lse(shape, q, k, v, topk_idx, out, lse, stream=None):
    _check(lib().dsa_sparse_attention_fwd_lse(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(out),
                                              _ptr(lse), _stream(stream)), "dsa_sparse_attention_fwd_lse")


def dsa_sparse_attention_bwd_workspace_size(shape: PrefillShape) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().dsa_sparse_attention_bwd_workspace_size(ctypes.byref(shape), ctypes.byref(n)),
           "dsa_sparse_attention_bwd_workspace_size")
    return n.value


def dsa_sparse_attention_bwd(shape, q, k, v, topk_idx, out, lse, d_out, dq, dk, dv, workspace, stream=None):
    _check(lib().dsa_sparse_attention_bwd(ctypes.byref(shape), _ptr(q), _ptr(k), _ptr(v), _ptr(topk_idx), _ptr(out),
                                          _ptr(lse), _ptr(d_out), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                                          _nbytes(workspace), _stream(stream)), "dsa_sparse_attention_bwd")
