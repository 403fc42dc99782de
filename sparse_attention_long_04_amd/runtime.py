"""Device-side plumbing around the C ABI: upload seeded inputs into torch device tensors,
allocate outputs and workspaces, and call the entry points of :mod:`.dsa`.

PyTorch is used here only for device memory and streams; every step of the hot path runs
in the HIP kernels of libdsa.so.
"""
from __future__ import annotations

import numpy as np
import torch

from . import dsa


def _dev(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


class PrefillBatch:
    """A packed prefill batch resident in HBM, with its workspace."""

    def __init__(self, p, device="cuda", workspace=True):
        self.p = p
        self.device = device
        self.cu = _dev(p.cu_seqlens.astype(np.int32), device)
        self.q_idx = _dev(p.q_idx, device)
        self.k_idx = _dev(p.k_idx, device)
        self.w_idx = _dev(p.w_idx.astype(np.float32), device)
        self.q = _dev(p.q, device)
        self.k = _dev(p.k, device)
        self.v = _dev(p.v, device)
        T = p.total_tokens
        self.shape = dsa.prefill_shape(self.cu, T, p.max_seqlen, topk=p.topk, idx_heads=p.q_idx.shape[1],
                                       idx_dim=p.q_idx.shape[2], idx_dtype=p.idx_dtype,
                                       q_heads=p.q.shape[1], kv_heads=p.k.shape[1], head_dim=p.q.shape[2],
                                       softmax_scale=p.softmax_scale)
        self.out = torch.empty((T, p.q.shape[1], p.q.shape[2]), dtype=torch.int16, device=device)
        self.topk_idx = torch.empty((T, p.topk), dtype=torch.int32, device=device)
        self.ws = None
        if workspace:
            n = dsa.dsa_prefill_workspace_size(self.shape, p.cu_seqlens)
            self.ws = torch.empty(max(n, 256), dtype=torch.uint8, device=device)

    # --- entry points ---------------------------------------------------------------
    def prefill(self, stream=None):
        dsa.dsa_prefill(self.shape, self.q_idx, self.k_idx, self.w_idx, self.q, self.k, self.v, self.out,
                        self.topk_idx, self.ws, stream)

    def timing_events(self):
        """Events a timed prefill of this batch records (3 + 2 x indexer chunks)."""
        return dsa.dsa_prefill_timing_events(self.shape)

    def prefill_timed(self, events, stream=None):
        dsa.dsa_prefill_timed(self.shape, self.q_idx, self.k_idx, self.w_idx, self.q, self.k, self.v, self.out,
                              self.topk_idx, self.ws, events, stream)

    def index_topk(self, stream=None):
        dsa.dsa_index_topk(self.shape, self.q_idx, self.k_idx, self.w_idx, self.topk_idx, self.ws, stream)

    def sparse_attention(self, stream=None):
        dsa.dsa_sparse_attention(self.shape, self.q, self.k, self.v, self.topk_idx, self.out, stream)

    def dense(self, out=None, stream=None):
        out = self.out if out is None else out
        dsa.dense_causal_attention(self.shape, self.q, self.k, self.v, out, self.ws, stream)
        return out

    # --- adjacent-query dedup ----------------------------------------------------------
    def _dedup_ws(self):
        if getattr(self, "dws", None) is None:
            self.dws = torch.empty(max(dsa.dsa_dedup_workspace_size(self.shape), 256), dtype=torch.uint8,
                                   device=self.device)
        return self.dws

    def prefill_dedup(self, events=None, stream=None):
        dsa.dsa_prefill_dedup(self.shape, self.q_idx, self.k_idx, self.w_idx, self.q, self.k, self.v, self.out,
                              self.topk_idx, self.ws, self._dedup_ws(), events, stream)

    def dedup_unions(self):
        """After sparse_attention_dedup: (sched [n, 2] = (sequence, 16-row block), union sizes [n],
        union positions and row masks per block) read back from the dedup workspace, whose layout
        is counts int[64] | sched int2[nb] | ucount int[nb] | ukeys int32[nb][16k] |
        umask uint16[nb][16k], each part 256-byte aligned, nb = ceil(T/16) + #sequences."""
        def up(x):
            return (x + 255) // 256 * 256
        T, B, k = self.p.total_tokens, len(self.p.lengths), self.p.topk
        nb, us = (T + 15) // 16 + B, 16 * k
        o_sched = 256
        o_cnt = up(o_sched + nb * 8)
        o_keys = up(o_cnt + nb * 4)
        o_mask = up(o_keys + nb * us * 4)
        w = self.dws
        n = int(w[0:4].view(torch.int32).item())
        sched = w[o_sched:o_sched + n * 8].view(torch.int32).view(n, 2)
        cnt = w[o_cnt:o_cnt + n * 4].view(torch.int32)
        keys = w[o_keys:o_keys + n * us * 4].view(torch.int32).view(n, us)
        mask = w[o_mask:o_mask + n * us * 2].view(torch.int16).view(n, us)
        return sched, cnt, keys, mask

    def sparse_attention_dedup(self, out=None, stream=None):
        out = self.out if out is None else out
        dsa.dsa_sparse_attention_dedup(self.shape, self.q, self.k, self.v, self.topk_idx, out, self._dedup_ws(), stream)
        return out

    def index_scores(self, stream=None):
        T = self.p.total_tokens
        scores = torch.empty((T, max(1, self.p.max_seqlen)), dtype=torch.float32, device=self.device)
        dsa.dsa_index_scores(self.shape, self.q_idx, self.k_idx, self.w_idx, scores, self.ws, stream)
        return scores


def bf16_to_float(t: torch.Tensor) -> np.ndarray:
    """bf16 bit patterns (int16 tensor) -> float64 numpy (host)."""
    return t.cpu().view(torch.bfloat16).to(torch.float64).numpy()


class DecodeState:
    """Decode caches resident in HBM plus one step's new-token tensors."""

    def __init__(self, d, device="cuda"):
        self.d = d
        self.device = device
        B = d.batch
        self.k_idx_cache = _dev(d.k_idx_cache, device)
        self.k_cache = _dev(d.k_cache, device)
        self.v_cache = _dev(d.v_cache, device)
        self.lens = torch.full((B,), d.ctx_len, dtype=torch.int32, device=device)
        self.len_host = np.full(B, d.ctx_len, dtype=np.int64)
        self.out = torch.empty((B, d.q_heads, d.head_dim), dtype=torch.int16, device=device)
        self.topk_idx = torch.empty((B, d.topk), dtype=torch.int32, device=device)
        self.shape = self._shape()
        self.ws = torch.empty(dsa.dsa_decode_workspace_size(self.shape), dtype=torch.uint8, device=device)

    def _shape(self):
        d = self.d
        return dsa.decode_shape(self.lens, d.capacity, d.capacity, topk=d.topk, idx_heads=d.idx_heads,
                                idx_dim=d.idx_dim, idx_dtype=d.idx_dtype, q_heads=d.q_heads,
                                kv_heads=d.kv_heads, head_dim=d.head_dim, softmax_scale=d.softmax_scale)

    def load_step(self, i):
        s = self.d.step(i)
        self.step_host = s
        self.step_dev = {k: _dev(v, self.device) for k, v in s.items()}
        return s

    def append(self, stream=None):
        """Append the loaded step's token at row cache_lens[b]; the kernel also counts it."""
        if int(self.len_host.max()) >= self.d.capacity:
            raise ValueError("decode cache is full")
        sd = self.step_dev
        dsa.dsa_kv_append(self.shape, sd["k_idx_new"], sd["k_new"], sd["v_new"], self.lens, self.k_idx_cache,
                          self.k_cache, self.v_cache, stream)
        self.len_host += 1

    def decode(self, stream=None):
        sd = self.step_dev
        dsa.dsa_decode(self.shape, sd["q_idx"], sd["w_idx"], sd["q"], self.k_idx_cache, self.k_cache, self.v_cache,
                       self.out, self.topk_idx, self.ws, stream)

    def decode_timed(self, events, stream=None):
        sd = self.step_dev
        dsa.dsa_decode_timed(self.shape, sd["q_idx"], sd["w_idx"], sd["q"], self.k_idx_cache, self.k_cache,
                             self.v_cache, self.out, self.topk_idx, self.ws, events, stream)

    def dense(self, out=None, stream=None):
        out = self.out if out is None else out
        dsa.dense_decode_attention(self.shape, self.step_dev["q"], self.k_cache, self.v_cache, out, self.ws, stream)
        return out


def timing_events(n):
    """n timing events, each recorded once so that its handle exists and it counts as recorded."""
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
    for e in evs:
        e.record()
    return evs
