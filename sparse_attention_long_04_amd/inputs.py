"""Seeded synthetic inputs for the DSA hot path (indexer -> top-k -> sparse GQA attention).

This module only *constructs inputs*: random draws, the video-like key layout and the
encoding of values into the storage formats (bf16 bit patterns, OCP fp8-e4m3fn codes).
It holds none of the method's arithmetic, so both the GPU path and the CPU oracle can be
fed from it.  Every array is produced from a ``numpy.random.SeedSequence`` tree in
fixed-size chunks, so the values do not depend on the number of threads used.

Input recipe (all integer-valued indexer inputs, so indexer scores are exact):

* indexer queries ``q_idx[T, H_I, d_I]`` and keys ``k_idx[T, d_I]``: integers drawn
  uniformly from ``{-R..R}`` and stored as bf16 or fp8-e4m3fn bit patterns;
* indexer head weights ``w_idx[T, H_I]``: ``2**-j`` with ``j`` uniform in ``{0..3}`` (fp32);
* attention ``q[T, Hq, d]``, ``k[T, Hkv, d]``, ``v[T, Hkv, d]``: N(0, 1) rounded to bf16;
* "video" keys: each sequence is a run of frames of 16 timestamp-text tokens followed by
  1008 vision tokens.  Vision keys are a per-frame mean vector (N(0, I)) plus 0.3 N(0, I)
  noise, text keys are N(0, I).  Indexer keys are ``clamp(rint(2 x), -4, 4)``; attention
  keys use their own per-frame, per-KV-head means.  This mirrors the long-video token
  layout of the Keye-VL-2.0 summary page (gsyq.cn), section 三: every frame is an image
  preceded by a natural-language timestamp.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

FRAME_TEXT = 16
FRAME_VISION = 1008
FRAME_LEN = FRAME_TEXT + FRAME_VISION

_CHUNK_ROWS_TARGET = 1 << 21  # elements per generator chunk (fixed: keeps results thread-independent)


def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


# ----------------------------------------------------------------------------------------
# storage-format encoders (input construction only)
# ----------------------------------------------------------------------------------------

def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round-to-nearest-even) and return the uint16 patterns."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _int_code_table(fmt: str, rng_max: int) -> np.ndarray:
    """Bit patterns of the integers -rng_max..rng_max in ``fmt`` (index i <-> value i-rng_max)."""
    import torch

    vals = torch.arange(-rng_max, rng_max + 1, dtype=torch.float32)
    if fmt == "bf16":
        return vals.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if fmt == "fp8_e4m3":
        return vals.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(fmt)


def _fmt_np_dtype(fmt: str):
    return np.uint16 if fmt == "bf16" else np.uint8


# ----------------------------------------------------------------------------------------
# chunked parallel fills
# ----------------------------------------------------------------------------------------

def _chunks(rows: int, row_elems: int):
    per = max(1, _CHUNK_ROWS_TARGET // max(1, row_elems))
    return [(r, min(rows, r + per)) for r in range(0, rows, per)]


def _par(fn, jobs):
    if len(jobs) <= 1:
        for j in jobs:
            fn(*j)
        return
    with ThreadPoolExecutor(_threads()) as ex:
        list(ex.map(lambda j: fn(*j), jobs))


def _fill_int_codes(ss: np.random.SeedSequence, shape, fmt: str, rng_max: int) -> np.ndarray:
    rows, row_elems = shape[0], int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, row_elems), dtype=_fmt_np_dtype(fmt))
    table = _int_code_table(fmt, rng_max)
    parts = _chunks(rows, row_elems)
    kids = ss.spawn(len(parts))

    def work(i, r0, r1):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        ints = g.integers(0, 2 * rng_max + 1, size=(r1 - r0, row_elems), dtype=np.uint8)
        np.take(table, ints, out=out[r0:r1])

    _par(work, [(i, a, b) for i, (a, b) in enumerate(parts)])
    return out.reshape(shape)


def _fill_normal_bf16(ss: np.random.SeedSequence, shape) -> np.ndarray:
    rows, row_elems = shape[0], int(np.prod(shape[1:])) if len(shape) > 1 else 1
    out = np.empty((rows, row_elems), dtype=np.uint16)
    parts = _chunks(rows, row_elems)
    kids = ss.spawn(len(parts))

    def work(i, r0, r1):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        x = g.standard_normal(size=(r1 - r0, row_elems), dtype=np.float32)
        out[r0:r1] = bf16_bits(x)

    _par(work, [(i, a, b) for i, (a, b) in enumerate(parts)])
    return out.reshape(shape)


def _pow2_weights(ss: np.random.SeedSequence, shape) -> np.ndarray:
    g = np.random.Generator(np.random.PCG64(ss))
    j = g.integers(0, 4, size=shape)
    return np.ldexp(np.float32(1.0), -j).astype(np.float32)


def _video_keys(ss: np.random.SeedSequence, lengths, idx_dim, kv_heads, head_dim, idx_fmt):
    """Frame-clustered indexer keys (integer codes) and attention keys (bf16 bits)."""
    T = int(sum(lengths))
    k_idx = np.empty((T, idx_dim), dtype=_fmt_np_dtype(idx_fmt))
    k_att = np.empty((T, kv_heads, head_dim), dtype=np.uint16)
    table = _int_code_table(idx_fmt, 4)
    jobs = []
    kids = ss.spawn(len(lengths))
    off = 0
    for s, L in enumerate(lengths):
        n_frames = (L + FRAME_LEN - 1) // FRAME_LEN
        fk = kids[s].spawn(n_frames + 1)
        # per-sequence frame means: [frame, idx_dim] and [frame, kv_heads, head_dim]
        gm = np.random.Generator(np.random.PCG64(fk[n_frames]))
        mean_idx = gm.standard_normal(size=(n_frames, idx_dim), dtype=np.float32)
        mean_att = gm.standard_normal(size=(n_frames, kv_heads, head_dim), dtype=np.float32)
        for f in range(n_frames):
            p0 = f * FRAME_LEN
            p1 = min(L, p0 + FRAME_LEN)
            jobs.append((fk[f], off + p0, off + p1, p1 - p0, mean_idx[f], mean_att[f]))
        off += L

    def work(seed, a, b, n, m_idx, m_att):
        g = np.random.Generator(np.random.PCG64(seed))
        xi = g.standard_normal(size=(n, idx_dim), dtype=np.float32)
        xa = g.standard_normal(size=(n, kv_heads, head_dim), dtype=np.float32)
        nt = min(n, FRAME_TEXT)
        xi[nt:] = m_idx[None, :] + np.float32(0.3) * xi[nt:]
        xa[nt:] = m_att[None, :, :] + np.float32(0.3) * xa[nt:]
        codes = np.clip(np.rint(np.float32(2.0) * xi), -4, 4).astype(np.int64) + 4
        k_idx[a:b] = table[codes]
        k_att[a:b] = bf16_bits(xa)

    _par(lambda *j: work(*j), jobs)
    return k_idx, k_att


# ----------------------------------------------------------------------------------------
# public containers
# ----------------------------------------------------------------------------------------

@dataclass
class PrefillInputs:
    """One packed prefill batch.  All arrays are host numpy arrays of storage bit patterns."""

    cu_seqlens: np.ndarray   # int32 [B+1]
    q_idx: np.ndarray        # uint16 (bf16) or uint8 (fp8-e4m3fn) [T, H_I, d_I]
    k_idx: np.ndarray        # same dtype [T, d_I]
    w_idx: np.ndarray        # float32 [T, H_I]
    q: np.ndarray            # uint16 bf16 [T, Hq, d]
    k: np.ndarray            # uint16 bf16 [T, Hkv, d]
    v: np.ndarray            # uint16 bf16 [T, Hkv, d]
    idx_dtype: str           # "bf16" | "fp8_e4m3"
    topk: int
    softmax_scale: float

    @property
    def lengths(self):
        return np.diff(self.cu_seqlens).astype(np.int64)

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def max_seqlen(self) -> int:
        return int(self.lengths.max()) if len(self.lengths) else 0


def _drifting_query_codes(ss: np.random.SeedSequence, lengths, idx_heads, idx_dim, idx_fmt, rho,
                          rank=16) -> np.ndarray:
    """Indexer queries that drift slowly along each sequence: a rank-``rank`` latent AR(1)
    process z_t = rho z_{t-1} + sqrt(1 - rho^2) e_t (z_0 = e_0, e ~ N(0, I)) mapped through a
    fixed Gaussian matrix M [rank, H_I d_I] / sqrt(rank), so every coordinate is N(0, 1) with
    lag-1 correlation rho; codes = clamp(rint(2x), -4, 4), as for the keys."""
    from scipy.signal import lfilter
    T = int(sum(lengths))
    D = idx_heads * idx_dim
    kids = ss.spawn(len(lengths) + 1)
    gm = np.random.Generator(np.random.PCG64(kids[-1]))
    M = gm.standard_normal(size=(rank, D), dtype=np.float32) / np.float32(math.sqrt(rank))
    z = np.empty((T, rank), dtype=np.float32)
    off = 0
    for s, L in enumerate(lengths):
        if L:
            g = np.random.Generator(np.random.PCG64(kids[s]))
            e = g.standard_normal(size=(L, rank))
            zz = np.empty_like(e)
            zz[0] = e[0]
            if L > 1:
                zz[1:] = lfilter([math.sqrt(1.0 - rho * rho)], [1.0, -rho], e[1:], axis=0,
                                 zi=(rho * e[0])[None, :])[0]
            z[off:off + L] = zz
        off += L
    table = _int_code_table(idx_fmt, 4)
    out = np.empty((T, D), dtype=_fmt_np_dtype(idx_fmt))

    def work(a, b):
        x = z[a:b] @ M
        out[a:b] = table[np.clip(np.rint(np.float32(2.0) * x), -4, 4).astype(np.int64) + 4]

    step = 4096
    _par(work, [(a, min(T, a + step)) for a in range(0, T, step)])
    return out.reshape(T, idx_heads, idx_dim)


def make_prefill(lengths, *, idx_heads, idx_dim, idx_dtype, idx_range, topk, seed,
                 video=False, q_heads=32, kv_heads=4, head_dim=128,
                 softmax_scale=None, query_corr=None) -> PrefillInputs:
    """Draw a packed prefill batch.  Draw order: q_idx, k_idx, w, q, k, v.

    ``query_corr`` (rho in (0, 1)): indexer queries drift along each sequence
    (_drifting_query_codes) and the head weights are one 2^-j per head and sequence, so
    adjacent tokens' selections overlap -- the correlated-query workload."""
    lengths = [int(x) for x in lengths]
    T = sum(lengths)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    root = np.random.SeedSequence(seed)
    s_qi, s_ki, s_w, s_q, s_k, s_v = root.spawn(6)
    if query_corr is None:
        q_idx = _fill_int_codes(s_qi, (T, idx_heads, idx_dim), idx_dtype, idx_range)
    else:
        q_idx = _drifting_query_codes(s_qi, lengths, idx_heads, idx_dim, idx_dtype, float(query_corr))
    if video:
        k_idx, k = _video_keys(s_ki, lengths, idx_dim, kv_heads, head_dim, idx_dtype)
    else:
        k_idx = _fill_int_codes(s_ki, (T, idx_dim), idx_dtype, idx_range)
        k = None
    if query_corr is None:
        w = _pow2_weights(s_w, (T, idx_heads))
    else:
        per_seq = _pow2_weights(s_w, (len(lengths), idx_heads))
        w = np.repeat(per_seq, lengths, axis=0).astype(np.float32)
    q = _fill_normal_bf16(s_q, (T, q_heads, head_dim))
    if k is None:
        k = _fill_normal_bf16(s_k, (T, kv_heads, head_dim))
    v = _fill_normal_bf16(s_v, (T, kv_heads, head_dim))
    if softmax_scale is None:
        softmax_scale = 1.0 / math.sqrt(head_dim)
    return PrefillInputs(cu, q_idx, k_idx, w, q, k, v, idx_dtype, int(topk), float(softmax_scale))


def varlen_lengths(seed: int, n_seqs=6, total=262144, lo=8192, hi=98304):
    """``n_seqs-1`` lengths log-uniform in [lo, hi]; the last is ``total - sum`` and the draw
    is rejected unless that one also lies in [lo, hi]."""
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0]))
    while True:
        xs = np.rint(np.exp(g.uniform(math.log(lo), math.log(hi), size=n_seqs - 1))).astype(np.int64)
        last = total - int(xs.sum())
        if lo <= last <= hi:
            return [int(x) for x in xs] + [last]


@dataclass
class DecodeInputs:
    """Decode caches for ``batch`` sequences plus the per-step new-token tensors."""

    batch: int
    capacity: int
    ctx_len: int
    idx_heads: int
    idx_dim: int
    idx_dtype: str
    topk: int
    softmax_scale: float
    k_idx_cache: np.ndarray   # [B, cap, d_I] codes
    k_cache: np.ndarray       # uint16 [B, cap, Hkv, d]
    v_cache: np.ndarray       # uint16 [B, cap, Hkv, d]
    q_heads: int = 32
    kv_heads: int = 4
    head_dim: int = 128
    idx_range: int = 4
    seed: int = 0
    _step_seeds: list = field(default_factory=list, repr=False)

    def step(self, i: int):
        """New-token tensors of decode step ``i``: q_idx [B,H_I,d_I], w [B,H_I], q [B,Hq,d],
        k_idx_new [B,d_I], k_new [B,Hkv,d], v_new [B,Hkv,d].  Appended tokens are text-like
        (i.i.d.); draw order q_idx, w, q, k_idx_new, k_new, v_new."""
        ss = self._step_seeds[i]
        a, b, c, d, e, f = ss.spawn(6)
        B = self.batch
        q_idx = _fill_int_codes(a, (B, self.idx_heads, self.idx_dim), self.idx_dtype, self.idx_range)
        w = _pow2_weights(b, (B, self.idx_heads))
        q = _fill_normal_bf16(c, (B, self.q_heads, self.head_dim))
        k_idx_new = _fill_int_codes(d, (B, self.idx_dim), self.idx_dtype, self.idx_range)
        k_new = _fill_normal_bf16(e, (B, self.kv_heads, self.head_dim))
        v_new = _fill_normal_bf16(f, (B, self.kv_heads, self.head_dim))
        return dict(q_idx=q_idx, w_idx=w, q=q, k_idx_new=k_idx_new, k_new=k_new, v_new=v_new)


def make_decode(batch, ctx_len, capacity, steps, *, idx_heads, idx_dim, idx_dtype, topk,
                seed, video=True, q_heads=32, kv_heads=4, head_dim=128, idx_range=4) -> DecodeInputs:
    """Caches hold ``ctx_len`` valid tokens per sequence (video-like keys when ``video``)."""
    root = np.random.SeedSequence(seed)
    s_ctx, s_v, s_steps = root.spawn(3)
    kc = np.zeros((batch, capacity, idx_dim), dtype=_fmt_np_dtype(idx_dtype))
    kk = np.zeros((batch, capacity, kv_heads, head_dim), dtype=np.uint16)
    vv = np.zeros((batch, capacity, kv_heads, head_dim), dtype=np.uint16)
    if video:
        k_idx, k_att = _video_keys(s_ctx, [ctx_len] * batch, idx_dim, kv_heads, head_dim, idx_dtype)
    else:
        a, b = s_ctx.spawn(2)
        k_idx = _fill_int_codes(a, (batch * ctx_len, idx_dim), idx_dtype, idx_range)
        k_att = _fill_normal_bf16(b, (batch * ctx_len, kv_heads, head_dim))
    kc[:, :ctx_len] = k_idx.reshape(batch, ctx_len, idx_dim)
    kk[:, :ctx_len] = k_att.reshape(batch, ctx_len, kv_heads, head_dim)
    vv[:, :ctx_len] = _fill_normal_bf16(s_v, (batch * ctx_len, kv_heads, head_dim)).reshape(
        batch, ctx_len, kv_heads, head_dim)
    return DecodeInputs(batch, capacity, ctx_len, idx_heads, idx_dim, idx_dtype, int(topk),
                        1.0 / math.sqrt(head_dim), kc, kk, vv, q_heads, kv_heads, head_dim,
                        idx_range, seed, list(s_steps.spawn(steps)))


def make_topk_scores(rows: int, n: int, *, seed: int, kind: str = "normal", masked: float = 0.0,
                     nans: float = 0.0, infs: float = 0.0, zeros: float = 0.0) -> np.ndarray:
    """float32 score rows [rows, n] for the standalone top-k.

    kind: "normal" (N(0,1)), "ties" (integers in {-3..3} / 2: few distinct values),
    "narrow" (1 + U[0, 0.25): one exponent, distinct low bits), "const" (all 1.5).
    Then, independently per element: a fraction ``masked`` becomes -inf, ``nans`` NaN (random
    sign and payload), ``infs`` +inf and ``zeros`` a signed zero."""
    out = np.empty((rows, n), dtype=np.float32)
    parts = _chunks(rows, max(n, 1))
    kids = np.random.SeedSequence(seed).spawn(len(parts))

    def work(i, r0, r1):
        g = np.random.Generator(np.random.PCG64(kids[i]))
        shape = (r1 - r0, n)
        if kind == "normal":
            x = g.standard_normal(size=shape, dtype=np.float32)
        elif kind == "ties":
            x = g.integers(-3, 4, size=shape).astype(np.float32) / np.float32(2)
        elif kind == "narrow":
            x = np.float32(1) + g.random(size=shape, dtype=np.float32) * np.float32(0.25)
        elif kind == "const":
            x = np.full(shape, 1.5, dtype=np.float32)
        else:
            raise ValueError(kind)
        if masked:
            x[g.random(size=shape) < masked] = -np.inf
        if nans:
            m = g.random(size=shape) < nans
            bits = (g.integers(0, 1 << 22, size=int(m.sum()), dtype=np.uint32) | np.uint32(0x7FC00000)
                    | (g.integers(0, 2, size=int(m.sum()), dtype=np.uint32) << np.uint32(31)))
            x[m] = bits.view(np.float32)
        if infs:
            x[g.random(size=shape) < infs] = np.inf
        if zeros:
            m = g.random(size=shape) < zeros
            x[m] = np.where(g.random(size=int(m.sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
        out[r0:r1] = x

    if n > 0:
        _par(work, [(i, a, b) for i, (a, b) in enumerate(parts)])
    return out


def make_grad_bf16(shape, seed: int) -> np.ndarray:
    """An upstream gradient (e.g. dO [T, Hq, d]): N(0,1) rounded to bf16 (bit patterns)."""
    return _fill_normal_bf16(np.random.SeedSequence(seed), tuple(shape))
