"""CPU oracle of the DSA hot path (Lightning Indexer -> top-k -> sparse GQA attention).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call this module.  The product path never routes through
it, and it shares no code with the HIP library: it decodes the storage formats itself and
computes everything in float64 with plain NumPy (a matrix product and a partition are the
only library primitives used as steps).

What it computes, and where the pages state it (Keye-VL-2.0 summary page, gsyq.cn):

* section 一: a lightweight "scout" (the Lightning Indexer) scans every position and scores
  which ones deserve attention; it is MQA-shared -- one set of "eyes", i.e. one indexer key
  per token shared by every indexer head;
* section 一 and the second Q&A: each current token then keeps the 2048 most relevant
  positions of its context, turning O(L^2) attention into O(Lk);
* section 一: full attention is then computed only among the selected positions, on a GQA
  base model (the GQA adaptation of DSA);
* section 八: the selection must be deterministic (torch.topk replaced by a deterministic
  top-k so that training and inference pick the same sets).

The pages print no formula.  Readings taken where they are silent (each is listed with its
reason in the design notes):

* indexer score  I[t, s] = sum_h w[t, h] * max(0, q_I[t, h, :] . k_I[s, :])  for s <= t;
* ties in the selection go to the lower key index; the selected positions are returned in
  ascending order and padded with -1 when a row has fewer than k valid keys;
* one index set per query token, shared by all query heads; query head h reads KV head
  h // (Hq / Hkv); softmax scale 1/sqrt(d); no bias, sink or positional term;
* decode: the new token is already in the cache (the cache length counts it);
* packed sequences: keys never cross a sequence boundary; indices are positions relative
  to the start of the query's own sequence.
"""
from __future__ import annotations

import numpy as np

# ----------------------------------------------------------------------------------------
# storage formats
# ----------------------------------------------------------------------------------------


def decode_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 is the upper 16 bits of an IEEE-754 binary32 value."""
    b = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def decode_e4m3fn(codes: np.ndarray) -> np.ndarray:
    """OCP 8-bit float E4M3 ("fn": finite, no infinities).  1 sign, 4 exponent (bias 7) and
    3 mantissa bits; exponent 0 is subnormal (2^-6 * m/8); S.1111.111 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    sign = np.where(c >> 7, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal) * sign
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


def decode(arr: np.ndarray, fmt: str) -> np.ndarray:
    if fmt == "bf16":
        return decode_bf16(arr)
    if fmt == "fp8_e4m3":
        return decode_e4m3fn(arr)
    if fmt == "f32":
        return np.asarray(arr, dtype=np.float32).astype(np.float64)
    raise ValueError(fmt)


# ----------------------------------------------------------------------------------------
# the three steps, one query row at a time
# ----------------------------------------------------------------------------------------


def index_score_row(q_idx_t: np.ndarray, k_idx_ctx: np.ndarray, w_t: np.ndarray) -> np.ndarray:
    """Lightning Indexer scores of one query token against its causal context.

    q_idx_t [H_I, d_I], k_idx_ctx [n, d_I] (keys 0..n-1 of the token's own sequence, the
    token itself included), w_t [H_I].  Returns I[s] = sum_h w_h * relu(q_h . k_s), float64.
    Summary page section 一: one MQA-shared key per position, scored by every indexer head.
    """
    dots = k_idx_ctx @ q_idx_t.T            # [n, H_I]: q_h . k_s
    return np.maximum(dots, 0.0) @ w_t      # weighted sum over heads of the ReLU


def select_topk_row(scores: np.ndarray, k: int) -> np.ndarray:
    """The first min(k, n) keys in the order (score descending, index ascending), returned
    in ascending index order and padded with -1 to length k.

    Summary page section 一: keep the k most relevant positions of the context; section 八:
    the choice is deterministic, which the lower-index-wins tie rule makes unique.
    """
    n = scores.shape[0]
    m = min(k, n)
    out = np.full(k, -1, dtype=np.int64)
    if m == n:
        out[:n] = np.arange(n)
        return out
    # value of the m-th largest score (the selection threshold)
    thr = np.partition(scores, n - m)[n - m]
    above = np.flatnonzero(scores > thr)
    ties = np.flatnonzero(scores == thr)          # ascending: lower indices first
    chosen = np.concatenate([above, ties[: m - above.size]])
    out[:m] = np.sort(chosen)
    return out


def attention_row(q_t: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray, scale: float) -> np.ndarray:
    """Scaled dot-product attention of one query token over the given key/value rows.

    q_t [Hq, d]; k_rows, v_rows [m, Hkv, d].  Query head h uses KV head h // (Hq // Hkv)
    (the GQA base model of the summary page, section 一).  Softmax in float64.
    """
    hq, d = q_t.shape
    hkv = k_rows.shape[1]
    g = hq // hkv
    out = np.empty((hq, d), dtype=np.float64)
    for j in range(hkv):
        z = scale * (q_t[j * g:(j + 1) * g] @ k_rows[:, j, :].T)   # [g, m]
        z -= z.max(axis=1, keepdims=True)
        p = np.exp(z)
        out[j * g:(j + 1) * g] = (p @ v_rows[:, j, :]) / p.sum(axis=1, keepdims=True)
    return out


# ----------------------------------------------------------------------------------------
# packed prefill, decode and dense attention over chosen rows
# ----------------------------------------------------------------------------------------


class Prefill:
    """Decoded views of one packed prefill batch (decoding is done lazily per row)."""

    def __init__(self, cu_seqlens, q_idx, k_idx, w_idx, q, k, v, idx_fmt, topk, scale):
        self.cu = np.asarray(cu_seqlens, dtype=np.int64)
        self.q_idx, self.k_idx, self.w = q_idx, k_idx, np.asarray(w_idx)
        self.q, self.k, self.v = q, k, v
        self.fmt, self.topk, self.scale = idx_fmt, int(topk), float(scale)
        self._seq_cache = {}

    def _seq(self, b):
        """Decoded keys/values of sequence b (indexer keys, attention keys, values)."""
        if b not in self._seq_cache:
            a, e = self.cu[b], self.cu[b + 1]
            self._seq_cache = {b: (decode(self.k_idx[a:e], self.fmt), decode_bf16(self.k[a:e]),
                                   decode_bf16(self.v[a:e]))}
        return self._seq_cache[b]

    def locate(self, t):
        b = int(np.searchsorted(self.cu, t, side="right") - 1)
        return b, int(t - self.cu[b])

    def scores(self, t):
        b, i = self.locate(t)
        kI, _, _ = self._seq(b)
        return index_score_row(decode(self.q_idx[t], self.fmt), kI[: i + 1],
                               self.w[t].astype(np.float64))

    def row(self, t):
        """(selected indices [k], output [Hq, d]) for global token row t."""
        b, i = self.locate(t)
        _, K, V = self._seq(b)
        sel = select_topk_row(self.scores(t), self.topk)
        s = sel[sel >= 0]
        out = attention_row(decode_bf16(self.q[t]), K[s], V[s], self.scale)
        return sel, out

    def dense_row(self, t):
        b, i = self.locate(t)
        _, K, V = self._seq(b)
        return attention_row(decode_bf16(self.q[t]), K[: i + 1], V[: i + 1], self.scale)

    def rows(self, ts):
        sels, outs = [], []
        for t in ts:
            s, o = self.row(int(t))
            sels.append(s)
            outs.append(o)
        return np.stack(sels), np.stack(outs)

    def dense_rows(self, ts):
        return np.stack([self.dense_row(int(t)) for t in ts])


def _decoded_keys(k_idx_cache, b, n, idx_fmt, memo):
    """Indexer keys 0..n-1 of cache b as float64.  With a ``memo`` dict the decoded rows of
    each sequence are kept between calls and only rows appended since are decoded (the values
    are the same either way; this only saves time over many steps)."""
    if memo is None:
        return decode(k_idx_cache[b, :n], idx_fmt)
    have = memo.get(b)
    if have is None or have.shape[0] < n:
        start = 0 if have is None else have.shape[0]
        new = decode(k_idx_cache[b, start:n], idx_fmt)
        have = new if have is None else np.concatenate([have, new])
        memo[b] = have
    return have[:n]


def decode_step(k_idx_cache, k_cache, v_cache, cache_lens, q_idx, w_idx, q, idx_fmt, topk, scale,
                seqs=None, memo=None):
    """One decode step: for each sequence b the newest token (row cache_lens[b]-1, already in
    the cache) scores all cached keys 0..n-1, keeps the top-k and attends over them.
    Returns (indices [B, k], output [B, Hq, d]) for the sequences in ``seqs``.
    Summary page section 一 (decode cost) and section 八 (DSA decode path).
    ``memo``: optional dict that keeps decoded indexer keys across steps (cached rows must not
    change between calls that share it; appending rows is fine)."""
    seqs = range(len(cache_lens)) if seqs is None else seqs
    sels, outs = [], []
    for b in seqs:
        n = int(cache_lens[b])
        sc = index_score_row(decode(q_idx[b], idx_fmt), _decoded_keys(k_idx_cache, b, n, idx_fmt, memo),
                             np.asarray(w_idx[b], dtype=np.float64))
        sel = select_topk_row(sc, topk)
        s = sel[sel >= 0]
        outs.append(attention_row(decode_bf16(q[b]), decode_bf16(k_cache[b, s]),
                                  decode_bf16(v_cache[b, s]), scale))
        sels.append(sel)
    return np.stack(sels), np.stack(outs)


def dense_decode(k_cache, v_cache, cache_lens, q, scale, seqs=None):
    """Full attention of the newest token over its whole cache (the decode cost reference)."""
    seqs = range(len(cache_lens)) if seqs is None else seqs
    out = []
    for b in seqs:
        n = int(cache_lens[b])
        out.append(attention_row(decode_bf16(q[b]), decode_bf16(k_cache[b, :n]),
                                 decode_bf16(v_cache[b, :n]), scale))
    return np.stack(out)


def index_score_matrix(cu_seqlens, q_idx, k_idx, w_idx, idx_fmt):
    """All indexer scores of a (small) packed batch as a [T, max_len] float64 matrix with
    -inf outside each row's causal context."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    T = int(cu[-1])
    lens = np.diff(cu)
    out = np.full((T, int(lens.max()) if lens.size else 0), -np.inf)
    for b in range(len(lens)):
        a = cu[b]
        kI = decode(k_idx[a:cu[b + 1]], idx_fmt)
        for i in range(int(lens[b])):
            out[a + i, : i + 1] = index_score_row(decode(q_idx[a + i], idx_fmt), kI[: i + 1],
                                                  np.asarray(w_idx[a + i], dtype=np.float64))
    return out
