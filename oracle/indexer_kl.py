"""CPU oracle of the Lightning Indexer's dense warm-up objective (forward and backward).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call this module; it shares no code with the HIP library.

What it computes (Keye-VL-2.0 summary page, gsyq.cn, section 一): training runs in two stages;
in the first, "dense warm-up", the full attention is left as it is and only the indexer (the
"scout") is trained, by making its judgement of which positions matter match the full
attention's distribution -- the gap is measured by a KL divergence, which is minimised.

Readings (the page gives no formula):

* target p_t: the full attention distribution of query token t, summed over the Hq query
  heads and L1-normalised over the key positions s <= t (= the mean of the heads' softmax
  distributions, each softmax(scale * q[t,h] . k[s, g(h)])); it is a constant (no gradient
  flows into the main attention);
* indexer distribution r_t = softmax over s <= t of the indexer scores
  I[t, s] = sum_h w[t,h] * max(0, q_I[t,h] . k_I[s]);
* loss per token KL(p_t || r_t) = sum_s p log(p / r) (terms with p = 0 contribute 0), and the
  objective is the sum over tokens;
* gradients of the summed loss with respect to the indexer inputs: with g = r - p (the
  gradient of KL(p || softmax(I)) with respect to I) and c[t,h,s] = q_I[t,h] . k_I[s],
      dw[t,h]   = sum_s g[t,s] * max(0, c[t,h,s])
      dq_I[t,h] = w[t,h] * sum_s g[t,s] * [c[t,h,s] > 0] * k_I[s]
      dk_I[s]   = sum_{t >= s} sum_h g[t,s] * w[t,h] * [c[t,h,s] > 0] * q_I[t,h]
  (ReLU's derivative is taken as 0 at 0).
"""
from __future__ import annotations

import numpy as np


def _softmax(x: np.ndarray) -> np.ndarray:
    m = x.max(axis=-1, keepdims=True)
    e = np.exp(x - m)
    return e / e.sum(axis=-1, keepdims=True)


def kl_row(q_t, k_ctx, qi_t, ki_ctx, w_t, scale):
    """One query token against its causal context (float64 arrays).

    q_t [Hq, d], k_ctx [n, Hkv, d], qi_t [H, dI], ki_ctx [n, dI], w_t [H].
    Returns (kl, p [n], r [n], g [n], c [H, n])."""
    Hq = q_t.shape[0]
    Hkv = k_ctx.shape[1]
    grp = Hq // Hkv
    z = np.stack([scale * (k_ctx[:, h // grp, :] @ q_t[h]) for h in range(Hq)])   # [Hq, n]
    p = _softmax(z).sum(axis=0)
    p = p / p.sum()
    c = qi_t @ ki_ctx.T                                                             # [H, n]
    scores = (w_t[:, None] * np.maximum(c, 0.0)).sum(axis=0)
    r = _softmax(scores)
    # log r as a log-softmax: r itself underflows to 0 when scores differ by more than ~745
    m = scores.max()
    log_r = scores - m - np.log(np.exp(scores - m).sum())
    pos = p > 0
    kl = float(np.sum(p[pos] * (np.log(p[pos]) - log_r[pos])))
    return kl, p, r, r - p, c


def kl_warmup(cu_seqlens, q, k, q_idx, k_idx, w_idx, scale, rows=None):
    """Forward and backward over packed sequences (float64 inputs, already decoded).

    q [T, Hq, d], k [T, Hkv, d], q_idx [T, H, dI], k_idx [T, dI], w_idx [T, H].
    Returns kl [T], dq_idx [T, H, dI], dk_idx [T, dI], dw [T, H]; with ``rows`` only those rows'
    kl, dq and dw are filled (dk then only gets those rows' contributions)."""
    T = q.shape[0]
    kl = np.zeros(T)
    dq = np.zeros(q_idx.shape)
    dk = np.zeros(k_idx.shape)
    dw = np.zeros(w_idx.shape)
    cu = np.asarray(cu_seqlens)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        s0, s1 = int(cu[b]), int(cu[b + 1])
        for t in range(s0, s1):
            if want is not None and t not in want:
                continue
            ctx = slice(s0, t + 1)
            kl[t], _, _, g, c = kl_row(q[t], k[ctx], q_idx[t], k_idx[ctx], w_idx[t], scale)
            on = (c > 0).astype(np.float64)
            dw[t] = (np.maximum(c, 0.0) * g[None, :]).sum(axis=1)
            gate = on * g[None, :] * w_idx[t][:, None]                                # [H, n]
            dq[t] = gate @ k_idx[ctx]
            dk[ctx] += gate.T @ q_idx[t]
    return kl, dq, dk, dw
