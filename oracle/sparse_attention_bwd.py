"""CPU oracle of the sparse GQA attention backward (gradients of the DSA attention stage).

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call this module; it shares no code with the HIP library.

What it computes: the Keye-VL-2.0 summary page (gsyq.cn, section 一) describes a second
training stage, "sparse adaptation", in which every parameter is unfrozen and the model is
trained in the sparse mode with the ordinary next-token objective; that needs the gradients of
the sparse attention itself.  With the forward (float64)

    z[t,h,s] = scale * q[t,h] . k[s, g(h)]          for s in S_t (the row's selected keys)
    P[t,h,s] = softmax over s in S_t of z[t,h,s]
    O[t,h]   = sum_{s in S_t} P[t,h,s] v[s, g(h)]

and an upstream gradient dO, the gradients of sum <dO, O> are the standard softmax-attention
backward restricted to the selected pairs:

    dP[t,h,s] = dO[t,h] . v[s, g(h)],   D[t,h] = sum_s P dP = dO[t,h] . O[t,h]
    dS[t,h,s] = P[t,h,s] (dP[t,h,s] - D[t,h])
    dq[t,h]    = scale * sum_{s in S_t} dS[t,h,s] k[s, g(h)]
    dk[s,g]    = scale * sum over (t, h in group g) with s in S_t of dS[t,h,s] q[t,h]
    dv[s,g]    = sum over (t, h in group g) with s in S_t of P[t,h,s] dO[t,h]

Index sets follow the selection's conventions: ascending positions relative to the sequence
start, padded with -1.  The selection itself is not differentiated (it is discrete).
"""
from __future__ import annotations

import numpy as np


def sparse_attention_bwd(cu_seqlens, q, k, v, idx, d_out, scale, rows=None):
    """q [T, Hq, d], k/v [T, Hkv, d], idx int [T, K], d_out [T, Hq, d] (float64).

    Returns out [T, Hq, d], dq [T, Hq, d], dk [T, Hkv, d], dv [T, Hkv, d]; with ``rows`` only
    those query rows are taken (their dq, and their contributions to dk and dv)."""
    T, Hq, d = q.shape
    Hkv = k.shape[1]
    grp = Hq // Hkv
    out = np.zeros_like(q)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    cu = np.asarray(cu_seqlens)
    want = None if rows is None else set(int(r) for r in rows)
    for b in range(len(cu) - 1):
        s0 = int(cu[b])
        for t in range(s0, int(cu[b + 1])):
            if want is not None and t not in want:
                continue
            sel = idx[t][idx[t] >= 0].astype(np.int64) + s0
            for h in range(Hq):
                g = h // grp
                z = scale * (k[sel, g, :] @ q[t, h])
                p = np.exp(z - z.max())
                p /= p.sum()
                o = p @ v[sel, g, :]
                out[t, h] = o
                dp = v[sel, g, :] @ d_out[t, h]
                ds = p * (dp - d_out[t, h] @ o)
                dq[t, h] = scale * (ds @ k[sel, g, :])
                dk[sel, g, :] += scale * ds[:, None] * q[t, h][None, :]
                dv[sel, g, :] += p[:, None] * d_out[t, h][None, :]
    return out, dq, dk, dv
