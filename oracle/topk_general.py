"""CPU oracle of the standalone deterministic top-k over general float32 rows.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py`` may import or call this module; it shares no code with the HIP library.

What it computes: the Keye-VL-2.0 summary page (gsyq.cn), section 八, replaces torch.topk in
the DSA selection by a deterministic top-k, so that the same scores always give the same
positions.  As a standalone op, that selection runs over arbitrary float32 rows (any length,
any values), not only over the indexer's exact scores.  The pages say nothing about special
values; the readings taken here:

* NaN (any sign or payload) and -inf are masked: they are never selected (-inf is the usual
  way to mask a position out of a score row, and a NaN has no place in an order);
* +inf and every finite value are selectable; +0 and -0 are the same score;
* among selectable positions the order is (score descending, index ascending) -- ties go to
  the lower index, as in the DSA path;
* each row keeps its first min(k, #selectable) positions under that order, written in
  ascending position order and padded with -1.
"""
from __future__ import annotations

import numpy as np


def select_topk_general_row(row: np.ndarray, k: int) -> np.ndarray:
    """One row: the definition above, with a stable library sort as the ordering step."""
    x = np.asarray(row, dtype=np.float32).astype(np.float64)
    pos = np.arange(x.size)
    ok = ~np.isnan(x) & (x != -np.inf)
    cand, val = pos[ok], x[ok]
    order = np.lexsort((cand, -val))          # score descending, then index ascending
    keep = np.sort(cand[order[:k]])
    out = np.full(k, -1, dtype=np.int32)
    out[:keep.size] = keep
    return out


def topk_general(scores: np.ndarray, k: int, row_lens=None) -> np.ndarray:
    """Batched rows [R, n]; row r uses its first row_lens[r] elements (clamped to [0, n]) when
    row_lens is given."""
    s = np.asarray(scores, dtype=np.float32)
    R, n = s.shape
    out = np.empty((R, k), dtype=np.int32)
    for r in range(R):
        m = n if row_lens is None else max(0, min(n, int(row_lens[r])))
        out[r] = select_topk_general_row(s[r, :m], k)
    return out
