"""Pins of the standalone top-k oracle (oracle/topk_general.py) against things other than itself:
a hand-worked fixture, the pairwise definition checked by brute force on tiny rows, a library
top-k on rows of distinct finite values, and special cases.  Each planted-mistake variant (a
plausible bug written into a copy of the oracle's rule) must fail at least one pin."""
import math
import os

import numpy as np
import pytest
import torch

from oracle.topk_general import select_topk_general_row, topk_general

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "topk_general.txt")


def _f32(tok):
    if tok == "-nan":  # a negative NaN with a payload
        return np.array([0xFFC00001], dtype=np.uint32).view(np.float32)[0]
    return np.float32(float(tok))


def _golden():
    row, cases = None, []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("row "):
            row = np.array([_f32(t) for t in line.split()[1:]], dtype=np.float32)
        else:
            k, sel = line[2:].split(":")
            cases.append((int(k), np.array([int(x) for x in sel.split()], dtype=np.int32)))
    return row, cases


def _check_golden(fn):
    row, cases = _golden()
    return all(np.array_equal(fn(row, k), sel) for k, sel in cases)


def _pairwise_ok(fn, row, k):
    """The defining property, checked over all pairs."""
    sel = fn(row, k)
    x = row.astype(np.float64)
    ok = ~np.isnan(x) & (x != -np.inf)
    nvalid = int(ok.sum())
    m = min(k, nvalid)
    if not (np.all(sel[m:] == -1) and np.all(np.diff(sel[:m]) > 0)):
        return False
    kept = set(int(s) for s in sel[:m])
    if not all(ok[s] for s in kept):
        return False
    for s in kept:
        for u in range(x.size):
            if ok[u] and u not in kept and not (x[s] > x[u] or (x[s] == x[u] and s < u)):
                return False
    return True


def _special_row(rng, n):
    """Few distinct values (many ties) with NaN, +-inf and +-0 sprinkled in."""
    x = rng.integers(-3, 4, size=n).astype(np.float32) / np.float32(2)
    x[rng.random(n) < 0.1] = np.nan
    x[rng.random(n) < 0.1] = -np.inf
    x[rng.random(n) < 0.05] = np.inf
    z = rng.random(n) < 0.1
    x[z] = np.where(rng.random(int(z.sum())) < 0.5, np.float32(-0.0), np.float32(0.0))
    return x


def test_golden_hand_worked():
    assert _check_golden(select_topk_general_row)


@pytest.mark.parametrize("seed", range(6))
def test_pairwise_brute_force_small(seed):
    rng = np.random.default_rng(seed)
    for _ in range(20):
        n = int(rng.integers(0, 64))
        x = _special_row(rng, n)
        for k in (1, 3, 17, 64):
            assert _pairwise_ok(select_topk_general_row, x, k)


def test_distinct_values_match_library_topk():
    rng = np.random.default_rng(7)
    for n, k in ((1000, 10), (5000, 2048), (300, 300)):
        x = rng.permutation(n).astype(np.float32) - np.float32(n / 2)   # distinct finite values
        ref = torch.topk(torch.from_numpy(x), k).indices.numpy()
        assert np.array_equal(select_topk_general_row(x, k), np.sort(ref))


def test_special_cases():
    assert np.all(select_topk_general_row(np.array([np.nan, -np.inf, np.nan], dtype=np.float32), 4) == -1)
    assert np.all(select_topk_general_row(np.zeros(0, dtype=np.float32), 3) == -1)
    eq = np.full(100, 2.5, dtype=np.float32)
    assert np.array_equal(select_topk_general_row(eq, 7), np.arange(7))
    inf = np.array([1.0, np.inf, 5.0, np.inf], dtype=np.float32)
    assert np.array_equal(select_topk_general_row(inf, 2), [1, 3])
    neg = np.array([-5.0, -1.0, -3.0, -1e30], dtype=np.float32)          # all negative: order kept
    assert np.array_equal(select_topk_general_row(neg, 2), [1, 2])


def test_row_lens_clamp():
    rng = np.random.default_rng(8)
    s = rng.standard_normal((4, 50)).astype(np.float32)
    got = topk_general(s, 5, row_lens=[50, 3, 0, 999])
    assert np.array_equal(got[0], select_topk_general_row(s[0], 5))
    assert np.array_equal(got[1], select_topk_general_row(s[1, :3], 5))
    assert np.all(got[2] == -1)
    assert np.array_equal(got[3], select_topk_general_row(s[3], 5))


# ---- planted mistakes: each must be rejected by a pin ---------------------------------------

def _variant(nan_largest=False, high_index_wins=False, neg_inf_selectable=False, signed_zero=False):
    def fn(row, k):
        x = np.asarray(row, dtype=np.float32)
        bits = x.view(np.uint32).astype(np.int64)
        pos = np.arange(x.size)
        ok = np.ones(x.size, bool) if nan_largest else ~np.isnan(x)
        if not neg_inf_selectable:
            ok &= x != -np.inf
        v = x.astype(np.float64)
        if nan_largest:
            v = np.where(np.isnan(v), np.inf, v)
            big = np.isnan(x)
        else:
            big = np.zeros(x.size, bool)
        tie = -pos if high_index_wins else pos
        zero_rank = np.where(signed_zero & (v == 0), (bits >> 31) == 0, 0) if signed_zero else np.zeros(x.size)
        order = np.lexsort((tie[ok], -zero_rank[ok], -v[ok], -big[ok].astype(np.int64)))
        keep = np.sort(pos[ok][order[:k]])
        out = np.full(k, -1, dtype=np.int32)
        out[:keep.size] = keep
        return out
    return fn


@pytest.mark.parametrize("mistake", ["nan_largest", "high_index_wins", "neg_inf_selectable", "signed_zero"])
def test_planted_mistakes_are_caught(mistake):
    fn = _variant(**{mistake: True})
    rng = np.random.default_rng(9)
    pairwise = all(_pairwise_ok(fn, _special_row(rng, 40), k) for k in (1, 5, 20) for _ in range(5))
    assert not (_check_golden(fn) and pairwise)


def test_variant_without_mistakes_passes():
    """The planted-mistake harness itself is sound: with no mistake it agrees with the pins."""
    assert _check_golden(_variant())
