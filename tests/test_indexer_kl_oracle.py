"""Pins of the dense warm-up KL oracle (oracle/indexer_kl.py): hand-worked KL values
(tests/golden/indexer_kl.txt), central differences of the summed loss for every gradient,
the per-head attention weights against the (separately pinned) attention oracle, and special
cases.  Planted mistakes in a copy of the rule must each fail a pin."""
import math
import os

import numpy as np
import pytest

from oracle import dsa_oracle as O
from oracle.indexer_kl import kl_row, kl_warmup

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "indexer_kl.txt")


def _golden():
    out = {}
    for line in open(GOLDEN):
        if line.startswith("case "):
            _, name, val = line.split()
            out[name] = float(val)
    return out


def _two_key_case(head_logits):
    """Keys chosen so that head h's logits are head_logits[h]: d = 2, k_s = (0, 1) and q_h = (0, z1) for
    logits (0, z1) with scale 1; indexer scores equal (q_I = 0) so r is uniform."""
    Hq = len(head_logits)
    q = np.array([[0.0, z[1]] for z in head_logits])[None]          # [1, Hq, 2]
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])                        # [2, 1, 2]
    # logits of head h: scale * q_h . k_s = (0, z1) for s = 0, 1
    qi = np.zeros((1, 1, 2))
    ki = np.array([[1.0, 0.0], [0.0, 1.0]])
    w = np.ones((1, 1))
    return q, np.broadcast_to(k, (2, 1, 2)), qi, ki, w, Hq


def test_golden_two_key_cases():
    g = _golden()
    for name, logits in (("A", [[0.0, math.log(3)]]), ("B", [[0.0, math.log(3)], [0.0, 0.0]])):
        q, k, qi, ki, w, Hq = _two_key_case(logits)
        kl, p, r, _, _ = kl_row(q[0], k, qi[0], ki, w[0], 1.0)
        assert abs(kl - g[name]) < 1e-12, name
        assert np.allclose(r, [0.5, 0.5])


def _rand(seed, lens=(5, 7), Hq=4, Hkv=2, d=8, H=3, dI=6):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    return (cu, rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, H, dI)),
            rng.standard_normal((T, dI)), rng.uniform(0.2, 1.0, (T, H)), 0.4)


def _loss(args):
    cu, q, k, qi, ki, w, sc = args
    return kl_warmup(cu, q, k, qi, ki, w, sc)[0].sum()


@pytest.mark.parametrize("seed", [1, 2])
def test_gradients_match_central_differences(seed):
    args = _rand(seed)
    cu, q, k, qi, ki, w, sc = args
    # keep away from ReLU kinks so the loss is smooth around the point
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            assert np.abs(qi[t] @ ki[cu[b]:t + 1].T).min() > 1e-3
    _, dq, dk, dw = kl_warmup(cu, q, k, qi, ki, w, sc)
    eps = 1e-6
    for name, arr, grad in (("q_idx", qi, dq), ("k_idx", ki, dk), ("w", w, dw)):
        flat = arr.reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 25)):
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(args)
            flat[j] = old - eps
            lm = _loss(args)
            flat[j] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[j]) < 1e-6 * max(1.0, abs(fd)), (name, j, fd, grad.reshape(-1)[j])


def test_head_weights_match_attention_oracle():
    """Each head's softmax is the attention oracle's weights: with one-hot V rows the attention
    output of head h is exactly its weight vector, and the mean over heads is p."""
    rng = np.random.default_rng(3)
    n, Hq, Hkv, d = 6, 4, 2, 8
    q = rng.standard_normal((Hq, d))
    k = rng.standard_normal((n, Hkv, d))
    v = np.zeros((n, Hkv, d))
    for s in range(n):
        v[s, :, s] = 1.0
    out = O.attention_row(q, k, v, 0.3)                 # [Hq, d]
    _, p, _, _, _ = kl_row(q, k, np.zeros((1, 2)), np.zeros((n, 2)), np.ones(1), 0.3)
    assert np.allclose(out[:, :n].mean(axis=0), p, atol=1e-14)


def test_special_cases():
    cu, q, k, qi, ki, w, sc = _rand(4)
    kl, dq, dk, dw = kl_warmup(cu, q, k, qi, ki, w, sc)
    assert kl[0] == 0.0 and kl[cu[1]] == 0.0              # one key: p = r = [1]
    assert np.all(dw[0] == 0) and np.all(dq[0] == 0)
    assert np.all(kl >= -1e-15)
    # uniform target and uniform indexer -> zero loss and zero gradients
    kl0, dq0, dk0, dw0 = kl_warmup(cu, np.zeros_like(q), k, np.zeros_like(qi), ki, w, sc)
    assert np.allclose(kl0, 0, atol=1e-15) and np.allclose(dw0, 0, atol=1e-15)


# ---- planted mistakes ----------------------------------------------------------------------

def _kl_variant(mistake):
    def row(q_t, k_ctx, qi_t, ki_ctx, w_t, scale):
        Hq, Hkv = q_t.shape[0], k_ctx.shape[1]
        grp = Hq // Hkv
        z = np.stack([scale * (k_ctx[:, h // grp, :] @ q_t[h]) for h in range(Hq)])
        if mistake == "average_logits":
            e = np.exp(z.mean(0) - z.mean(0).max())
            p = e / e.sum()
        else:
            e = np.exp(z - z.max(1, keepdims=True))
            p = (e / e.sum(1, keepdims=True)).mean(0)
        c = qi_t @ ki_ctx.T
        sco = (w_t[:, None] * np.maximum(c, 0)).sum(0)
        r = np.exp(sco - sco.max())
        r /= r.sum()
        if mistake == "reversed":
            return float(np.sum(r * np.log(r / p)))
        return float(np.sum(p * np.log(p / r)))
    return row


@pytest.mark.parametrize("mistake", ["average_logits", "reversed"])
def test_planted_forward_mistakes_are_caught(mistake):
    g = _golden()
    fn = _kl_variant(mistake)
    ok = True
    for name, logits in (("A", [[0.0, math.log(3)]]), ("B", [[0.0, math.log(3)], [0.0, 0.0]])):
        q, k, qi, ki, w, _ = _two_key_case(logits)
        ok &= abs(fn(q[0], k, qi[0], ki, w[0], 1.0) - g[name]) < 1e-9
    assert not ok


@pytest.mark.parametrize("mistake", ["no_w_in_dq", "no_gate_in_dk", "sign"])
def test_planted_backward_mistakes_are_caught(mistake):
    args = _rand(5)
    cu, q, k, qi, ki, w, sc = args
    _, dq, dk, dw = kl_warmup(cu, q, k, qi, ki, w, sc)
    if mistake == "no_w_in_dq":
        dq = dq / np.repeat(w[:, :, None], dq.shape[2], axis=2)
    elif mistake == "no_gate_in_dk":
        dk = dk * 0
        for b in range(len(cu) - 1):
            for t in range(cu[b], cu[b + 1]):
                _, _, _, g, c = kl_row(q[t], k[cu[b]:t + 1], qi[t], ki[cu[b]:t + 1], w[t], sc)
                dk[cu[b]:t + 1] += (g[None, :] * w[t][:, None]).T @ qi[t]
    else:
        dw = -dw
    eps = 1e-6
    bad = False
    for arr, grad in ((qi, dq), (ki, dk), (w, dw)):
        flat = arr.reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 10)):
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(args)
            flat[j] = old - eps
            lm = _loss(args)
            flat[j] = old
            bad |= abs((lp - lm) / (2 * eps) - grad.reshape(-1)[j]) > 1e-5
    assert bad


def test_kl_finite_when_indexer_softmax_underflows():
    """Indexer scores 0 and 1000: r = [e^-1000 / (1 + e^-1000), ~1] underflows in float64, but
    KL(p || r) is finite: with p = [1/2, 1/2] it equals 1/2 ln(1/2 / r0) + 1/2 ln(1/2 / r1)
    = 1/2 (1000 + ln(1 + e^-1000)) + ln(1/2) + 1/2 ln(1 + e^-1000) = 500 - ln 2 (to double precision)."""
    q = np.zeros((1, 1, 2))                                  # equal main logits -> p = [1/2, 1/2]
    k = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    qi = np.array([[0.0, 1000.0]])                           # scores c = q_I . k_I = [0, 1000]
    ki = np.array([[1.0, 0.0], [0.0, 1.0]])
    kl, p, r, _, _ = kl_row(q[0], k, qi, ki, np.ones(1), 1.0)
    assert np.allclose(p, [0.5, 0.5]) and r[0] == 0.0
    assert abs(kl - (500.0 - math.log(2.0))) < 1e-9
