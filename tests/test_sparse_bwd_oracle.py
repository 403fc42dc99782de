"""Pins of the sparse attention backward oracle (oracle/sparse_attention_bwd.py): central
differences of sum <dO, O> for every gradient, torch autograd through float64 causal SDPA when
every row keeps all its keys (k >= L), the forward against the attention oracle, and planted
mistakes that each pin must catch."""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from oracle.sparse_attention_bwd import sparse_attention_bwd


def _case(seed, lens=(6, 9), Hq=4, Hkv=2, d=8, k=4):
    rng = np.random.default_rng(seed)
    T = sum(lens)
    cu = np.concatenate([[0], np.cumsum(lens)])
    idx = np.full((T, k), -1, dtype=np.int32)
    for b in range(len(lens)):
        for i in range(lens[b]):
            n = min(k, i + 1)
            idx[cu[b] + i, :n] = np.sort(rng.choice(i + 1, size=n, replace=False))
    return (cu, rng.standard_normal((T, Hq, d)), rng.standard_normal((T, Hkv, d)), rng.standard_normal((T, Hkv, d)),
            idx, rng.standard_normal((T, Hq, d)), 0.35)


def _loss(cu, q, k, v, idx, dout, sc):
    return float((sparse_attention_bwd(cu, q, k, v, idx, dout, sc)[0] * dout).sum())


@pytest.mark.parametrize("seed", [1, 2])
def test_gradients_match_central_differences(seed):
    cu, q, k, v, idx, dout, sc = _case(seed)
    _, dq, dk, dv = sparse_attention_bwd(cu, q, k, v, idx, dout, sc)
    eps = 1e-6
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        flat = arr.reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 30)):
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(cu, q, k, v, idx, dout, sc)
            flat[j] = old - eps
            lm = _loss(cu, q, k, v, idx, dout, sc)
            flat[j] = old
            fd = (lp - lm) / (2 * eps)
            assert abs(fd - grad.reshape(-1)[j]) < 1e-6 * max(1.0, abs(fd))


def test_full_selection_matches_torch_autograd_sdpa():
    """k >= L: every row keeps all its keys, so the gradients are dense causal attention's,
    computed here by torch autograd through float64 scaled_dot_product_attention."""
    cu, q, k, v, _, dout, sc = _case(3, lens=(11,), k=11)
    T = 11
    idx = np.array([[s if s <= t else -1 for s in range(T)] for t in range(T)], dtype=np.int32)
    out, dq, dk, dv = sparse_attention_bwd(cu, q, k, v, idx, dout, sc)
    Hq, Hkv = q.shape[1], k.shape[1]
    tq = torch.tensor(q.transpose(1, 0, 2), requires_grad=True)
    tk = torch.tensor(k.transpose(1, 0, 2), requires_grad=True)
    tv = torch.tensor(v.transpose(1, 0, 2), requires_grad=True)
    kk = tk.repeat_interleave(Hq // Hkv, dim=0)
    vv = tv.repeat_interleave(Hq // Hkv, dim=0)
    o = torch.nn.functional.scaled_dot_product_attention(tq, kk, vv, is_causal=True, scale=sc)
    (o * torch.tensor(dout.transpose(1, 0, 2))).sum().backward()
    assert np.allclose(out, o.detach().numpy().transpose(1, 0, 2), atol=1e-12)
    assert np.allclose(dq, tq.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    assert np.allclose(dk, tk.grad.numpy().transpose(1, 0, 2), atol=1e-12)
    assert np.allclose(dv, tv.grad.numpy().transpose(1, 0, 2), atol=1e-12)


def test_forward_matches_attention_oracle():
    cu, q, k, v, idx, dout, sc = _case(4)
    out = sparse_attention_bwd(cu, q, k, v, idx, dout, sc)[0]
    for b in range(len(cu) - 1):
        for t in range(cu[b], cu[b + 1]):
            sel = idx[t][idx[t] >= 0] + cu[b]
            assert np.allclose(out[t], O.attention_row(q[t], k[sel], v[sel], sc), atol=1e-13)


@pytest.mark.parametrize("mistake", ["no_D", "dk_unscaled", "dv_from_ds"])
def test_planted_mistakes_are_caught(mistake):
    cu, q, k, v, idx, dout, sc = _case(5)
    _, dq, dk, dv = sparse_attention_bwd(cu, q, k, v, idx, dout, sc)
    T, Hq, d = q.shape
    grp = Hq // k.shape[1]
    if mistake == "dk_unscaled":
        dk = dk / sc
    else:
        dq2, dk2, dv2 = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        for b in range(len(cu) - 1):
            for t in range(cu[b], cu[b + 1]):
                sel = idx[t][idx[t] >= 0].astype(np.int64) + cu[b]
                for h in range(Hq):
                    g = h // grp
                    z = sc * (k[sel, g] @ q[t, h])
                    p = np.exp(z - z.max())
                    p /= p.sum()
                    dp = v[sel, g] @ dout[t, h]
                    ds = p * dp if mistake == "no_D" else p * (dp - dp @ p)
                    dq2[t, h] = sc * ds @ k[sel, g]
                    dk2[sel, g] += sc * ds[:, None] * q[t, h]
                    dv2[sel, g] += (ds if mistake == "dv_from_ds" else p)[:, None] * dout[t, h]
        dq, dk, dv = dq2, dk2, dv2
    eps = 1e-6
    bad = False
    for arr, grad in ((q, dq), (k, dk), (v, dv)):
        flat = arr.reshape(-1)
        for j in range(0, flat.size, max(1, flat.size // 10)):
            old = flat[j]
            flat[j] = old + eps
            lp = _loss(cu, q, k, v, idx, dout, sc)
            flat[j] = old - eps
            lm = _loss(cu, q, k, v, idx, dout, sc)
            flat[j] = old
            bad |= abs((lp - lm) / (2 * eps) - grad.reshape(-1)[j]) > 1e-5
    assert bad
