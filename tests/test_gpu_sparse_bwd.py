"""GPU parity of the sparse attention backward (dsa_sparse_attention_fwd_lse +
dsa_sparse_attention_bwd, through the C ABI) against the float64 oracle
(oracle/sparse_attention_bwd.py).

Tolerances: the gradients use D = dO . O from the bf16 forward output (as the API takes it),
whose rounding (2^-9 relative) reaches dS = P (dP - D) at ~1e-3 of its scale; S and dP are fp32
(fp16 copies of the bf16 inputs, exact in fp16's normal range, and fp32 MFMA accumulation) and
P and dS enter the final products rounded to fp16 (2^-11 relative, unbiased, so the mean error
of a sum over many keys shrinks with their count).  Bars: each gradient within 1e-2 of its
largest reference magnitude element by element, and within mean-relative 3e-3; lse within 1e-4
absolute; out as the forward (max-abs 1e-2, mean-rel 2e-3)."""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from oracle.sparse_attention_bwd import sparse_attention_bwd
from sparse_attention_long_04_amd import dsa
from sparse_attention_long_04_amd import inputs as gen
from sparse_attention_long_04_amd.runtime import PrefillBatch, bf16_to_float

from gpu_util import assert_out_close, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _run(p, seed=91):
    pb = PrefillBatch(p)
    pb.index_topk()
    T, Hq, d = p.q.shape
    Hkv = p.k.shape[1]
    out = torch.empty_like(pb.out)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attention_fwd_lse(pb.shape, pb.q, pb.k, pb.v, pb.topk_idx, out, lse)
    dout_np = gen.make_grad_bf16((T, Hq, d), seed)
    dout = torch.from_numpy(dout_np.view(np.int16)).cuda()
    ws = torch.empty(max(dsa.dsa_sparse_attention_bwd_workspace_size(pb.shape), 256), dtype=torch.uint8, device="cuda")
    dq = torch.empty((T, Hq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((T, Hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty((T, Hkv, d), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attention_bwd(pb.shape, pb.q, pb.k, pb.v, pb.topk_idx, out, lse, dout, dq, dk, dv, ws)
    torch.cuda.synchronize()
    res = dict(idx=pb.topk_idx.cpu().numpy(), out=bf16_to_float(out), lse=lse.cpu().numpy().astype(np.float64),
               dq=dq.cpu().numpy().astype(np.float64), dk=dk.cpu().numpy().astype(np.float64),
               dv=dv.cpu().numpy().astype(np.float64), dout=O.decode(dout_np, "bf16"))
    return res


def _grad_close(name, got, ref):
    big = max(np.abs(ref).max(), 1e-12)
    err = np.abs(got - ref)
    assert err.max() <= 1e-2 * big, f"{name}: max err {err.max():.3e} vs {big:.3e}"
    mrel = err.sum() / max(np.abs(ref).sum(), 1e-30)
    assert mrel <= 3e-3, f"{name}: mean-rel {mrel:.3e}"


CASES = {
    # name: (lengths, k, q_heads, kv_heads, query_corr)
    "single_700": ([700], 256, 32, 4, None),
    "varlen": ([129, 0, 17, 300, 1, 520], 100, 32, 4, None),
    "corr_1500": ([1500], 512, 32, 4, 0.95),
    "g16": ([600], 128, 16, 1, None),
    "g4": ([450, 70], 64, 16, 4, None),
    "g2": ([333, 64], 96, 8, 4, None),
    "k_ge_L": ([300], 512, 32, 4, None),
    # dk/dv partials are summed over 4096-row slices of a sequence: rows over 3 slices, and two
    # sequences of 2 slices each (slices count from each sequence's start)
    "slices_9000": ([9000], 128, 8, 1, None),
    "slices_varlen": ([5000, 4500], 96, 8, 2, None),
}


@pytest.mark.parametrize("name", list(CASES))
def test_sparse_bwd_parity(name):
    lens, k, hq, hkv, rho = CASES[name]
    p = gen.make_prefill(lens, idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=k, seed=92,
                         video=True, q_heads=hq, kv_heads=hkv, query_corr=rho)
    print(f"[bwd] {name}: T={p.total_tokens}", flush=True)
    r = _run(p)
    q, kk, vv = O.decode(p.q, "bf16"), O.decode(p.k, "bf16"), O.decode(p.v, "bf16")
    out, dq, dk, dv = sparse_attention_bwd(p.cu_seqlens, q, kk, vv, r["idx"], r["dout"], p.softmax_scale)
    assert_out_close(r["out"], out, f"bwd forward {name}")
    # lse: natural log of sum exp over the selected keys
    for t in range(0, p.total_tokens, max(1, p.total_tokens // 40)):
        b = int(np.searchsorted(p.cu_seqlens, t, side="right") - 1)
        sel = r["idx"][t][r["idx"][t] >= 0] + p.cu_seqlens[b]
        for h in range(0, hq, 5):
            z = p.softmax_scale * (kk[sel, h // (hq // hkv)] @ q[t, h])
            ref = z.max() + np.log(np.exp(z - z.max()).sum())
            assert abs(r["lse"][t, h] - ref) < 1e-4, (t, h)
    _grad_close("dq", r["dq"], dq)
    _grad_close("dk", r["dk"], dk)
    _grad_close("dv", r["dv"], dv)


def test_sparse_bwd_deterministic():
    p = gen.make_prefill([2000], idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=512, seed=93,
                         video=True)
    a, b = _run(p), _run(p)
    for key in ("dq", "dk", "dv"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.timeout(900)
def test_sparse_bwd_32k_identities():
    """32768 tokens, k = 2048 (the size the benchmark times).  The scores are bilinear in q and
    k, so sum <q, dq> = sum <k, dk> (both = sum dS z); and sum <v, dv> = sum <dO, O>.  Both hold at
    any size; checked against float64 sums of the kernel's outputs."""
    p = gen.make_prefill([32768], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048, seed=94,
                         video=True)
    r = _run(p)
    q, kk, vv = O.decode(p.q, "bf16"), O.decode(p.k, "bf16"), O.decode(p.v, "bf16")
    a, b = float((q * r["dq"]).sum()), float((kk * r["dk"]).sum())
    scale_ab = float(np.abs(q * r["dq"]).sum())
    assert abs(a - b) <= 1e-3 * scale_ab, (a, b, scale_ab)
    c, d = float((vv * r["dv"]).sum()), float((r["dout"] * r["out"]).sum())
    scale_cd = float(np.abs(r["dout"] * r["out"]).sum())
    assert abs(c - d) <= 1e-3 * scale_cd, (c, d, scale_cd)
    # and a few rows' dq against the oracle (dq only needs the row itself)
    rows = np.array([0, 5, 2047, 2048, 20000, 32767])
    _, rdq, _, _ = sparse_attention_bwd(p.cu_seqlens, q, kk, vv, r["idx"], r["dout"], p.softmax_scale, rows=rows)
    _grad_close("dq rows", r["dq"][rows], rdq[rows])
