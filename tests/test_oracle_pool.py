"""The parallel oracle runner used by the full-size GPU parity tests (tests/oracle_pool.py),
checked on the CPU: worker processes rebuilding the seeded inputs must reproduce the oracle run
in this process row for row, and a planted index or output mistake must be reported."""
import numpy as np

from oracle import dsa_oracle as O
from sparse_attention_long_04_amd import inputs as gen
from sparse_attention_long_04_amd import workloads

import oracle_pool


def test_prefill_pool_matches_in_process_oracle_and_catches_mistakes():
    name = workloads.TINY
    p = workloads.make(name)
    o = O.Prefill(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.q, p.k, p.v, p.idx_dtype, p.topk, p.softmax_scale)
    rows = np.array([0, 1, 255, 256, 257, 1000, 2047], dtype=np.int64)
    sel, out = o.rows(rows)
    drows = rows[[1, 4, 6]]
    dense = o.dense_rows(drows)
    bad, eo, ed = oracle_pool.check_prefill(name, rows, sel.astype(np.int32), out, dense, drows, n_workers=2, chunk=3)
    assert bad == [] and eo.max_abs == 0.0 and ed.max_abs == 0.0 and ed.count == dense.size
    sel2, out2 = sel.copy(), out.copy()
    sel2[5, 3] += 1                 # row 1000: one wrong index
    out2[2, 7, 9] += 0.02           # row 255: one output off by more than the bar
    bad, eo, _ = oracle_pool.check_prefill(name, rows, sel2.astype(np.int32), out2, n_workers=2, chunk=2)
    assert bad == [1000]
    assert abs(eo.max_abs - 0.02) < 1e-12


def test_decode_pool_every_step_matches_in_process_oracle():
    spec = dict(batch=3, ctx_len=700, capacity=704, steps=4, idx_heads=8, idx_dim=128, idx_dtype="fp8_e4m3",
                topk=64, seed=77)
    d = gen.make_decode(**spec)
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    idx, out = [], []
    for i in range(spec["steps"]):
        s = d.step(i)
        n = d.ctx_len + i
        kc[:, n], kk[:, n], vv[:, n] = s["k_idx_new"], s["k_new"], s["v_new"]
        lens = np.full(d.batch, n + 1)
        a, b = O.decode_step(kc, kk, vv, lens, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk, d.softmax_scale)
        idx.append(a.astype(np.int32))
        out.append(b)
    idx, out = np.stack(idx), np.stack(out)
    bad, eo = oracle_pool.check_decode(spec, idx, out, n_workers=2)
    assert bad == [] and eo.max_abs == 0.0 and eo.count == out.size
    idx[2, 1, 0] = -1
    bad, _ = oracle_pool.check_decode(spec, idx, out, n_workers=2)
    assert bad == [(2, 1)]
