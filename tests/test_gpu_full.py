"""GPU parity at the full workload sizes, through the same entry points and launch
configuration that bench.py times.

* 32768-token prefill: every row (indices, output, and the dense causal output);
* 128K video prefill and the packed 256K varlen prefill: a deterministic row sample — each
  sequence's first and last 2048 rows, the rows at every frame boundary, and 4096 seeded rows;
  dense on a subset of it;
* 16 x 128K decode: every sequence at every one of the 64 steps.

The oracle rows run in worker processes (tests/oracle_pool.py) that rebuild the seeded inputs.
Bars: selected indices bit-exact; bf16 outputs within max-abs 1e-2 and mean-rel 2e-3."""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_04_amd import workloads
from sparse_attention_long_04_amd.runtime import DecodeState, PrefillBatch, bf16_to_float

import oracle_pool
from gpu_util import MAX_ABS, MEAN_REL, gpu_available, survey_sample_rows

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]


def _assert_bars(e, what):
    print(f"  {what}: {e.count} values, max_abs={e.max_abs:.3e} mean_rel={e.mean_rel:.3e}", flush=True)
    assert e.count > 0 and e.finite, what
    assert e.max_abs <= MAX_ABS, f"{what}: max abs {e.max_abs}"
    assert e.mean_rel <= MEAN_REL, f"{what}: mean rel {e.mean_rel}"


def _check_prefill(name, rows, dense_rows):
    p = workloads.make(name)
    print(f"[full] {name}: T={p.total_tokens} lengths={list(p.lengths)}; {len(rows)} rows checked, "
          f"{0 if dense_rows is None else len(dense_rows)} dense", flush=True)
    pb = PrefillBatch(p)
    pb.prefill()
    r = torch.from_numpy(rows).to(pb.topk_idx.device)
    idx = pb.topk_idx[r].cpu().numpy()
    out = bf16_to_float(pb.out[r])
    dense = None
    if dense_rows is not None:
        d = pb.dense(out=torch.empty_like(pb.out))
        dense = bf16_to_float(d[torch.from_numpy(dense_rows).to(d.device)])
        del d
    del pb, p
    torch.cuda.empty_cache()
    bad, eo, ed = oracle_pool.check_prefill(name, rows, idx, out, dense, dense_rows)
    assert not bad, f"index mismatch on {len(bad)} rows, first {bad[:10]}"
    _assert_bars(eo, name)
    if dense_rows is not None:
        _assert_bars(ed, name + " dense")


@pytest.mark.timeout(900)
def test_prefill_32k_every_row():
    T = sum(workloads.lengths_of(workloads.P32K))
    rows = np.arange(T, dtype=np.int64)
    _check_prefill(workloads.P32K, rows, rows)


@pytest.mark.timeout(900)
def test_prefill_128k_video_sampled():
    cu = np.concatenate([[0], np.cumsum(workloads.lengths_of(workloads.P128K))])
    rows = survey_sample_rows(cu, seed=128)
    rng = np.random.default_rng(129)
    frames = survey_sample_rows(cu, seed=128, edge=0, n_random=0)        # frame boundaries only
    dense = np.unique(np.concatenate([frames, rng.choice(rows, 1024, replace=False)]))
    _check_prefill(workloads.P128K, rows, dense)


@pytest.mark.timeout(900)
def test_varlen_256k_sampled():
    cu = np.concatenate([[0], np.cumsum(workloads.lengths_of(workloads.VARLEN))])
    rows = survey_sample_rows(cu, seed=256)
    _check_prefill(workloads.VARLEN, rows, None)


@pytest.mark.timeout(900)
def test_prefill_single_256k_sequence_sampled():
    """One 262144-token video-like sequence (the longest context the pages name): the indexer's
    chunked score buffer (512 blocks of 16 rows x 262144 scores, 8 GiB) bounds the workspace to
    about 10 GiB instead of the 137 GB score triangle.
    Rows: the first 256, the last 512, every 16th frame boundary and 256 seeded rows."""
    L = 262144
    p = workloads.make(workloads.P128K, lengths=[L])
    pb = PrefillBatch(p)
    ws_gib = pb.ws.numel() / 2**30
    print(f"[full] single 256K sequence: workspace {ws_gib:.2f} GiB", flush=True)
    assert ws_gib < 12
    pb.prefill()
    rng = np.random.default_rng(262)
    rows = np.unique(np.concatenate([np.arange(256), np.arange(L - 512, L), np.arange(1024, L, 16 * 1024) - 1,
                                     np.arange(1024, L, 16 * 1024), rng.integers(0, L, 256)]))
    r = torch.from_numpy(rows).to(pb.topk_idx.device)
    idx = pb.topk_idx[r].cpu().numpy()
    out = bf16_to_float(pb.out[r])
    del pb, p
    torch.cuda.empty_cache()
    bad, eo, _ = oracle_pool.check_prefill(workloads.P128K, rows, idx, out, lengths=[L], chunk=8)
    assert not bad, f"index mismatch on {len(bad)} rows, first {bad[:10]}"
    _assert_bars(eo, "single 256K sequence")


@pytest.mark.timeout(900)
def test_decode_16x128k_every_step():
    d = workloads.make(workloads.DECODE)
    st = DecodeState(d)
    steps = workloads.WORKLOADS[workloads.DECODE]["steps"]
    idx, out = [], []
    kc, kk, vv = d.k_idx_cache, d.k_cache, d.v_cache   # host copies, appended in step
    for i in range(steps):
        s = st.load_step(i)
        st.append()
        n = int(st.len_host[0])
        kc[:, n - 1], kk[:, n - 1], vv[:, n - 1] = s["k_idx_new"], s["k_new"], s["v_new"]
        st.decode()
        idx.append(st.topk_idx.cpu().numpy())
        out.append(bf16_to_float(st.out))
        if i == steps - 1:
            seqs = [0, 7, 15]
            dense = bf16_to_float(st.dense(out=torch.empty_like(st.out)))[seqs]
            dref = O.dense_decode(kk, vv, st.len_host, s["q"], d.softmax_scale, seqs=seqs)
    print(f"[full] decode: {steps} steps of {d.batch} sequences run; oracle on every one", flush=True)
    # appended rows landed where the host copy has them
    lo, hi = d.ctx_len, d.ctx_len + steps
    assert np.array_equal(st.k_idx_cache[:, lo:hi].cpu().numpy(), kc[:, lo:hi])
    assert np.array_equal(st.k_cache[:, lo:hi].cpu().numpy().view(np.uint16), kk[:, lo:hi])
    assert np.array_equal(st.v_cache[:, lo:hi].cpu().numpy().view(np.uint16), vv[:, lo:hi])
    del st, kc, kk, vv, d
    torch.cuda.empty_cache()
    e = oracle_pool.ErrSum()
    e.add(dense, dref)
    _assert_bars(e, "dense decode (final step, sequences 0, 7, 15)")
    bad, eo = oracle_pool.check_decode(workloads.DECODE, np.stack(idx), np.stack(out))
    assert not bad, f"index mismatch at (step, sequence) {bad[:10]} ({len(bad)} in all)"
    _assert_bars(eo, "decode, every step and sequence")


@pytest.mark.timeout(900)
def test_topk_rows_past_single_pass_limit():
    """One 200000-token video sequence: rows of up to 196608 keys take the top-k's single-pass
    path, longer rows its exact two-pass select.  Rows on both sides of that boundary, and the
    sequence end, must match the oracle exactly."""
    from sparse_attention_long_04_amd import inputs as gen
    n = 200000
    p = gen.make_prefill([n], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048, seed=51,
                         video=True)
    print(f"[full] topk past the single-pass limit: T={n}", flush=True)
    pb = PrefillBatch(p)
    pb.index_topk()
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(196600, 196616), [n - 1], rng.integers(150000, n, 4)]))
    idx = pb.topk_idx[torch.from_numpy(rows).to(pb.topk_idx.device)].cpu().numpy()
    del pb
    torch.cuda.empty_cache()
    o = O.Prefill(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.q, p.k, p.v, p.idx_dtype, p.topk, p.softmax_scale)
    bad = [int(t) for t, got in zip(rows, idx) if not np.array_equal(got, O.select_topk_row(o.scores(int(t)), p.topk))]
    assert not bad, f"index mismatch on rows {bad}"
