"""GPU parity of the HIP path (through the C ABI) against the float64 CPU oracle, at sizes the
oracle finishes in seconds: several tiles, ragged tails, empty and short sequences.

Bars: indexer scores and selected indices bit-exact; bf16 outputs within max-abs 1e-2 and
mean-rel 2e-3 of the oracle."""
import numpy as np
import pytest
import torch

from oracle import dsa_oracle as O
from sparse_attention_long_04_amd import dsa
from sparse_attention_long_04_amd import inputs as gen
from sparse_attention_long_04_amd import workloads
from sparse_attention_long_04_amd.runtime import DecodeState, PrefillBatch, _dev, bf16_to_float

from gpu_util import assert_out_close, gpu_available

pytestmark = [pytest.mark.gpu, pytest.mark.skipif(not gpu_available(), reason="needs a GPU")]

CASES = {
    # name: (lengths, idx_heads, idx_dim, idx_dtype, idx_range, topk, video)
    "tiny_bf16_2k": ([2048], 16, 64, "bf16", 8, 256, False),
    "fp8_ragged_700": ([700], 64, 128, "fp8_e4m3", 4, 256, False),
    "bf16_d128_333": ([333], 32, 128, "bf16", 8, 64, False),
    "fp8_varlen_empty": ([129, 0, 17, 300, 1000, 1], 64, 128, "fp8_e4m3", 4, 100, True),
    "fp8_video_3k": ([3100], 64, 128, "fp8_e4m3", 4, 2048, True),
}


def make(name, seed=7):
    lens, H, dI, dt, rng_, k, video = CASES[name]
    return gen.make_prefill(lens, idx_heads=H, idx_dim=dI, idx_dtype=dt, idx_range=rng_, topk=k, seed=seed,
                            video=video)


def oracle_of(p):
    return O.Prefill(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.q, p.k, p.v, p.idx_dtype, p.topk, p.softmax_scale)


@pytest.mark.parametrize("name", list(CASES))
def test_index_scores_bitexact(name):
    p = make(name)
    print(f"[index_scores] {name} T={p.total_tokens}", flush=True)
    pb = PrefillBatch(p)
    got = pb.index_scores().cpu().numpy().astype(np.float64)
    torch.cuda.synchronize()
    ref = O.index_score_matrix(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.idx_dtype)
    assert got.shape == ref.shape
    bad = np.argwhere(~((got == ref) | (np.isneginf(got) & np.isneginf(ref))))
    assert bad.size == 0, f"{len(bad)} mismatches, first {bad[:5].tolist()}"


@pytest.mark.parametrize("name", list(CASES))
def test_topk_bitexact(name):
    p = make(name)
    print(f"[topk] {name} T={p.total_tokens} k={p.topk}", flush=True)
    pb = PrefillBatch(p)
    pb.index_topk()
    got = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    for t in range(p.total_tokens):
        ref = O.select_topk_row(o.scores(t), p.topk)
        assert np.array_equal(got[t], ref), f"row {t}: {got[t][:8]} vs {ref[:8]}"


@pytest.mark.parametrize("name", ["tiny_bf16_2k", "fp8_ragged_700", "fp8_varlen_empty", "fp8_video_3k"])
def test_prefill_parity(name):
    p = make(name)
    print(f"[prefill] {name} T={p.total_tokens}", flush=True)
    pb = PrefillBatch(p)
    pb.prefill()
    idx = pb.topk_idx.cpu().numpy()
    out = bf16_to_float(pb.out)
    o = oracle_of(p)
    rows = np.arange(p.total_tokens)
    sel, ref = o.rows(rows)
    assert np.array_equal(idx, sel)
    assert_out_close(out, ref, name)


@pytest.mark.parametrize("name", ["fp8_ragged_700", "fp8_varlen_empty", "fp8_video_3k"])
def test_dense_causal_parity(name):
    p = make(name)
    print(f"[dense] {name} T={p.total_tokens}", flush=True)
    pb = PrefillBatch(p)
    out = bf16_to_float(pb.dense())
    ref = oracle_of(p).dense_rows(range(p.total_tokens))
    assert_out_close(out, ref, name + " dense")


def test_sparse_with_k_ge_L_equals_dense():
    p = gen.make_prefill([1000, 37], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=1024,
                         seed=3)
    pb = PrefillBatch(p)
    pb.prefill()
    sparse = bf16_to_float(pb.out)
    dense = bf16_to_float(pb.dense(out=torch.empty_like(pb.out)))
    ref = oracle_of(p).dense_rows(range(p.total_tokens))
    assert_out_close(sparse, ref, "sparse k>=L")
    assert_out_close(dense, ref, "dense")
    assert np.abs(sparse - dense).max() <= 2 * 2.0 ** -8 * max(1.0, np.abs(ref).max())


def test_given_indices_sparse_attention():
    """dsa_sparse_attention on an index set that is not a top-k (every third key, reversed
    padding), checked against the oracle attention over the same sets."""
    p = make("fp8_ragged_700")
    pb = PrefillBatch(p)
    T, K = p.total_tokens, p.topk
    idx = np.full((T, K), -1, dtype=np.int32)
    for t in range(T):
        s = np.arange(0, t + 1, 3)[:K]
        idx[t, : s.size] = s
    pb.topk_idx.copy_(torch.from_numpy(idx))
    pb.sparse_attention()
    out = bf16_to_float(pb.out)
    q, k, v = O.decode_bf16(p.q), O.decode_bf16(p.k), O.decode_bf16(p.v)
    ref = np.stack([O.attention_row(q[t], k[idx[t][idx[t] >= 0]], v[idx[t][idx[t] >= 0]], p.softmax_scale)
                    for t in range(T)])
    assert_out_close(out, ref, "given indices")


def test_prefill_is_deterministic():
    p = make("fp8_video_3k")
    pb = PrefillBatch(p)
    pb.prefill()
    a_idx, a_out = pb.topk_idx.clone(), pb.out.clone()
    pb.out.zero_()
    pb.topk_idx.zero_()
    pb.prefill()
    assert torch.equal(a_idx, pb.topk_idx) and torch.equal(a_out, pb.out)


@pytest.mark.parametrize("ctx,cap,k,steps", [(3000, 3100, 256, 2), (500, 520, 2048, 2), (9000, 9100, 2048, 2)])
def test_decode_parity(ctx, cap, k, steps):
    d = gen.make_decode(3, ctx, cap, steps, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=k, seed=5)
    st = DecodeState(d)
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    for i in range(steps):
        s = st.load_step(i)
        st.append()
        n = int(st.len_host[0])
        kc[:, n - 1], kk[:, n - 1], vv[:, n - 1] = s["k_idx_new"], s["k_new"], s["v_new"]
        st.decode()
        torch.cuda.synchronize()
        print(f"[decode] ctx={ctx} step={i} n={n}", flush=True)
        assert np.array_equal(st.k_idx_cache.cpu().numpy(), kc)
        assert np.array_equal(st.k_cache.cpu().numpy().view(np.uint16), kk)
        assert np.array_equal(st.v_cache.cpu().numpy().view(np.uint16), vv)
        sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                                 d.softmax_scale)
        assert np.array_equal(st.topk_idx.cpu().numpy(), sel)
        assert_out_close(bf16_to_float(st.out), ref, f"decode step {i}")
        dense = bf16_to_float(st.dense(out=torch.empty_like(st.out)))
        assert_out_close(dense, O.dense_decode(kk, vv, st.len_host, s["q"], d.softmax_scale), f"dense decode {i}")


@pytest.mark.parametrize("hq,hkv,k", [(32, 4, 3000), (12, 4, 300), (16, 1, 512), (8, 8, 64), (32, 2, 2048)])
def test_decode_gqa_shapes_and_k(hq, hkv, k):
    """Decode attention for other head layouts, and a selection larger than one workgroup's
    slices (k = 3000 takes the split path with a separate combine)."""
    d = gen.make_decode(2, 3500, 3600, 1, idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", topk=k, seed=57,
                        q_heads=hq, kv_heads=hkv)
    st = DecodeState(d)
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    s = st.load_step(0)
    st.append()
    st.decode()
    torch.cuda.synchronize()
    n = int(st.len_host[0])
    kc[:, n - 1], kk[:, n - 1], vv[:, n - 1] = s["k_idx_new"], s["k_new"], s["v_new"]
    sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                             d.softmax_scale)
    assert np.array_equal(st.topk_idx.cpu().numpy(), sel)
    assert_out_close(bf16_to_float(st.out), ref, f"decode {hq}/{hkv} k={k}")


def test_topk_all_ties_prefill():
    """Degenerate case: every score equal (zero indexer queries) -> each row keeps its first
    min(k, i+1) keys; rows longer than the LDS candidate list take the multi-pass path."""
    p = gen.make_prefill([9000, 300], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048,
                         seed=9)
    p.q_idx[:] = 0
    pb = PrefillBatch(p)
    pb.prefill()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    for t in [0, 5, 2046, 2047, 2048, 5000, 8191, 8192, 8999, 9000, 9299]:
        assert np.array_equal(idx[t], O.select_topk_row(o.scores(t), p.topk)), t
    rows = np.array([0, 2047, 2048, 8999, 9150])
    _, ref = o.rows(rows)
    assert_out_close(bf16_to_float(pb.out)[rows], ref, "all ties")


@pytest.mark.parametrize("zero_q", [False, True])
def test_decode_chunked_topk(zero_q):
    """Caches of ~20K rows: the decode top-k runs over several 4096-key chunks; with zero
    queries every score is 0, the row is flat and the first k keys are kept without a select."""
    d = gen.make_decode(2, 20000, 20064, 1, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=2048, seed=15)
    st = DecodeState(d)
    s = st.load_step(0)
    if zero_q:
        st.step_dev["q_idx"].zero_()
        s["q_idx"][:] = 0
    st.append()
    st.decode()
    torch.cuda.synchronize()
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    kc[:, 20000], kk[:, 20000], vv[:, 20000] = s["k_idx_new"], s["k_new"], s["v_new"]
    sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                             d.softmax_scale)
    assert np.array_equal(st.topk_idx.cpu().numpy(), sel)
    assert_out_close(bf16_to_float(st.out), ref, f"decode chunked zero_q={zero_q}")


def test_index_scores_large_linear_term_bitexact():
    """fp8 queries in [-8, 8] with all weights 1: sum_h w_h q_h reaches several hundred, beyond
    the e4m3 range, so the indexer's linear term runs with a power-of-two block scale."""
    p = gen.make_prefill([520, 77], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=8, topk=64, seed=21)
    p.w_idx[:] = 1.0
    p.q_idx[:, :, :] = p.q_idx[:1, :1, :]  # same query in every head and token: |q_lin| up to 512
    pb = PrefillBatch(p)
    got = pb.index_scores().cpu().numpy().astype(np.float64)
    ref = O.index_score_matrix(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.idx_dtype)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_index_scores_general_weights_close():
    """Weights that are not powers of two: scores are no longer exactly representable.

    Error model of the kernel (score = (sum_h w_h c_h + sum_h w_h |c_h|) / 2, c_h = q_h . k exact):
    * the |c| sum is an fp32 FMA chain over H = 64 heads: <= ~H u sum_h w_h |c_h|  (u = 2^-24);
    * the linear sum contracts q_lin = sum_h w_h q_h (an fp32 chain, <= ~H u sum_h |w_h||q_h,e| per
      dim) against k in fp32 MFMA accumulation (<= ~128 u relative to sum_e |q_lin,e||k_e|);
    * q_lin is split into five e4m3 pieces on a power-of-two scale S per 16-row block with
      max|q_lin| / S in (64, 240]: each piece leaves at most 2^-4 of the residual or the
      subnormal floor 2^-10 S, so the last residual is <= 2^-10 S <= 2^-16 max_blk |q_lin| per dim.
    Bound: 256 u (sum_h w_h |c_h| + sum_e sum_h w_h |q_h,e| |k_e|) + 2^-16 max_blk|q_lin| sum_e |k_e|
    (256 covers 64 + 128 + the piece sums with headroom)."""
    p = make("fp8_ragged_700", seed=22)
    rng = np.random.default_rng(0)
    p.w_idx[:] = rng.uniform(0.01, 1.0, size=p.w_idx.shape).astype(np.float32)
    pb = PrefillBatch(p)
    got = pb.index_scores().cpu().numpy().astype(np.float64)
    ref = O.index_score_matrix(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.idx_dtype)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin)
    q = O.decode(p.q_idx, p.idx_dtype)            # [T, H, d]
    k = O.decode(p.k_idx, p.idx_dtype)            # [T, d]
    w = p.w_idx.astype(np.float64)                # [T, H]
    cu = np.asarray(p.cu_seqlens)
    T = p.total_tokens
    qlin = np.einsum("th,thd->td", w, q)          # sum_h w_h q_h
    qabs = np.einsum("th,thd->td", np.abs(w), np.abs(q))
    bound = np.zeros_like(ref)
    for t in range(T):
        b = int(np.searchsorted(cu, t, side="right") - 1)
        i = t - cu[b]
        blk = slice(cu[b] + (i // 16) * 16, min(cu[b + 1], cu[b] + (i // 16) * 16 + 16))
        ks = np.abs(k[cu[b]: t + 1])              # the row's keys (positions relative to cu[b])
        a = np.abs(k[cu[b]: t + 1] @ q[t].T) @ w[t]   # sum_h w_h |c_h|
        bq = ks @ qabs[t]
        floor = 2.0 ** -16 * np.abs(qlin[blk]).max() * ks.sum(axis=1)
        bound[t, : i + 1] = 256 * 2.0 ** -24 * (a + bq) + floor
    err = np.abs(got[fin] - ref[fin])
    assert (err <= bound[fin]).all(), (err.max(), (err / bound[fin].clip(1e-30)).max())


@pytest.mark.parametrize("hq,hkv", [(6, 2), (8, 8), (16, 1)])
def test_other_gqa_shapes(hq, hkv):
    """Head counts other than 32q/4kv: odd group size (3), plain MHA (1), one KV head (16)."""
    p = gen.make_prefill([300, 129], idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=64,
                         seed=31, q_heads=hq, kv_heads=hkv)
    pb = PrefillBatch(p)
    pb.prefill()
    o = oracle_of(p)
    sel, ref = o.rows(range(p.total_tokens))
    assert np.array_equal(pb.topk_idx.cpu().numpy(), sel)
    assert_out_close(bf16_to_float(pb.out), ref, f"sparse {hq}/{hkv}")
    dense = bf16_to_float(pb.dense(out=torch.empty_like(pb.out)))
    assert_out_close(dense, o.dense_rows(range(p.total_tokens)), f"dense {hq}/{hkv}")


def _two_valued(p, rng):
    """Indexer inputs whose scores take two values: keys are all-ones or all-zero rows and
    every query is all ones, so each row's threshold bin holds thousands of tied keys."""
    one = 0x38 if p.idx_dtype == "fp8_e4m3" else 0x3F80
    p.q_idx[:] = one
    hot = rng.random(p.k_idx.shape[0]) < 0.5
    p.k_idx[:] = 0
    p.k_idx[hot] = one


def test_topk_two_valued_scores_prefill():
    p = gen.make_prefill([9000, 2500], idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048,
                         seed=41)
    _two_valued(p, np.random.default_rng(0))
    pb = PrefillBatch(p)
    pb.index_topk()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    for t in [2047, 2048, 4100, 8999, 9000 + 2047, 9000 + 2048, 11499]:
        assert np.array_equal(idx[t], O.select_topk_row(o.scores(t), p.topk)), t


@pytest.mark.parametrize("hot_frac", [0.3, 0.5, 0.8])
def test_topk_two_valued_scores_decode(hot_frac):
    """Keys tie at two scores; a fraction ``hot_frac`` of the 20000 cached keys share the top
    score, so the threshold bin holds all of them.  At 0.3 (about 6000 tied keys) the selection's
    candidate list fits its 8192 LDS entries, and the tie group, larger than the 1024 entries
    ranked directly, goes through the second radix digit and the emit's lowest-positions-first
    rule; at 0.5 and 0.8 (about 10000 and 16000) the list would overflow and the select runs over
    the blocks' lists in HBM.  The row is never flat (the other keys score 0)."""
    d = gen.make_decode(2, 20000, 20064, 1, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=2048, seed=42)
    rng = np.random.default_rng(1)
    hot = rng.random(d.k_idx_cache.shape[:2]) < hot_frac
    d.k_idx_cache[:] = 0
    d.k_idx_cache[hot] = 0x38
    st = DecodeState(d)
    s = st.load_step(0)
    s["q_idx"][:] = 0x38
    st.step_dev["q_idx"].fill_(0x38)
    st.append()
    st.decode()
    torch.cuda.synchronize()
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    kc[:, 20000], kk[:, 20000], vv[:, 20000] = s["k_idx_new"], s["k_new"], s["v_new"]
    sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                             d.softmax_scale)
    assert np.array_equal(st.topk_idx.cpu().numpy(), sel)
    assert_out_close(bf16_to_float(st.out), ref, f"decode two-valued, hot fraction {hot_frac}")


def test_decode_unequal_cache_lengths():
    """Sequences of one batch at different lengths: 1 token, fewer than k, about k, many chunks."""
    lens = [1, 700, 2048, 2049, 13000]
    cap = 13100
    d = gen.make_decode(len(lens), max(lens), cap, 1, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=2048,
                        seed=51)
    st = DecodeState(d)
    st.lens.copy_(torch.tensor([L - 1 for L in lens], dtype=torch.int32))
    st.len_host[:] = [L - 1 for L in lens]
    s = st.load_step(0)
    st.append()
    st.decode()
    torch.cuda.synchronize()
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    for b, L in enumerate(lens):
        kc[b, L - 1], kk[b, L - 1], vv[b, L - 1] = s["k_idx_new"][b], s["k_new"][b], s["v_new"][b]
    assert list(st.len_host) == lens
    assert st.lens.cpu().tolist() == lens, "the append kernel counts the new token"
    sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                             d.softmax_scale)
    assert np.array_equal(st.topk_idx.cpu().numpy(), sel)
    assert_out_close(bf16_to_float(st.out), ref, "decode unequal lengths")
    dense = bf16_to_float(st.dense(out=torch.empty_like(st.out)))
    assert_out_close(dense, O.dense_decode(kk, vv, st.len_host, s["q"], d.softmax_scale), "dense unequal lengths")


def _decode_one_step(d, setup=None):
    """Append step 0's token and run dsa_decode; returns (indices, output, oracle indices, oracle
    output).  ``setup(s)`` may edit the step's host tensors before they are uploaded."""
    st = DecodeState(d)
    s = st.load_step(0)
    if setup is not None:
        setup(s)
        st.step_dev = {k: _dev(v, st.device) for k, v in s.items()}
    st.append()
    st.decode()
    torch.cuda.synchronize()
    n = d.ctx_len
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    kc[:, n], kk[:, n], vv[:, n] = s["k_idx_new"], s["k_new"], s["v_new"]
    sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                             d.softmax_scale)
    return st.topk_idx.cpu().numpy(), bf16_to_float(st.out), sel, ref


@pytest.mark.parametrize("k", [2048, 4096])
def test_decode_select_planted_outliers(k):
    """A few cached keys score far above the rest (more than 16 times the k-th score, beyond the
    four octaves each indexer block's histogram window spans), so the windows cannot place the
    threshold and the selection takes its exact pass over the whole score row.  With k = 4096 the
    other rows' candidate lists also exceed the LDS list more often."""
    d = gen.make_decode(3, 30000, 30016, 1, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=k, seed=57)
    rng = np.random.default_rng(58)
    codes = {v: int(c) for v, c in zip(range(-4, 5), gen._int_code_table("fp8_e4m3", 4))}
    small = np.vectorize(codes.get)(rng.integers(-1, 2, size=d.k_idx_cache.shape)).astype(np.uint8)
    d.k_idx_cache[:] = small
    qv = rng.integers(-4, 5, size=128)
    qv[qv == 0] = 1
    planted = np.vectorize(codes.get)(4 * np.sign(qv)).astype(np.uint8)
    for b in range(3):
        d.k_idx_cache[b, rng.choice(30000, 5, replace=False)] = planted

    def setup(s):
        s["q_idx"][:] = np.vectorize(codes.get)(qv).astype(np.uint8)[None, None, :]
    idx, out, sel, ref = _decode_one_step(d, setup)
    assert np.array_equal(idx, sel)
    assert_out_close(out, ref, f"decode planted outliers k={k}")


def test_kv_append_full_cache_untouched():
    """A sequence whose cache is full keeps its length and its rows; the others append."""
    cap = 40
    d = gen.make_decode(3, 30, cap, 1, idx_heads=16, idx_dim=64, idx_dtype="bf16", topk=16, seed=53)
    st = DecodeState(d)
    st.lens.copy_(torch.tensor([cap, 10, cap - 1], dtype=torch.int32))
    s = st.load_step(0)
    before = [t.clone() for t in (st.k_idx_cache, st.k_cache, st.v_cache)]
    dsa.dsa_kv_append(st.shape, st.step_dev["k_idx_new"], st.step_dev["k_new"], st.step_dev["v_new"], st.lens,
                      st.k_idx_cache, st.k_cache, st.v_cache)
    torch.cuda.synchronize()
    assert st.lens.cpu().tolist() == [cap, 11, cap]
    after = (st.k_idx_cache, st.k_cache, st.v_cache)
    news = (s["k_idx_new"], s["k_new"], s["v_new"])
    for b0, a0, new in zip(before, after, news):
        a, b = a0.cpu().numpy(), b0.cpu().numpy()
        new = new.view(a.dtype)
        assert np.array_equal(a[0], b[0]), "full cache must stay unchanged"
        assert np.array_equal(a[1, 10], new[1]) and np.array_equal(a[2, cap - 1], new[2])
        a[1, 10], a[2, cap - 1] = b[1, 10], b[2, cap - 1]
        assert np.array_equal(a, b), "only the appended rows change"


def test_empty_prefill_batch():
    p = gen.make_prefill([0, 0], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=16, seed=52)
    pb = PrefillBatch(p)
    pb.prefill()
    pb.dense(out=torch.empty_like(pb.out))
    torch.cuda.synchronize()
    assert pb.out.numel() == 0


@pytest.mark.parametrize("k", [1, 4096])
def test_topk_extreme_k(k):
    p = gen.make_prefill([5000, 33], idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=k,
                         seed=53, video=True)
    pb = PrefillBatch(p)
    pb.prefill()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    rows = np.array([0, 1, 17, 4094, 4095, 4096, 4999, 5000, 5032])
    sel, ref = o.rows(rows)
    assert np.array_equal(idx[rows], sel)
    assert_out_close(bf16_to_float(pb.out)[rows], ref, f"k={k}")


@pytest.mark.parametrize("H,dt,dI", [(16, "fp8_e4m3", 128), (32, "fp8_e4m3", 128), (32, "bf16", 128), (64, "bf16", 64)])
def test_indexer_head_shapes(H, dt, dI):
    p = gen.make_prefill([1200, 250], idx_heads=H, idx_dim=dI, idx_dtype=dt, idx_range=4 if dt == "fp8_e4m3" else 8,
                         topk=300, seed=54)
    pb = PrefillBatch(p)
    got = pb.index_scores().cpu().numpy().astype(np.float64)
    ref = O.index_score_matrix(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.idx_dtype)
    assert np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])
    pb.index_topk()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    for t in [0, 299, 300, 1199, 1200, 1449]:
        assert np.array_equal(idx[t], O.select_topk_row(o.scores(t), p.topk)), t


def test_topk_long_rows_sampled_threshold():
    """Rows of 8K..20K keys take the sampled-threshold single pass; every one of a spread of
    rows must match the oracle's select exactly."""
    p = gen.make_prefill([20000], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048,
                         seed=43, video=True)
    pb = PrefillBatch(p)
    pb.index_topk()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    rng = np.random.default_rng(3)
    rows = np.concatenate([[8190, 8191, 8192, 8193, 12345, 19999], rng.integers(8192, 20000, 14)])
    for t in rows:
        assert np.array_equal(idx[t], O.select_topk_row(o.scores(int(t)), p.topk)), int(t)


@pytest.mark.parametrize("hot_on_sampled", [False, True])
def test_topk_sample_misleads(hot_on_sampled):
    """Keys are zeroed (score exactly 0) on one class of 32-key lines: either the lines a 1-in-8
    sample of 128-byte lines reads in a row that starts on a 128-byte boundary, or the others.
    The sample then over- or under-estimates the threshold (too many candidates, or fewer than
    k); the select must still match the oracle exactly.  Rows 8193 and 9001 start 64 bytes past
    a boundary (row t of block j = t // 16 starts (t % 16)(j + 1) 64-byte units into the block),
    so their sample straddles the planted lines."""
    n = 20000
    p = gen.make_prefill([n], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048, seed=44)
    sampled = (np.arange(n) // 32) % 8 == 0
    cold = ~sampled if hot_on_sampled else sampled
    p.k_idx[cold] = 0
    pb = PrefillBatch(p)
    pb.index_topk()
    idx = pb.topk_idx.cpu().numpy()
    o = oracle_of(p)
    for t in [8191, 8192, 8193, 9000, 9001, 15000, 19999]:
        assert np.array_equal(idx[t], O.select_topk_row(o.scores(t), p.topk)), t


_IDX_CFGS = [("fp8_e4m3", 128, 16), ("fp8_e4m3", 128, 48), ("fp8_e4m3", 128, 64), ("bf16", 64, 32),
             ("bf16", 64, 64), ("bf16", 128, 16), ("bf16", 128, 32)]
_GQA = [(32, 4), (16, 1), (8, 8), (12, 4), (24, 3), (40, 8), (64, 4), (7, 7), (10, 5), (6, 1)]
_TOPKS = [1, 5, 64, 333, 1024, 2048, 3000]


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes(seed):
    """Seeded random combinations of indexer format and heads, GQA grouping (including head
    counts that do not divide the 8 XCDs, which take the general gather kernel), k and packed
    lengths (empty, one token, k - 1, k, k + 1, random): every row's selection bit-exact and
    every output within the bar."""
    rng = np.random.default_rng(1000 + seed)
    dt, dI, H = _IDX_CFGS[(5 * seed) % len(_IDX_CFGS)]  # every format, grouping and k is drawn
    hq, hkv = _GQA[seed % len(_GQA)]
    k = _TOPKS[(3 * seed) % len(_TOPKS)]
    pool = [0, 1, max(1, k - 1), k, k + 1] + [int(x) for x in rng.integers(2, 1500, 3)]
    lens = [min(int(pool[i]), 2000) for i in rng.integers(len(pool), size=int(rng.integers(1, 4)))]
    if sum(lens) == 0:
        lens.append(7)
    print(f"[random {seed}] idx {dt}/{dI}/{H} gqa {hq}/{hkv} k={k} lengths={lens}", flush=True)
    p = gen.make_prefill(lens, idx_heads=H, idx_dim=dI, idx_dtype=dt, idx_range=4 if dt == "fp8_e4m3" else 8,
                         topk=k, seed=2000 + seed, video=bool(seed % 2), q_heads=hq, kv_heads=hkv)
    pb = PrefillBatch(p)
    pb.prefill()
    idx = pb.topk_idx.cpu().numpy()
    out = bf16_to_float(pb.out)
    o = oracle_of(p)
    sel, ref = o.rows(range(p.total_tokens))
    bad = [t for t in range(p.total_tokens) if not np.array_equal(idx[t], sel[t])]
    assert not bad, f"index mismatch on rows {bad[:10]}"
    assert_out_close(out, ref, f"random {seed}")


@pytest.mark.parametrize("seed", range(8))
def test_random_decode(seed):
    """Seeded random decode steps: batch 1..6, unequal cache lengths (1 .. ~9000, some below k),
    capacity slack, GQA grouping and k drawn per seed, two consecutive steps (append + decode);
    selections bit-exact and outputs within the bar after each step."""
    rng = np.random.default_rng(3000 + seed)
    hq, hkv = _GQA[(seed + 3) % len(_GQA)]
    k = _TOPKS[(2 * seed + 1) % len(_TOPKS)]
    B = int(rng.integers(1, 7))
    lens = [int(x) for x in rng.integers(1, 9000, B)]
    lens[0] = max(1, min(lens[0], k - 1))  # one sequence with fewer than k cached keys
    cap = max(lens) + 2 + int(rng.integers(0, 40))
    print(f"[random decode {seed}] B={B} gqa {hq}/{hkv} k={k} lens={lens} cap={cap}", flush=True)
    d = gen.make_decode(B, max(lens), cap, 2, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", topk=k,
                        seed=4000 + seed, q_heads=hq, kv_heads=hkv)
    st = DecodeState(d)
    st.lens.copy_(torch.tensor(lens, dtype=torch.int32))
    st.len_host[:] = lens
    kc, kk, vv = d.k_idx_cache.copy(), d.k_cache.copy(), d.v_cache.copy()
    for step in range(2):
        s = st.load_step(step)
        st.append()
        st.decode()
        torch.cuda.synchronize()
        for b in range(B):
            n = int(st.len_host[b])
            kc[b, n - 1], kk[b, n - 1], vv[b, n - 1] = s["k_idx_new"][b], s["k_new"][b], s["v_new"][b]
        assert st.lens.cpu().tolist() == list(st.len_host)
        sel, ref = O.decode_step(kc, kk, vv, st.len_host, s["q_idx"], s["w_idx"], s["q"], d.idx_dtype, d.topk,
                                 d.softmax_scale)
        assert np.array_equal(st.topk_idx.cpu().numpy(), sel), f"step {step}"
        assert_out_close(bf16_to_float(st.out), ref, f"random decode {seed} step {step}")


def test_ordered_gather_matches_natural_order():
    """dsa_prefill gathers rows in the order of their dominant key block; dsa_sparse_attention
    on the same index sets takes them in natural order.  Rows are independent, so the outputs
    must be bit-identical.  The output starts as a NaN pattern, so a row the order skipped (a
    hole or a repeat in the permutation) cannot match."""
    p = gen.make_prefill([5000, 3000, 1, 2100], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4,
                         topk=2048, seed=61, video=True)
    pb = PrefillBatch(p)
    pb.out.fill_(-1)  # 0xffff: a bf16 NaN
    pb.prefill()
    ordered = pb.out.clone()
    pb.out.zero_()
    pb.sparse_attention()
    torch.cuda.synchronize()
    assert torch.equal(pb.out, ordered)


def test_many_sequences_keep_natural_order():
    """17000 sequences of one or two tokens: the gather's row order would need a key per
    sequence and 1024-key block, more than its 16384-key limit, so the rows keep their natural
    order.  Every selection bit-exact and every output within the bar.  V is halved (exact in
    bf16): an output here is a mean of at most two V rows, and at magnitudes of 4 and above the
    bf16 output grid alone (half-ulp 2^-6) would exceed the bar's 1e-2."""
    rng = np.random.default_rng(77)
    lens = [int(x) for x in rng.integers(1, 3, 17000)]
    p = gen.make_prefill(lens, idx_heads=16, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=4, seed=78)
    v = (p.v.astype(np.uint32) << 16).view(np.float32) * np.float32(0.5)
    p.v = (v.view(np.uint32) >> 16).astype(np.uint16)
    print(f"[many sequences] T={p.total_tokens}", flush=True)
    pb = PrefillBatch(p)
    pb.prefill()
    idx = pb.topk_idx.cpu().numpy()
    out = bf16_to_float(pb.out)
    o = oracle_of(p)
    sel, ref = o.rows(range(p.total_tokens))
    bad = [t for t in range(p.total_tokens) if not np.array_equal(idx[t], sel[t])]
    assert not bad, f"index mismatch on rows {bad[:10]}"
    assert_out_close(out, ref, "many sequences")

