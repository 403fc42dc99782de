"""CPU tests of the C-ABI library: it loads, exports every declared symbol, and rejects bad
arguments on the host before touching the GPU.  No kernel is launched here."""
import ctypes
import os
import re

import numpy as np
import pytest

from sparse_attention_long_04_amd import dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dsa.lib_path()), reason="libdsa.so not built")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", src, flags=re.M)
    return sorted(set(n for n in names if n not in ("if",)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ["dsa_index_topk", "dsa_prefill", "dsa_decode", "dense_causal_attention", "dsa_sparse_attention",
              "dense_decode_attention", "dsa_kv_append", "dsa_index_scores", "dsa_prefill_workspace_size",
              "dsa_decode_workspace_size", "dsa_status_string", "dsa_last_hip_error", "dsa_topk",
              "dsa_prefill_dedup", "dsa_sparse_attention_dedup", "dsa_dedup_workspace_size",
              "dsa_indexer_kl", "dsa_indexer_kl_workspace_size"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(dsa.lib_path())
    for n in declared_functions():
        assert hasattr(L, n), n
    # and the binding wraps each of them
    assert set(declared_functions()) <= set(dsa.EXPORTS)


def test_status_strings():
    assert dsa.dsa_status_string(0) == "ok"
    assert "workspace" in dsa.dsa_status_string(3)
    assert dsa.dsa_status_string(99) == "unknown status"


FAKE = 1 << 20  # a non-null, 16-byte aligned "device pointer" that is never dereferenced
WS = (FAKE, 1 << 62)


def shape(**kw):
    base = dict(topk=2048, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", q_heads=32, kv_heads=4,
                head_dim=128, softmax_scale=128 ** -0.5)
    base.update(kw)
    T = base.pop("T", 4096)
    ms = base.pop("max_seqlen", 4096)
    ns = base.pop("num_seqs", 1)
    return dsa.prefill_shape(FAKE, T, ms, num_seqs=ns, **base)


@pytest.mark.parametrize("kw,code", [
    (dict(topk=0), 1), (dict(topk=5000), 1), (dict(kv_heads=3), 1), (dict(head_dim=64), 2),
    (dict(idx_heads=24), 2), (dict(idx_heads=128), 2), (dict(idx_dim=64), 2), (dict(idx_dtype=7), 1),
    (dict(softmax_scale=0.0), 1), (dict(softmax_scale=float("nan")), 1), (dict(kv_heads=1), 2),
    (dict(max_seqlen=5000), 1), (dict(num_seqs=0), 1), (dict(T=-1), 1),
])
def test_prefill_rejects_bad_shapes_before_launch(kw, code):
    s = shape(**kw)
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_prefill(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, stream=0)
    assert ei.value.status == code


def test_kv_spans_past_32bit_offsets_are_refused_before_launch():
    """The attention kernels address K/V rows with 32-bit byte offsets from a sequence's (or a
    cache's) first row.  A batch of 4.2M tokens with 4 KV heads of 128 dims (4.3 GB of K) is
    refused as unsupported before any launch by the calls that run attention, while the
    workspace query (shared with the index-only calls) still answers; a decode cache of 5M rows
    is refused the same way."""
    big = shape(T=4_200_000, max_seqlen=4096, num_seqs=1100)
    assert dsa.dsa_prefill_workspace_size(big) > 0
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_prefill(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, stream=0)
    assert ei.value.status == 2
    d = dsa.decode_shape(FAKE, 5_000_000, 1000, batch=2, topk=64, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3")
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode(d, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, WS, stream=0)
    assert ei.value.status == 2


def test_prefill_rejects_null_and_misaligned_pointers():
    s = shape()
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_prefill(s, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, WS, stream=0)
    assert ei.value.status == 1
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_index_topk(s, FAKE + 4, FAKE, FAKE, FAKE, WS, stream=0)
    assert ei.value.status == 1


def test_workspace_too_small_is_reported():
    s = shape()
    L = dsa.lib()
    need = dsa.dsa_prefill_workspace_size(s)
    rc = L.dsa_prefill(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, need - 1, 0)
    assert rc == 3


def test_workspace_is_bounded_by_the_chunk_buffer():
    """The indexer scores 512 blocks of 16 rows at a time (256 long and 256 short ones) into a
    reusable buffer of 512 x 16 x max_seqlen floats; the prefill workspace is that buffer plus
    O(T k) of indices and per-row state -- a few GiB at 128K and 256K tokens, not the score
    triangle."""
    for T in (131072, 262144):
        s = shape(T=T, max_seqlen=T)
        n = dsa.dsa_prefill_workspace_size(s, np.array([0, T]))
        chunk = 512 * 16 * T * 4
        idx = T * 2048 * 4
        dense_v = T * 4 * 128 * 2
        assert chunk + idx + dense_v <= n < chunk + idx + dense_v + T * 64 + (1 << 22)
        nb = T // 16
        assert n < 128 * nb * (nb + 1) * 4 / 4          # well under the whole triangle
    # 8193 blocks bound the 16-row schedule of one 131072-token sequence: 17 chunks of 512
    assert dsa.dsa_prefill_timing_events(shape(T=131072, max_seqlen=131072)) == 3 + 2 * 17


def test_varlen_workspace_bound_holds_for_any_split():
    rng = np.random.default_rng(0)
    for _ in range(50):
        lens = rng.integers(0, 3000, size=int(rng.integers(1, 8)))
        T = int(lens.sum())
        if T == 0:
            continue
        cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
        s = shape(T=T, max_seqlen=int(lens.max()), num_seqs=len(lens), topk=64)
        bound = dsa.dsa_prefill_workspace_size(s)
        exact = dsa.dsa_prefill_workspace_size(s, cu)
        assert bound >= 4 * 256 * 16 * ((int(lens.max()) + 15) // 16 * 16)
        assert exact == bound


def test_decode_rejects_bad_shapes():
    s = dsa.decode_shape(FAKE, 1000, 2000, batch=2, topk=64, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3")
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode_workspace_size(s)
    assert ei.value.status == 1
    s = dsa.decode_shape(FAKE, 1000, 900, batch=2, topk=64, idx_heads=64, idx_dim=64, idx_dtype="bf16")
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode(s, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, WS, stream=0)
    assert ei.value.status == 2


def test_decode_cache_length_limit():
    """Caches up to 2^20 rows are sized; one row more is refused as unsupported."""
    lim = 1 << 20
    s = dsa.decode_shape(FAKE, lim + 1, lim, batch=2, topk=2048, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3")
    assert dsa.dsa_decode_workspace_size(s) > 2 * (lim + 1) * 4
    s = dsa.decode_shape(FAKE, lim + 1, lim + 1, batch=2, topk=2048, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3")
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode_workspace_size(s)
    assert ei.value.status == 2


def test_schedule_rank_is_a_longest_first_permutation():
    """Host model of the device work schedule: ranks of (sequence, block) pairs ordered by
    block index descending then sequence ascending form a permutation."""
    rng = np.random.default_rng(1)
    for _ in range(100):
        nbs = rng.integers(0, 20, size=int(rng.integers(1, 6)))
        pairs = [(b, j) for b, nb in enumerate(nbs) for j in range(nb)]
        ranks = []
        for b, j in pairs:
            r = sum(max(0, int(nb) - j - 1) for nb in nbs) + sum(1 for s in range(b) if nbs[s] > j)
            ranks.append(r)
        assert sorted(ranks) == list(range(len(pairs)))
        order = [p for _, p in sorted(zip(ranks, pairs))]
        assert order == sorted(pairs, key=lambda p: (-p[1], p[0]))


def test_empty_prefill_batch_is_a_noop_with_null_pointers():
    s = shape(T=0, max_seqlen=0)
    for fn in (lambda: dsa.dsa_prefill(s, None, None, None, None, None, None, None, None, None, stream=0),
               lambda: dsa.dsa_index_topk(s, None, None, None, None, None, stream=0),
               lambda: dsa.dsa_sparse_attention(s, None, None, None, None, None, stream=0),
               lambda: dsa.dense_causal_attention(s, None, None, None, None, None, stream=0)):
        fn()


@pytest.mark.parametrize("args,code", [
    (dict(rows=4, n=100, ld=100, k=0), 1),          # k < 1
    (dict(rows=-1, n=100, ld=100, k=8), 1),         # negative rows
    (dict(rows=4, n=-3, ld=100, k=8), 1),           # negative n
    (dict(rows=4, n=100, ld=99, k=8), 1),           # row stride shorter than the row
    (dict(rows=4, n=100, ld=100, k=8, scores=None), 1),
    (dict(rows=4, n=100, ld=100, k=8, out=None), 1),
    (dict(rows=1 << 31, n=100, ld=100, k=8), 1),    # more rows than one launch takes
])
def test_topk_rejects_bad_arguments_before_launch(args, code):
    a = dict(scores=FAKE, row_lens=None, out=FAKE)
    a.update(args)
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_topk(a["scores"], a["rows"], a["n"], a["ld"], a["row_lens"], a["k"], a["out"], stream=0)
    assert ei.value.status == code


def test_topk_zero_rows_is_a_noop_with_null_pointers():
    dsa.dsa_topk(None, 0, 100, 100, None, 16, None, stream=0)


def test_dedup_workspace_layout_and_unsupported_groups():
    s = shape(T=4096, max_seqlen=4096, topk=2048)
    n = dsa.dsa_dedup_workspace_size(s)
    nb16 = 4096 // 16 + 1
    unions = nb16 * 16 * 2048 * 6          # key positions (int32) and row masks (uint16) per block
    vh = 4096 * s.kv_heads * 128 * 2       # the fp16 copy of V the masked products read
    assert n >= unions + vh
    assert n < unions + vh + (1 << 20)
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_dedup_workspace_size(shape(q_heads=24, kv_heads=4))   # G = 6
    assert ei.value.status == 2
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_sparse_attention_dedup(s, FAKE, FAKE, FAKE, FAKE, FAKE, (FAKE, n - 1), stream=0)
    assert ei.value.status == 3
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_sparse_attention_dedup(s, FAKE, FAKE, FAKE, None, FAKE, (FAKE, n), stream=0)
    assert ei.value.status == 1


def test_indexer_kl_rejects_unsupported_shapes():
    ok = shape(T=4096, max_seqlen=4096)
    n = dsa.dsa_indexer_kl_workspace_size(ok)
    assert n > 4096 * 32 * 4
    for kw in (dict(idx_dtype="bf16", idx_dim=64), dict(idx_heads=48), dict(kv_heads=8, q_heads=32)):
        with pytest.raises(dsa.DSAError) as ei:
            dsa.dsa_indexer_kl_workspace_size(shape(T=4096, max_seqlen=4096, **kw))
        assert ei.value.status == 2, kw
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_indexer_kl(ok, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, (FAKE, n - 1), stream=0)
    assert ei.value.status == 3


def test_decode_noalloc_rejects_shapes_beyond_its_scratch_before_launch():
    """The allocation-free decode refuses, on the host, any shape whose workspace would not fit
    its static scratch; 16 x 131136-row caches with k = 2048 fit."""
    assert dsa.dsa_status_string(5) == "shape needs more than the static decode scratch"
    ok = dsa.decode_shape(FAKE, 131136, 131136, batch=16, topk=2048, idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3")
    assert dsa.dsa_decode_workspace_size(ok) <= 64 << 20
    big = dsa.decode_shape(FAKE, 1 << 20, 1 << 20, batch=16, topk=2048, idx_heads=64, idx_dim=128,
                           idx_dtype="fp8_e4m3")
    assert dsa.dsa_decode_workspace_size(big) > 64 << 20
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode_noalloc(big, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == 5
    bad = dsa.decode_shape(FAKE, 1000, 900, batch=2, topk=64, idx_heads=64, idx_dim=64, idx_dtype="bf16")
    with pytest.raises(dsa.DSAError) as ei:
        dsa.dsa_decode_noalloc(bad, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, stream=0)
    assert ei.value.status == 2
