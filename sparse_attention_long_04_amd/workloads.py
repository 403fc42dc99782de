"""Named synthetic workloads of the DSA hot path, with their shapes and seeds.

The shapes follow the Keye-VL-2.0 summary page (gsyq.cn): top-2048 key positions per query
token from one MQA-shared Lightning Indexer (section 一), GQA attention in the base LLM
(section 一), 128K-token prefill/decode as the quoted operating point (section 一) and 256K
as the longest context (section 一, section 四).  Indexer sizes, dtypes and the tiny case
are this framework's choices, stated here once.
"""
from __future__ import annotations

from . import inputs

TINY = "prefill_2k_tiny"
P32K = "prefill_32k"
P128K = "prefill_128k_video"
DECODE = "decode_16x128k_video"
VARLEN = "varlen_256k_video"
TOPK = "topk_2048x131072"
P128K_CORR = "prefill_128k_video_corr"

WORKLOADS = {
    TINY: dict(kind="prefill", lengths=[2048], idx_heads=16, idx_dim=64, idx_dtype="bf16",
               idx_range=8, topk=256, video=False, seed=1000),
    P32K: dict(kind="prefill", lengths=[32768], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3",
               idx_range=4, topk=2048, video=False, seed=1001),
    P128K: dict(kind="prefill", lengths=[131072], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3",
                idx_range=4, topk=2048, video=True, seed=1002),
    DECODE: dict(kind="decode", batch=16, ctx_len=131072, capacity=131136, steps=64, idx_heads=64,
                 idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048, video=True, seed=1003),
    VARLEN: dict(kind="prefill", lengths=None, n_seqs=6, total=262144, idx_heads=64, idx_dim=128,
                 idx_dtype="fp8_e4m3", idx_range=4, topk=2048, video=True, seed=1004),
    # the 128K video prefill with slowly drifting indexer queries (adjacent-query dedup)
    P128K_CORR: dict(kind="prefill", lengths=[131072], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3",
                     idx_range=4, topk=2048, video=True, seed=1006, query_corr=0.95),
    # standalone top-k: 2048 rows x 131072 N(0,1) fp32 scores, 1% masked with -inf, k = 2048
    TOPK: dict(kind="topk", rows=2048, n=131072, topk=2048, masked=0.01, seed=1005),
}


def lengths_of(name: str):
    w = WORKLOADS[name]
    if w.get("lengths") is not None:
        return list(w["lengths"])
    return inputs.varlen_lengths(w["seed"], n_seqs=w["n_seqs"], total=w["total"])


def make(name: str, lengths=None):
    """Build the inputs of a named workload (``lengths`` overrides the sequence lengths)."""
    w = WORKLOADS[name]
    if w["kind"] == "topk":
        return inputs.make_topk_scores(w["rows"], w["n"], seed=w["seed"], masked=w["masked"])
    if w["kind"] == "decode":
        return inputs.make_decode(w["batch"], w["ctx_len"], w["capacity"], w["steps"],
                                  idx_heads=w["idx_heads"], idx_dim=w["idx_dim"],
                                  idx_dtype=w["idx_dtype"], topk=w["topk"], seed=w["seed"],
                                  video=w["video"], idx_range=w["idx_range"])
    return inputs.make_prefill(lengths if lengths is not None else lengths_of(name),
                               idx_heads=w["idx_heads"], idx_dim=w["idx_dim"],
                               idx_dtype=w["idx_dtype"], idx_range=w["idx_range"],
                               topk=w["topk"], seed=w["seed"], video=w["video"],
                               query_corr=w.get("query_corr"))
