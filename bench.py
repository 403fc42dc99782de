#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.  Prints ONE JSON line.

A step is one ``dsa_prefill`` (Lightning Indexer -> top-k -> sparse GQA attention) over the
128K-token video-like prefill workload (131072 tokens = 128 frames x (16 timestamp-text +
1008 vision tokens), k = 2048, indexer 64 heads x 128 fp8, GQA 32q/4kv, d = 128 bf16), with
all inputs resident in HBM.  ``value`` is prefill tokens/s.  The same line also reports, from
the same run: per-stage times with HIP events, the indexer's roofline fraction, the dense
causal attention time on the same inputs (DSA/dense ratio), the decode step time for 16
sequences x 128K cached tokens over 64 steps (with the dense-decode ratio), the packed 256K
varlen prefill throughput, and the CPU oracle timed on a bounded row sample.

    python bench.py [--gpus 1] [--steps 3] [--warmup 1] [--quick]
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "DSA prefill tokens/s & decode µs/step at 128K ctx; % MFMA/HBM peak; ratio vs dense"
PEAK_FP8 = 5.0e15      # MI355X dense fp8 MFMA, FLOP/s
PEAK_BF16 = 2.5e15     # MI355X dense bf16 MFMA, FLOP/s
PEAK_HBM = 8.0e12      # MI355X HBM3E, B/s


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def pairs_of(lengths):
    return sum(L * (L + 1) // 2 for L in lengths)


def selected_of(lengths, k):
    """sum over rows of min(k, i+1): the selected (query, key) pairs."""
    return sum(L * (L + 1) // 2 if L <= k else k * (k + 1) // 2 + (L - k) * k for L in lengths)


def ms_between(a, b):
    return a.elapsed_time(b)


def roof(bound, achieved, peak, unit, traffic_bytes, work, work_unit, **extra):
    """Roofline entry: achieved/peak in TFLOP/s or GB/s from algorithmic work per launch."""
    scale = 1e12 if unit == "TFLOP/s" else 1e9
    return {"bound": bound, "achieved": round(achieved / scale, 1), "peak": round(peak / scale, 1), "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": traffic_bytes, "work_per_launch": work,
            "work_unit": work_unit, **extra}


def read_traffic():
    """HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated) from the committed profile
    summary; a kernel whose sources (its own, and for the gather the row order that shapes its
    traffic) changed since the counters were taken gets no entry."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "prefill_128k_video_traffic.md")
    out = {}
    if not os.path.exists(path):
        return out
    for line in open(path):
        if not line.startswith("traffic ") or "fetch_bytes=" not in line:
            continue
        f = dict(kv.split("=", 1) for kv in line.split()[2:])
        # source=a.hip,b.hip sha256=h1,h2: every listed source must be unchanged
        current = True
        for name, digest in zip(f["source"].split(","), f["sha256"].split(",")):
            src = os.path.join(ROOT, "sparse_attention_long_04_amd", "csrc", name)
            if not os.path.exists(src) or hashlib.sha256(open(src, "rb").read()).hexdigest()[:16] != digest:
                current = False
        if current:
            out[line.split()[1]] = int(f["fetch_bytes"]) + int(f["write_bytes"])
    return out


def bench_prefill(name, steps, warmup, with_dense=True):
    import torch
    from sparse_attention_long_04_amd import workloads
    from sparse_attention_long_04_amd.runtime import PrefillBatch, timing_events

    t0 = time.time()
    p = workloads.make(name)
    log(f"{name}: inputs generated in {time.time() - t0:.1f}s, T={p.total_tokens}, lengths={list(p.lengths)}")
    pb = PrefillBatch(p)
    torch.cuda.synchronize()
    log(f"{name}: resident in HBM (workspace {pb.ws.numel() / 2**30:.1f} GiB)")
    st = torch.cuda.current_stream()
    nev = pb.timing_events()
    ev = [timing_events(nev) for _ in range(steps)]
    for _ in range(warmup):
        pb.prefill()
    torch.cuda.synchronize()
    start, end = timing_events(2)
    start.record(st)
    for s in range(steps):
        pb.prefill_timed(ev[s])
    end.record(st)
    torch.cuda.synchronize()
    total_ms = ms_between(start, end)
    # per-stage: [0] after the schedule; chunk c: [1 + 2c] after its indexer, [2 + 2c] after its
    # top-k; [nev - 2] after the row order, [nev - 1] after the attention
    nch = (nev - 3) // 2
    idx_ms = [sum(ms_between(e[2 * c], e[2 * c + 1]) for c in range(nch)) for e in ev]
    topk_ms = [sum(ms_between(e[2 * c + 1], e[2 * c + 2]) for c in range(nch)) + ms_between(e[nev - 3], e[nev - 2])
               for e in ev]
    attn_ms = [ms_between(e[nev - 2], e[nev - 1]) for e in ev]
    log(f"{name}: {total_ms / steps:.2f} ms/step  indexer {np.mean(idx_ms):.2f}  topk {np.mean(topk_ms):.2f}  "
        f"attention {np.mean(attn_ms):.2f}")
    res = dict(p=p, T=p.total_tokens, lengths=[int(x) for x in p.lengths], ms=total_ms / steps,
               indexer_ms=float(np.mean(idx_ms)), topk_ms=float(np.mean(topk_ms)), attn_ms=float(np.mean(attn_ms)))
    if with_dense:
        out = torch.empty_like(pb.out)
        pb.dense(out=out)
        torch.cuda.synchronize()
        a, b = timing_events(2)
        a.record(st)
        for _ in range(steps):
            pb.dense(out=out)
        b.record(st)
        torch.cuda.synchronize()
        res["dense_ms"] = ms_between(a, b) / steps
        log(f"{name}: dense causal {res['dense_ms']:.2f} ms")
    del pb
    torch.cuda.empty_cache()
    return res


def bench_dense(name, steps):
    """dense_causal_attention alone on a prefill workload's inputs (profiling aid)."""
    import torch
    from sparse_attention_long_04_amd import workloads
    from sparse_attention_long_04_amd.runtime import PrefillBatch, timing_events

    p = workloads.make(name)
    pb = PrefillBatch(p)
    out = torch.empty_like(pb.out)
    torch.cuda.synchronize()
    a, b = timing_events(2)
    a.record()
    for _ in range(steps):
        pb.dense(out=out)
    b.record()
    torch.cuda.synchronize()
    ms = ms_between(a, b) / steps
    log(f"{name}: dense causal {ms:.2f} ms")
    return dict(workload=name, dense_ms=ms)


def bench_decode(steps_total=64, stage_reps=16):
    """The decode workload's steps back to back: each step appends every sequence's new token
    (row and length, dsa_kv_append) and then runs dsa_decode; events around each call time
    dsa_decode alone (the step time reported) and the append separately.  The per-stage
    split comes from a second pass of dsa_decode_timed at the final cache length (no append);
    its events between stages add small gaps, so stage times sum to a little more than a step."""
    import torch
    from sparse_attention_long_04_amd import workloads
    from sparse_attention_long_04_amd.runtime import DecodeState, timing_events

    t0 = time.time()
    d = workloads.make(workloads.DECODE)
    log(f"decode: caches generated in {time.time() - t0:.1f}s")
    st_ = DecodeState(d)
    steps = []
    for i in range(steps_total):
        st_.load_step(i)
        steps.append(st_.step_dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [timing_events(3) for _ in range(steps_total)]
    for i in range(steps_total):
        st_.step_dev = steps[i]
        evs[i][0].record(stream)
        st_.append()
        evs[i][1].record(stream)
        st_.decode()
        evs[i][2].record(stream)
    torch.cuda.synchronize()
    us = np.array([ms_between(e[1], e[2]) * 1e3 for e in evs])          # dsa_decode alone
    app_us = np.array([ms_between(e[0], e[1]) * 1e3 for e in evs])      # dsa_kv_append
    both_us = np.array([ms_between(e[0], e[2]) * 1e3 for e in evs])
    sev = [timing_events(4) for _ in range(stage_reps)]
    for e in sev:
        e[0].record(stream)
        st_.decode_timed(e[1:])
    torch.cuda.synchronize()
    idx_us = np.array([ms_between(e[0], e[1]) * 1e3 for e in sev])
    topk_us = np.array([ms_between(e[1], e[2]) * 1e3 for e in sev])
    attn_us = np.array([ms_between(e[2], e[3]) * 1e3 for e in sev])
    dense_ms = []
    dout = torch.empty_like(st_.out)
    for _ in range(3):
        a, b = timing_events(2)
        a.record(stream)
        st_.dense(out=dout)
        b.record(stream)
        torch.cuda.synchronize()
        dense_ms.append(ms_between(a, b))
    # the first step also pays one-time costs; report mean over steps 1..63 and p50 over all
    res = dict(us_mean=float(us[1:].mean()), us_p50=float(np.median(us)), append_us=float(app_us[1:].mean()),
               step_with_append_us=float(both_us[1:].mean()), indexer_us=float(idx_us[1:].mean()),
               topk_us=float(topk_us[1:].mean()), attn_us=float(attn_us[1:].mean()),
               dense_us=float(np.mean(dense_ms[1:]) * 1e3), batch=d.batch, ctx=d.ctx_len)
    n_mean = d.ctx_len + (steps_total + 1) / 2
    idx_bytes = d.batch * n_mean * d.idx_dim * (1 if d.idx_dtype == "fp8_e4m3" else 2)
    bytes_step = idx_bytes + d.batch * (d.topk * d.kv_heads * d.head_dim * 2 * 2 + n_mean * 4 * 2)
    res["hbm_gbs"] = bytes_step / (res["us_mean"] * 1e-6) / 1e9
    n_end = d.ctx_len + steps_total
    res["indexer_gbs"] = d.batch * n_end * d.idx_dim * (1 if d.idx_dtype == "fp8_e4m3" else 2) / (
        res["indexer_us"] * 1e-6) / 1e9
    res["attn_gbs"] = d.batch * d.topk * d.kv_heads * d.head_dim * 2 * 2 / (res["attn_us"] * 1e-6) / 1e9
    log(f"decode: dsa_decode {res['us_mean']:.1f} us/step (p50 {res['us_p50']:.1f}), append {res['append_us']:.1f}, "
        f"both {res['step_with_append_us']:.1f}; stages indexer {res['indexer_us']:.1f} "
        f"topk {res['topk_us']:.1f} attn {res['attn_us']:.1f}; dense {res['dense_us']:.1f} us")
    del st_
    torch.cuda.empty_cache()
    return res


def bench_dedup(steps=3):
    """Adjacent-query dedup on the correlated 128K workload (indexer queries drifting along the
    sequence): dsa_prefill (gather path) and dsa_prefill_dedup on the same inputs, per-stage
    HIP-event times, and the masked MFMA work the dedup kernel executes."""
    import torch
    from sparse_attention_long_04_amd import workloads
    from sparse_attention_long_04_amd.runtime import PrefillBatch, timing_events

    name = workloads.P128K_CORR
    p = workloads.make(name)
    pb = PrefillBatch(p)
    st = torch.cuda.current_stream()
    res = {}
    nev = pb.timing_events()
    for mode in ("gather", "dedup"):
        runs = []
        for it in range(steps + 1):
            ev = timing_events(nev)
            a, = timing_events(1)
            a.record(st)
            if mode == "gather":
                pb.prefill_timed(ev)
            else:
                pb.prefill_dedup(events=ev)
            torch.cuda.synchronize()
            runs.append([ms_between(a, ev[nev - 1]), ms_between(ev[nev - 2], ev[nev - 1])])
        r = np.array(runs[1:]).mean(0)
        res[mode] = dict(ms=float(r[0]), attention_ms=float(r[1]))
    pb.sparse_attention_dedup(out=torch.empty_like(pb.out))
    torch.cuda.synchronize()
    _, cnt, _, _ = pb.dedup_unions()
    u = cnt.double()
    Hq, Hkv, d = p.q.shape[1], p.k.shape[1], p.q.shape[2]
    # executed: every 64-key tile of a union against the block's 16 rows x Hq heads
    executed = float((torch.ceil(u / 64) * 64).sum()) * 16 * Hq * d * 4
    useful = selected_of(p.lengths, p.topk) * Hq * d * 4
    out = dict(workload=name, T=int(p.total_tokens), gather=res["gather"], dedup=res["dedup"],
               union_mean=float(u.mean()), union_per_row=float(u.sum()) / p.total_tokens,
               executed_flop=float(executed), useful_flop=float(useful))
    log(f"dedup {name}: gather {res['gather']['ms']:.2f} ms (attention {res['gather']['attention_ms']:.2f}); "
        f"dedup {res['dedup']['ms']:.2f} ms (attention {res['dedup']['attention_ms']:.2f}); mean union of 16 rows "
        f"{out['union_mean']:.0f}")
    del pb
    torch.cuda.empty_cache()
    return out


def bench_indexer_kl(reps=3):
    """The indexer's dense warm-up objective (dsa_indexer_kl: KL value per token and gradients for
    q_I, k_I, w) on one 32768-token sequence with the 32K prefill shapes (indexer 64 x 128 e4m3,
    GQA 32q/4kv d128), timed with HIP events over ``reps`` calls."""
    import torch
    from sparse_attention_long_04_amd import dsa
    from sparse_attention_long_04_amd import inputs as gen
    from sparse_attention_long_04_amd.runtime import PrefillBatch, timing_events

    L = 32768
    p = gen.make_prefill([L], idx_heads=64, idx_dim=128, idx_dtype="fp8_e4m3", idx_range=4, topk=2048, seed=1007,
                         video=True)
    pb = PrefillBatch(p, workspace=False)
    H = 64
    ws = torch.empty(dsa.dsa_indexer_kl_workspace_size(pb.shape), dtype=torch.uint8, device="cuda")
    kl = torch.empty(L, dtype=torch.float32, device="cuda")
    dq = torch.empty((L, H, 128), dtype=torch.float32, device="cuda")
    dk = torch.empty((L, 128), dtype=torch.float32, device="cuda")
    dw = torch.empty((L, H), dtype=torch.float32, device="cuda")
    args = (pb.shape, pb.q_idx, pb.k_idx, pb.w_idx, pb.q, pb.k, kl, dq, dk, dw, ws)
    dsa.dsa_indexer_kl(*args)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a, b = timing_events(2)
    a.record(st)
    for _ in range(reps):
        dsa.dsa_indexer_kl(*args)
    b.record(st)
    torch.cuda.synchronize()
    ms = ms_between(a, b) / reps
    pairs = pairs_of([L])
    # MFMA work executed per call: two bf16 passes of QK^T over all query heads (log-sum-exp,
    # target), the fp8 indexer scores, and per gradient kernel an fp8 recompute of the indexer
    # products plus the G contraction twice (bf16 hi + lo)
    bf16_flop = 2 * 32 * 128 * 2 * pairs + 2 * (H * 128 * 2 * pairs * 2)
    fp8_flop = 3 * H * 128 * 2 * pairs
    log(f"indexer KL 32K: {ms:.2f} ms per call (forward + gradients)")
    del pb, ws, dq
    torch.cuda.empty_cache()
    return dict(ms=ms, tokens=L, bf16_flop=float(bf16_flop), fp8_flop=float(fp8_flop))


def bench_sparse_bwd(reps=3):
    """Sparse attention backward on one 32768-token sequence with k = 2048 (the 32K prefill
    shapes): dsa_sparse_attention_bwd given the forward's out and lse, timed with HIP events."""
    import torch
    from sparse_attention_long_04_amd import dsa, workloads
    from sparse_attention_long_04_amd import inputs as gen
    from sparse_attention_long_04_amd.runtime import PrefillBatch, timing_events

    p = workloads.make(workloads.P32K)
    pb = PrefillBatch(p)
    pb.index_topk()
    T, Hq, d = p.q.shape
    Hkv = p.k.shape[1]
    out = torch.empty_like(pb.out)
    lse = torch.empty((T, Hq), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attention_fwd_lse(pb.shape, pb.q, pb.k, pb.v, pb.topk_idx, out, lse)
    dout = torch.from_numpy(gen.make_grad_bf16((T, Hq, d), 1008).view(np.int16)).cuda()
    pb.ws = None
    torch.cuda.empty_cache()
    ws = torch.empty(dsa.dsa_sparse_attention_bwd_workspace_size(pb.shape), dtype=torch.uint8, device="cuda")
    dq = torch.empty((T, Hq, d), dtype=torch.float32, device="cuda")
    dk = torch.empty((T, Hkv, d), dtype=torch.float32, device="cuda")
    dv = torch.empty((T, Hkv, d), dtype=torch.float32, device="cuda")
    args = (pb.shape, pb.q, pb.k, pb.v, pb.topk_idx, out, lse, dout, dq, dk, dv, ws)
    dsa.dsa_sparse_attention_bwd(*args)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    a, b = timing_events(2)
    a.record(st)
    for _ in range(reps):
        dsa.dsa_sparse_attention_bwd(*args)
    b.record(st)
    torch.cuda.synchronize()
    ms = ms_between(a, b) / reps
    sel = selected_of([T], p.topk)
    useful = sel * Hq * d * 2 * 4  # dS (via dP), and the dq, dk, dv products: 4 x 2 flop per (pair, head, dim)
    log(f"sparse attention backward 32K: {ms:.2f} ms per call")
    del pb, ws, dq, dk, dv
    torch.cuda.empty_cache()
    return dict(ms=ms, tokens=T, useful_flop=float(useful))


def bench_topk_general(reps=5):
    """The standalone top-k (dsa_topk) on its workload: 2048 rows x 131072 fp32 scores, k = 2048,
    timed over ``reps`` back-to-back launches with HIP events.  torch.topk on the same scores is
    timed alongside as context only (it returns value-sorted positions with no tie rule)."""
    import torch
    from sparse_attention_long_04_amd import dsa, workloads
    from sparse_attention_long_04_amd.runtime import timing_events

    w = workloads.WORKLOADS[workloads.TOPK]
    rows, n, k = w["rows"], w["n"], w["topk"]
    t0 = time.time()
    dev = torch.from_numpy(workloads.make(workloads.TOPK)).cuda()
    log(f"topk: {rows} x {n} scores generated and uploaded in {time.time() - t0:.1f}s")
    out = torch.empty((rows, k), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()
    dsa.dsa_topk(dev, rows, n, n, None, k, out)
    torch.cuda.synchronize()
    a, b = timing_events(2)
    a.record(stream)
    for _ in range(reps):
        dsa.dsa_topk(dev, rows, n, n, None, k, out)
    b.record(stream)
    torch.cuda.synchronize()
    ms = ms_between(a, b) / reps
    torch.topk(dev, k, dim=1)
    torch.cuda.synchronize()
    a, b = timing_events(2)
    a.record(stream)
    for _ in range(reps):
        torch.topk(dev, k, dim=1)
    b.record(stream)
    torch.cuda.synchronize()
    tms = ms_between(a, b) / reps
    work = rows * n * 4 + rows * k * 4
    log(f"topk: {ms:.3f} ms per launch ({work / (ms * 1e-3) / 1e9:.0f} GB/s algorithmic); torch.topk {tms:.3f} ms")
    del dev, out
    torch.cuda.empty_cache()
    return dict(ms=ms, torch_topk_ms=tms, work=work, rows=rows, n=n, k=k)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:  # pragma: no cover
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(p, gpu_tokens_per_s, seconds=20.0, max_rows=4000, seed=0):
    """The oracle (as is) on a uniform random sample of the workload's rows, for a bounded time,
    each of its steps timed on its own: indexer scores, top-k select, sparse attention (these
    three are the oracle's prefill row), and dense causal attention of the same row."""
    from oracle import dsa_oracle as O
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = os.cpu_count() or 1
    o = O.Prefill(p.cu_seqlens, p.q_idx, p.k_idx, p.w_idx, p.q, p.k, p.v, p.idx_dtype, p.topk, p.softmax_scale)
    rng = np.random.default_rng(seed)
    rows = rng.integers(0, p.total_tokens, size=max_rows)
    o.row(int(rows[0]))  # decode the sequence's keys outside the timed part
    st = dict(scores=0.0, select=0.0, sparse_attention=0.0, dense=0.0)
    clock = time.perf_counter
    t0 = clock()
    n = 0
    for t in rows:
        t = int(t)
        b, _ = o.locate(t)
        _, K, V = o._seq(b)
        a = clock()
        sc = o.scores(t)
        b_ = clock()
        sel = O.select_topk_row(sc, o.topk)
        c = clock()
        s = sel[sel >= 0]
        O.attention_row(O.decode_bf16(o.q[t]), K[s], V[s], o.scale)
        d = clock()
        o.dense_row(t)
        e = clock()
        st["scores"] += b_ - a
        st["select"] += c - b_
        st["sparse_attention"] += d - c
        st["dense"] += e - d
        n += 1
        if clock() - t0 > seconds:
            break
    dsa_s = st["scores"] + st["select"] + st["sparse_attention"]
    value = n / dsa_s
    return dict(value=value, unit="tokens/s", cores=int(cores), kind="oracle",
                cpu_model=cpu_model(), cpu_count=os.cpu_count(),
                stage_tokens_per_s={k: round(n / v, 2) for k, v in st.items()},
                dense_tokens_per_s=round(n / st["dense"], 2),
                gpu_speedup=round(gpu_tokens_per_s / value, 1),
                sample=f"{n} uniformly drawn rows of the 131072-token prefill, float64; value = rows / (scores + "
                       f"select + sparse attention seconds) = {dsa_s:.1f} s; dense timed on the same rows "
                       f"({st['dense']:.1f} s)")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=3)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--quick", action="store_true", help="prefill only (no dense/decode/varlen/cpu)")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--only", choices=["decode", "topk", "dedup", "kl", "bwd", "dense"], default=None,
                    help="profiling aid: run only that measurement (dense: the 128K dense causal reference, "
                         "--steps launches)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device-to-device copy 3 times (scales the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the DSA path here runs on a single GPU with no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_attention_long_04_amd import workloads
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30, "copies": 3}), flush=True)
        return
    if args.only == "decode":
        print(json.dumps(bench_decode()), flush=True)
        return
    if args.only == "topk":
        print(json.dumps(bench_topk_general()), flush=True)
        return
    if args.only == "dedup":
        print(json.dumps(bench_dedup()), flush=True)
        return
    if args.only == "kl":
        print(json.dumps(bench_indexer_kl()), flush=True)
        return
    if args.only == "bwd":
        print(json.dumps(bench_sparse_bwd()), flush=True)
        return
    if args.only == "dense":
        print(json.dumps(bench_dense(args.workload or workloads.P128K, args.steps)), flush=True)
        return
    name = args.workload or workloads.P128K
    w = workloads.WORKLOADS[name]
    quick = args.quick

    pre = bench_prefill(name, args.steps, args.warmup, with_dense=not quick)
    T = pre["T"]
    value = T / (pre["ms"] * 1e-3)
    Hq, Hkv, d = 32, 4, 128
    pairs = pairs_of(pre["lengths"])
    sel = selected_of(pre["lengths"], w["topk"])
    peak_idx = PEAK_FP8 if w["idx_dtype"] == "fp8_e4m3" else PEAK_BF16
    traffic = read_traffic()
    # algorithmic work per launch (one launch of each kernel per step)
    idx_flops = pairs * w["idx_heads"] * w["idx_dim"] * 2
    idx_bytes = T * (w["idx_heads"] * w["idx_dim"] * (1 if w["idx_dtype"] == "fp8_e4m3" else 2) + w["idx_heads"] * 4) \
        + 4 * pairs
    topk_bytes = 4 * pairs + 4 * T * w["topk"]
    attn_flops = sel * Hq * d * 4
    attn_bytes = sel * Hkv * d * 2 * 2 + T * (2 * Hq * d * 2 + 4 * w["topk"])
    rooflines = {
        "indexer_prefill_kernel": roof("mfma", idx_flops / (pre["indexer_ms"] * 1e-3), peak_idx, "TFLOP/s",
                                       traffic.get("indexer_prefill_kernel"), idx_flops, "flop"),
        "topk_prefill_kernel": roof("hbm", topk_bytes / (pre["topk_ms"] * 1e-3), PEAK_HBM, "GB/s",
                                    traffic.get("topk_prefill_kernel"), topk_bytes, "byte"),
        # the gather's ceiling: its MFMA work against the bf16 peak, and the bytes it moves below
        # the L2 (counter traffic, when the profile matches the source) against the HBM peak; the
        # algorithmic gathered bytes are mostly served by the L2 and are reported as a rate only
        "gather_rows_kernel": roof("mfma", attn_flops / (pre["attn_ms"] * 1e-3), PEAK_BF16, "TFLOP/s",
                                   traffic.get("gather_rows_kernel"), attn_flops, "flop",
                                   gathered_GBps=round(attn_bytes / (pre["attn_ms"] * 1e-3) / 1e9, 1),
                                   gathered_bytes=attn_bytes,
                                   below_l2=None if traffic.get("gather_rows_kernel") is None else roof(
                                       "hbm", traffic["gather_rows_kernel"] / (pre["attn_ms"] * 1e-3), PEAK_HBM,
                                       "GB/s", traffic["gather_rows_kernel"], traffic["gather_rows_kernel"],
                                       "byte (counter traffic below the L2)")),
    }
    stage_ms = {"indexer_prefill_kernel": pre["indexer_ms"], "topk_prefill_kernel": pre["topk_ms"],
                "gather_rows_kernel": pre["attn_ms"]}
    dominant = max(stage_ms, key=stage_ms.get)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(pre["ms"], 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3+bf16",
        "data": "synthetic",
        "config": {"workload": name, "seq_len": T, "global_batch": len(pre["lengths"]), "topk": w["topk"],
                   "indexer": f"{w['idx_heads']}x{w['idx_dim']} {w['idx_dtype']}", "attention": "GQA 32q/4kv d128 bf16"},
        "roofline": dict(kernel=dominant, **rooflines[dominant]),
        "rooflines": rooflines,
        "stages_ms": {"indexer": round(pre["indexer_ms"], 3), "topk": round(pre["topk_ms"], 3),
                      "sparse_attention": round(pre["attn_ms"], 3)},
        "sparse_attention": {"tflops": round(attn_flops / (pre["attn_ms"] * 1e-3) / 1e12, 1),
                             "frac_bf16_peak": round(attn_flops / (pre["attn_ms"] * 1e-3) / PEAK_BF16, 4),
                             "gathered_GBps": round(sel * Hkv * d * 2 * 2 / (pre["attn_ms"] * 1e-3) / 1e9, 1)},
    }
    if not quick:
        line["dense"] = {"ms": round(pre["dense_ms"], 3), "ratio_dsa_over_dense": round(pre["ms"] / pre["dense_ms"], 4),
                         "dense_frac_bf16_peak": round(pairs_of(pre["lengths"]) * 32 * 128 * 4 /
                                                       (pre["dense_ms"] * 1e-3) / PEAK_BF16, 4)}
        dec = bench_decode()
        line["decode"] = {"us_per_step": round(dec["us_mean"], 2), "us_p50": round(dec["us_p50"], 2),
                          "timed": "dsa_decode alone; dsa_kv_append timed separately",
                          "append_us": round(dec["append_us"], 2),
                          "us_per_step_with_append": round(dec["step_with_append_us"], 2),
                          "stages_us": {"indexer": round(dec["indexer_us"], 2), "topk": round(dec["topk_us"], 2),
                                        "sparse_attention": round(dec["attn_us"], 2)},
                          "stage_timing": "separate pass at the final cache length, events between stages",
                          "hbm_GBps": round(dec["hbm_gbs"], 1), "hbm_frac": round(dec["hbm_gbs"] * 1e9 / PEAK_HBM, 4),
                          "indexer_hbm_frac": round(dec["indexer_gbs"] * 1e9 / PEAK_HBM, 4),
                          "attention_hbm_frac": round(dec["attn_gbs"] * 1e9 / PEAK_HBM, 4),
                          "dense_us": round(dec["dense_us"], 2),
                          "ratio_dsa_over_dense": round(dec["us_mean"] / dec["dense_us"], 4),
                          "workload": workloads.DECODE}
        tk = bench_topk_general()
        line["topk_general"] = {"workload": workloads.TOPK, "ms": round(tk["ms"], 3),
                                "roofline": roof("hbm", tk["work"] / (tk["ms"] * 1e-3), PEAK_HBM, "GB/s", None,
                                                 tk["work"], "byte"),
                                "torch_topk_ms_context": round(tk["torch_topk_ms"], 3)}
        dd = bench_dedup(max(1, args.steps - 1))
        line["dedup"] = {"workload": dd["workload"], "gather_ms": round(dd["gather"]["ms"], 3),
                         "dedup_ms": round(dd["dedup"]["ms"], 3),
                         "tokens_per_s_dedup": round(dd["T"] / (dd["dedup"]["ms"] * 1e-3), 1),
                         "attention_ms": {"gather": round(dd["gather"]["attention_ms"], 3),
                                          "dedup": round(dd["dedup"]["attention_ms"], 3)},
                         "union_mean_16_rows": round(dd["union_mean"], 1),
                         "roofline": roof("mfma", dd["executed_flop"] / (dd["dedup"]["attention_ms"] * 1e-3),
                                          PEAK_BF16, "TFLOP/s", None, dd["executed_flop"], "flop (masked MFMA)"),
                         "useful_tflops": round(dd["useful_flop"] / (dd["dedup"]["attention_ms"] * 1e-3) / 1e12, 1)}
        kr = bench_indexer_kl()
        kl_equiv = kr["bf16_flop"] + kr["fp8_flop"] / 2  # fp8 work counted at half a bf16 flop (twice the rate)
        line["indexer_kl"] = {"workload": "indexer dense warm-up KL, 32768 tokens, indexer 64x128 e4m3, GQA 32q/4kv",
                              "ms": round(kr["ms"], 3),
                              "tokens_per_s": round(kr["tokens"] / (kr["ms"] * 1e-3), 1),
                              "roofline": roof("mfma", kl_equiv / (kr["ms"] * 1e-3), PEAK_BF16, "TFLOP/s", None,
                                               kl_equiv, "bf16-equivalent flop (executed MFMA work)")}
        sb = bench_sparse_bwd()
        line["sparse_attention_bwd"] = {"workload": "prefill_32k (32768 tokens, k = 2048, GQA 32q/4kv d128)",
                                        "ms": round(sb["ms"], 3),
                                        "tokens_per_s": round(sb["tokens"] / (sb["ms"] * 1e-3), 1),
                                        "useful_tflops": round(sb["useful_flop"] / (sb["ms"] * 1e-3) / 1e12, 1)}
        vl = bench_prefill(workloads.VARLEN, max(1, args.steps - 1), 1, with_dense=True)
        line["varlen"] = {"workload": workloads.VARLEN, "tokens_per_s": round(vl["T"] / (vl["ms"] * 1e-3), 1),
                          "ms": round(vl["ms"], 3), "lengths": vl["lengths"],
                          "stages_ms": {"indexer": round(vl["indexer_ms"], 3), "topk": round(vl["topk_ms"], 3),
                                        "sparse_attention": round(vl["attn_ms"], 3)},
                          "dense_ms": round(vl["dense_ms"], 3),
                          "ratio_dsa_over_dense": round(vl["ms"] / vl["dense_ms"], 4),
                          "dense_frac_bf16_peak": round(pairs_of(vl["lengths"]) * 32 * 128 * 4 /
                                                        (vl["dense_ms"] * 1e-3) / PEAK_BF16, 4)}
        del vl
        p32 = bench_prefill(workloads.P32K, args.steps, 1, with_dense=True)
        line["prefill_32k"] = {"workload": workloads.P32K,
                               "tokens_per_s": round(p32["T"] / (p32["ms"] * 1e-3), 1), "ms": round(p32["ms"], 3),
                               "stages_ms": {"indexer": round(p32["indexer_ms"], 3), "topk": round(p32["topk_ms"], 3),
                                             "sparse_attention": round(p32["attn_ms"], 3)},
                               "indexer_frac_fp8_peak": round(pairs_of(p32["lengths"]) * 64 * 128 * 2 /
                                                              (p32["indexer_ms"] * 1e-3) / PEAK_FP8, 4),
                               "dense_ms": round(p32["dense_ms"], 3),
                               "ratio_dsa_over_dense": round(p32["ms"] / p32["dense_ms"], 4),
                               "dense_frac_bf16_peak": round(pairs_of(p32["lengths"]) * 32 * 128 * 4 /
                                                             (p32["dense_ms"] * 1e-3) / PEAK_BF16, 4)}
        del p32
        if not args.no_cpu:
            line["cpu_baseline"] = cpu_baseline(pre["p"], value)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
