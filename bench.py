#!/usr/bin/env python3
"""Benchmark of the DSA hot path on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
  * prefill of one causal 131072-token sequence (k = 2048, attention 32 query
    / 4 KV heads x 128, indexer 64 heads x 128): for each window of query rows
    dsa_index_scores -> dsa_topk -> dsa_sparse_attn_prefill;
  * decode of one new token for each of 64 sequences with 131072 cached
    tokens: dsa_index_scores -> dsa_topk -> dsa_sparse_attn_decode on one
    stream (--decode-groups G > 1 runs G row groups alternating between two
    streams instead).
Inputs are resident in HBM before the timed region starts.

Printed: ONE JSON line.  `value` is prefill tokens/s; decode queries/s, the
per-kernel times, the rooflines, a same-shape dense causal attention run (torch
SDPA, flash backend) and the CPU oracle on a bounded sample of the same
prefill are reported beside it.

    python bench.py [--steps K] [--warmup W] [--window ROWS] [--decode-groups G]
                    [--no-dense] [--no-cpu-baseline] [--cpu-rows N] [--gpus 1]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5000.0    # MI355X dense fp8 MFMA


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=5)
    from long_context_sparse_score_amd.pipeline import BENCH_PREFILL

    ap.add_argument("--window", type=int, default=BENCH_PREFILL.window,
                    help="prefill query rows per score window (with 1024-row attention "
                         "launches, 8192 rows: 156.7-157.1 ms per 128K prefill against "
                         "161.8-163.0 ms with 2048)")
    ap.add_argument("--attn-rows", type=int, default=BENCH_PREFILL.attn_rows,
                    help="split each window's attention into launches of this many rows "
                         "(1024: 50.6 ms against 50.9 ms with 512 and 51.9 ms with 2048)")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-grouped", action="store_true",
                    help="skip the grouped-attention comparison on the correlated-query workload")
    ap.add_argument("--no-kl", action="store_true",
                    help="skip the indexer warm-up step (scores, KL loss and backward; training side)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the optional fp8-indexer variant (reported beside the headline)")
    ap.add_argument("--no-two-stream", action="store_true",
                    help="skip the two-stream prefill (reported beside the one-stream headline)")
    ap.add_argument("--no-fused", action="store_true",
                    help="skip the fused indexer -> top-k variant (reported beside the headline)")
    ap.add_argument("--prefill-streams", type=int, default=1, choices=(1, 2),
                    help="2: each window's attention on a side stream, overlapping the next "
                         "window's indexer")
    ap.add_argument("--decode-groups", type=int, default=1,
                    help="decode row groups; more than one alternate between two streams "
                         "(measured slower here: the attention gathers compete with the next "
                         "group's indexer for HBM)")
    ap.add_argument("--cpu-rows", type=int, default=1024,
                    help="stratified prefill rows the CPU oracle baseline runs (about 20 s)")
    ap.add_argument("--no-workloads", action="store_true",
                    help="skip the 32K and varlen-512K prefill lines")
    ap.add_argument("--calib-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (counter calibration)")
    return ap.parse_args()


def upload_bf16(torch, bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to("cuda").view(torch.bfloat16)


def upload(torch, a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def gen_upload(torch, wl, parts, keep_host=False):
    dev, host = {}, {}
    for p in parts:
        t0 = time.time()
        a = getattr(wl, p)()
        dev[p] = upload(torch, a) if p == "w" else upload_bf16(torch, a)
        if keep_host:
            host[p] = a
        del a
        log(f"  {wl.name}.{p}: {tuple(dev[p].shape)} in {time.time() - t0:.1f}s")
    return dev, host


# ---------------------------------------------------------------- algorithmic counts

def prefill_counts(wl):
    """Work the method itself must do (causal pairs for the indexer, selected
    pairs for the attention)."""
    pairs = 0
    sel = 0
    for L in wl.seqlens_q:
        pairs += L * (L + 1) // 2
        # rows p = 0..L-1 select min(k, p + 1) positions
        k = wl.topk
        m = min(L, k)
        sel += m * (m + 1) // 2 + (L - m) * k
    f_idx = pairs * 2 * wl.n_heads_idx * wl.d_idx
    f_attn = sel * 4 * wl.n_heads_q * wl.head_dim
    b_gather = sel * 2 * wl.n_heads_kv * wl.head_dim * 2
    b_scores = pairs * 4 * 2  # fp32 write by the indexer + read by top-k
    T = sum(wl.seqlens_q)
    # indexer: qI and w read once, each key read once, every causal score written once
    b_idx = T * wl.n_heads_idx * (wl.d_idx * 2 + 4) + T * wl.d_idx * 2 + pairs * 4
    return dict(pairs=pairs, selected=sel, f_idx=f_idx, f_attn=f_attn, b_gather=b_gather,
                b_scores=b_scores, b_idx=b_idx)


def window_flops(wl, r0, n):
    """Indexer flops of packed rows [r0, r0 + n) of a single-sequence prefill."""
    pairs = sum(p + 1 for p in range(r0, r0 + n))
    return pairs * 2 * wl.n_heads_idx * wl.d_idx


def decode_bytes_fp8(wd):
    """Bytes per decode query with the fp8 indexer: the key cache is e4m3 codes
    plus one fp32 scale per key; the new queries are quantised in the step."""
    N = wd.seqlens_k[0]
    k = min(wd.topk, N)
    per = (N * (wd.d_idx + 4)                              # indexer key codes + scales
           + k * 2 * wd.n_heads_kv * wd.head_dim * 2       # gathered K and V rows
           + N * 4 * 2                                     # score write + read
           + wd.topk * 4 * 2                               # indices write + read
           + wd.n_heads_idx * wd.d_idx * (2 + 1 + 1)       # qI read, codes write + read
           + wd.n_heads_idx * 4 * 3                        # w, query scales write + read
           + 2 * wd.n_heads_q * wd.head_dim * 2)           # q, out
    return per * wd.batch, per


def decode_bytes(wd):
    N = wd.seqlens_k[0]
    k = min(wd.topk, N)
    per = (N * wd.d_idx * 2                                # indexer keys
           + k * 2 * wd.n_heads_kv * wd.head_dim * 2       # gathered K and V rows
           + N * 4 * 2                                     # score write + read
           + wd.topk * 4 * 2                               # indices write + read
           + wd.n_heads_idx * wd.d_idx * 2 + wd.n_heads_idx * 4   # qI, w
           + 2 * wd.n_heads_q * wd.head_dim * 2)           # q, out
    return per * wd.batch, per


# ---------------------------------------------------------------- CPU baseline

def counter_traffic(kernel_source, record, window_rows):
    """HBM bytes per launch from the committed FETCH_SIZE / WRITE_SIZE counter
    record, or None once the kernel source or the window size differs from
    the one measured."""
    import hashlib

    try:
        with open(os.path.join(ROOT, record)) as f:
            rec = json.load(f)
        with open(os.path.join(ROOT, kernel_source), "rb") as f:
            digest = hashlib.sha256(f.read()).hexdigest()
    except OSError:
        return None
    if rec.get("source_sha256") != digest or rec.get("window_rows") != window_rows:
        return None
    return int(rec["fetch_bytes_per_dispatch"] + rec["write_bytes_per_dispatch"])


def cpu_model():
    """The host CPU's model name (the lscpu "Model name" field, read from
    /proc/cpuinfo so no tool needs to be installed)."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def stratified_rows(L, k, n, seed=0):
    """n rows, one seeded row from each of n equal strata of [0, L), plus rows
    0, k - 1, k and L - 1."""
    rng = np.random.default_rng(seed)
    edges = np.linspace(0, L, n + 1).astype(np.int64)
    rows = {int(rng.integers(a, max(a + 1, b))) for a, b in zip(edges[:-1], edges[1:])}
    rows |= {0, k - 1, k, L - 1}
    return np.array(sorted(r for r in rows if 0 <= r < L), dtype=np.int64)


def cpu_baseline(wl, host, n_rows, wd=None, wd_host=None):
    """The oracle, untuned, on the GPU host's cores: the whole path (scores,
    top-k, attention in fp64) on a stratified sample of the prefill's rows
    (about n_rows, one per equal stratum of positions, plus rows 0, k-1, k and
    L-1), and on every query of the decode batch.  Stratified rows carry the
    prefill's mean causal length, so the sample's rows/s is its tokens/s."""
    import oracle

    cores = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    L = wl.seqlens_q[0]
    rows = stratified_rows(L, wl.topk, n_rows)
    t0 = time.time()
    oracle.dsa_rows(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"], host["q"],
                    host["k"], host["v"], rows, wl.topk, wl.softmax_scale)
    dt = time.time() - t0
    work = int((rows + 1).sum())
    full_work = L * (L + 1) // 2
    res = {
        "value": round(len(rows) / dt, 3),
        "unit": "tokens/s",
        "cores": cores,
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{len(rows)} query rows of the 131072-token prefill, one seeded row per equal "
                   f"stratum of positions plus rows 0, k-1, k and L-1; whole path (scores, top-k, "
                   f"attention) in fp64, {dt:.1f} s; the full prefill extrapolates to "
                   f"{dt * full_work / work / 3600:.1f} h (extrapolated, by causal pairs)"),
        "seconds": round(dt, 2),
    }
    if wd is not None:
        t0 = time.time()
        oracle.dsa_rows(wd.cu_q, wd.cu_k, wd_host["q_idx"], wd_host["k_idx"], wd_host["w"],
                        wd_host["q"], wd_host["k"], wd_host["v"], np.arange(wd.batch), wd.topk,
                        wd.softmax_scale)
        dt = time.time() - t0
        res["decode"] = {"value": round(wd.batch / dt, 3), "unit": "queries/s",
                         "sample": f"all {wd.batch} queries of the decode step (in full), {dt:.1f} s",
                         "seconds": round(dt, 2)}
    return res


# ---------------------------------------------------------------- main

def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (got --gpus {args.gpus}); this build has no "
              "multi-GPU path", file=sys.stderr)
        sys.exit(2)
    import torch

    import long_context_sparse_score_amd as dsa
    from long_context_sparse_score_amd import pipeline
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    dsa.load_library()
    stream = torch.cuda.current_stream()

    # ---- prefill workload: one causal 131072-token sequence
    wl = synth.prefill_128k()
    log(f"generating {wl.name}")
    P, P_host = gen_upload(torch, wl, ("q_idx", "k_idx", "w", "q", "k", "v"),
                           keep_host=not args.no_cpu_baseline)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    two = args.prefill_streams > 1
    bufs = pipeline.alloc_prefill(vl, wl.topk, args.window, overlap=two)
    pside = torch.cuda.Stream() if two else None
    out = torch.empty((wl.total_q, wl.n_heads_q, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.total_q, wl.n_heads_q), dtype=torch.float32, device="cuda")
    window = bufs.scores.shape[0]
    windows = [(r0, min(window, wl.total_q - r0)) for r0 in range(0, wl.total_q, window)]

    # ---- decode workload: 64 sequences x 131072 cached tokens
    wd = synth.decode_b64_128k()
    if not args.no_decode:
        log(f"generating {wd.name}")
        D, D_host = gen_upload(torch, wd, ("q_idx", "k_idx", "w", "q", "k", "v"),
                               keep_host=not args.no_cpu_baseline)
        vd = dsa.Varlen(wd.cu_q.tolist(), wd.cu_k.tolist())
        dbufs = pipeline.alloc_decode(vd, wd.n_heads_q, wd.head_dim, wd.topk,
                                      groups=args.decode_groups)
        dbufs1 = pipeline.alloc_decode(vd, wd.n_heads_q, wd.head_dim, wd.topk, groups=1)
        side = torch.cuda.Stream() if len(dbufs.groups) > 1 else None
        dout = torch.empty((wd.batch, wd.n_heads_q, wd.head_dim), dtype=torch.bfloat16,
                           device="cuda")
        dlse = torch.empty((wd.batch, wd.n_heads_q), dtype=torch.float32, device="cuda")

    def ev():
        return torch.cuda.Event(enable_timing=True)

    def run_prefill(rec):
        # The timed prefill: every window's index_scores -> topk -> attention
        # (with --prefill-streams 2, each window's attention on a side stream,
        # overlapping the next window's indexer), events around every call.
        pipeline.prefill(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"], P["v"], out, bufs,
                         lse=lse, stream=stream, side_stream=pside, record=rec,
                         attn_rows=args.attn_rows)

    def run_decode():
        # The timed decode step (with --decode-groups > 1: row groups alternating
        # between two streams).
        pipeline.decode(vd, D["q_idx"], D["k_idx"], D["w"], D["q"], D["k"], D["v"], dout, dbufs,
                        lse=dlse, side_stream=side)

    def decode_breakdown(rec):
        # The three calls one after the other on one stream, each between events
        # (per-kernel times; not the timed step).
        e = [ev() for _ in range(4)]
        e[0].record(stream)
        dsa.dsa_index_scores(vd, D["q_idx"], D["k_idx"], D["w"], dbufs1.scores)
        e[1].record(stream)
        dsa.dsa_topk(vd, dbufs1.scores, dbufs1.indices, workspace=dbufs1.topk_workspace)
        e[2].record(stream)
        dsa.dsa_sparse_attn_decode(vd, D["q"], D["k"], D["v"], dbufs1.indices, dout,
                                   dbufs1.workspaces[0], lse=dlse)
        e[3].record(stream)
        rec.append(e)

    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        run_prefill(None)
        torch.cuda.synchronize()
        log("  warmup prefill done")
        if not args.no_decode:
            run_decode()
            torch.cuda.synchronize()
            decode_breakdown([])
            torch.cuda.synchronize()
            log("  warmup decode done")

    log(f"timing {args.steps} step(s)")
    prec, drec, marks = [], [], []
    t_wall = time.time()
    for step in range(args.steps):
        m = [ev(), ev(), ev()]
        m[0].record(stream)
        run_prefill(prec)
        m[1].record(stream)
        if not args.no_decode:
            run_decode()
        m[2].record(stream)
        marks.append(m)
        # Waiting between steps leaves the event-timed regions unchanged.
        torch.cuda.synchronize()
        log(f"  step {step}: {m[0].elapsed_time(m[2]):.2f} ms")
    t_wall = time.time() - t_wall
    if not args.no_decode:
        for _ in range(args.steps):
            decode_breakdown(drec)
            torch.cuda.synchronize()

    pre_ms = sum(m[0].elapsed_time(m[1]) for m in marks)
    dec_ms = sum(m[1].elapsed_time(m[2]) for m in marks) if not args.no_decode else 0.0
    step_ms = (pre_ms + dec_ms) / args.steps
    def span(e, name):
        return e[name][0].elapsed_time(e[name][1])

    idx_ms = sum(span(e, "index_scores") for _, _, e in prec)
    topk_ms = sum(span(e, "topk") for _, _, e in prec)
    attn_ms = sum(span(e, "sparse_attn") for _, _, e in prec)
    n_idx_launches = len(prec)

    pc = prefill_counts(wl)
    tokens_per_s = wl.total_q * args.steps / (pre_ms / 1e3)
    f_idx_total = pc["f_idx"] * args.steps
    idx_tflops = f_idx_total / (idx_ms / 1e3) / 1e12
    t_mfma = (pc["f_idx"] + pc["f_attn"]) / (PEAK_BF16_TFLOPS * 1e12)
    t_comb = (pc["f_idx"] / (PEAK_BF16_TFLOPS * 1e12) + pc["b_scores"] / (PEAK_HBM_GBS * 1e9)
              + max(pc["f_attn"] / (PEAK_BF16_TFLOPS * 1e12), pc["b_gather"] / (PEAK_HBM_GBS * 1e9)))
    pre_s_per_step = pre_ms / 1e3 / args.steps

    result = {
        "metric": "DSA prefill tokens/s & decode queries/s at 128K ctx, k=2048; % of roofline",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(step_ms, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; block-clustered keys for prefill, N(0,1) caches for decode)",
        "config": {
            "workload": "prefill_128k (1 x 131072 tokens) + decode_b64_128k (64 x 131072 cached)",
            "seq_len": wl.seqlens_q[0], "topk": wl.topk, "n_heads_q": wl.n_heads_q,
            "n_heads_kv": wl.n_heads_kv, "head_dim": wl.head_dim,
            "n_heads_idx": wl.n_heads_idx, "d_idx": wl.d_idx, "decode_batch": wd.batch,
            "window_rows": window,
        },
        "roofline": {
            "bound": "mfma",
            "kernel": "index_scores (prefill)",
            "achieved": round(idx_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(idx_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": counter_traffic("long_context_sparse_score_amd/csrc/index_scores.hip",
                                       "profiles/index_scores_traffic.json", window),
            "traffic_unit": "HBM bytes per launch (calibrated FETCH_SIZE + WRITE_SIZE)",
            "algorithmic_bytes_per_launch": int(pc["b_idx"] / max(1, n_idx_launches // args.steps)),
            "launches_per_step": n_idx_launches // args.steps,
            "avg_launch_ms": round(idx_ms / n_idx_launches, 3),
            "flops_per_causal_pair": 2 * wl.n_heads_idx * wl.d_idx,
        },
        "prefill": {
            "ms": round(pre_ms / args.steps, 3),
            "tokens_per_s": round(tokens_per_s, 1),
            "streams": args.prefill_streams,
            "index_scores_ms": round(idx_ms / args.steps, 3),
            "topk_ms": round(topk_ms / args.steps, 3),
            "topk_score_read_GBps": round(pc["b_scores"] / 2 * args.steps / (topk_ms / 1e3) / 1e9, 1),
            "sparse_attn_ms": round(attn_ms / args.steps, 3),
            "sparse_attn_gather_GBps": round(pc["b_gather"] * args.steps / (attn_ms / 1e3) / 1e9, 1),
            "sparse_attn_tflops": round(pc["f_attn"] * args.steps / (attn_ms / 1e3) / 1e12, 2),
            "mfma_roofline_ms": round(t_mfma * 1e3, 3),
            "mfma_roofline_frac": round(t_mfma / pre_s_per_step, 4),
            "combined_roofline_ms": round(t_comb * 1e3, 3),
            "combined_roofline_frac": round(t_comb / pre_s_per_step, 4),
            "algorithmic": {k: int(v) for k, v in pc.items()},
        },
        "wall_s_timed": round(t_wall, 3),
        "device": device_info(torch),
    }

    if not args.no_decode:
        b_dec, per_q = decode_bytes(wd)
        d_idx_ms = sum(e[0].elapsed_time(e[1]) for e in drec)
        d_topk_ms = sum(e[1].elapsed_time(e[2]) for e in drec)
        d_attn_ms = sum(e[2].elapsed_time(e[3]) for e in drec)
        q_per_s = wd.batch * args.steps / (dec_ms / 1e3)
        achieved = b_dec * args.steps / (dec_ms / 1e3) / 1e9
        result["decode"] = {
            "value": round(q_per_s, 1),
            "unit": "queries/s",
            "ms": round(dec_ms / args.steps, 4),
            "groups": len(dbufs.groups),
            "streams": 2 if side is not None else 1,
            "index_scores_ms": round(d_idx_ms / args.steps, 4),
            "topk_ms": round(d_topk_ms / args.steps, 4),
            "sparse_attn_ms": round(d_attn_ms / args.steps, 4),
            "breakdown": "index_scores/topk/sparse_attn ms: the three calls for the whole batch "
                         "one after another on one stream (outside the timed step)",
            "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": round(achieved / PEAK_HBM_GBS, 4),
                         "bytes_per_query": per_q},
            "index_scores_GBps": round(wd.batch * wd.seqlens_k[0] * wd.d_idx * 2 * args.steps
                                       / (d_idx_ms / 1e3) / 1e9, 1),
        }

    att = attainable_peaks(torch, stream)
    result["attainable"] = att
    result["roofline"]["attainable_peak"] = att["mfma_bf16_tflops"]
    result["roofline"]["frac_of_attainable"] = round(idx_tflops / att["mfma_bf16_tflops"], 4)
    if "decode" in result:
        r = result["decode"]["roofline"]
        r["attainable_peak"] = att["read_GBps"]
        r["frac_of_attainable"] = round(r["achieved"] / att["read_GBps"], 4)

    if args.calib_copy:
        # A plain copy of known size: its FETCH_SIZE / WRITE_SIZE counter readings
        # calibrate the same counters taken on the DSA kernels.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    if not args.no_fp8:
        result["fp8_indexer"] = fp8_variant(torch, pipeline, args, stream, wl, vl, P, out, lse,
                                            None if args.no_decode else (wd, vd, D, dout, dlse))

    if not args.no_workloads:
        result["workloads"] = {w.name: workload_line(torch, pipeline, args, stream, w)
                               for w in (synth.prefill_32k(), synth.varlen_512k())}

    if args.prefill_streams == 1 and not args.no_two_stream:
        result["two_stream_prefill"] = two_stream_variant(torch, pipeline, args, stream, wl, vl, P,
                                                          out, lse, pre_ms / args.steps)

    if not args.no_fused:
        result["fused_index_topk"] = fused_variant(
            torch, dsa, pipeline, args, stream, wl, vl, P, out, lse, pre_ms / args.steps,
            idx_ms / args.steps + topk_ms / args.steps,
            None if args.no_decode else (wd, vd, D, dout, dlse, dec_ms / args.steps,
                                         (d_idx_ms + d_topk_ms) / args.steps))

    if not args.no_kl:
        result["indexer_warmup"] = kl_variant(torch, dsa, pipeline, args, stream, wl, vl, P)

    if not args.no_grouped:
        result["grouped_attention"] = grouped_variant(torch, dsa, pipeline, args, stream, wl, vl, P,
                                                      out, lse, attn_ms / args.steps)

    if not args.no_dense:
        result["dense"] = dense_comparator(torch, P, wl, args, pre_ms / args.steps)

    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_rows} sampled rows")
        result["cpu_baseline"] = cpu_baseline(wl, P_host, args.cpu_rows,
                                              None if args.no_decode else wd,
                                              None if args.no_decode else D_host)

    print(json.dumps(result), flush=True)


def two_stream_variant(torch, pipeline, args, stream, wl, vl, P, out, lse, single_ms):
    """The headline prefill with each window's attention on a second stream,
    overlapping the next window's indexer and top-k (same kernels, same
    launches, bitwise the same output).  Reported beside the one-stream
    headline, whose per-kernel events and roofline fractions measure kernels
    that run alone."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    bufs = pipeline.alloc_prefill(vl, wl.topk, args.window, overlap=True)
    side = torch.cuda.Stream()
    run = lambda: pipeline.prefill(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"], P["v"],  # noqa: E731
                                   out, bufs, lse=lse, stream=stream, side_stream=side,
                                   attn_rows=args.attn_rows)
    log("two-stream prefill")
    for _ in range(args.warmup):
        run()
    torch.cuda.synchronize()
    tot = 0.0
    for _ in range(args.steps):
        a, b = ev(), ev()
        a.record(stream)
        run()
        b.record(stream)
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    ms = tot / args.steps
    del bufs
    return {"note": "each window's attention on a second stream, overlapping the next window's "
                    "indexer and top-k; the kernels slow each other, so the headline's per-kernel "
                    "rooflines are taken on one stream",
            "ms": round(ms, 3), "tokens_per_s": round(wl.total_q / (ms / 1e3), 1),
            "one_stream_ms": round(single_ms, 3)}


def fp8_variant(torch, pipeline, args, stream, wl, vl, P, out, lse, dec):
    """The same prefill and decode steps with the optional fp8 indexer
    (e4m3 codes, one scale per vector).  Not the headline: the configuration's
    indexer is bf16.  Prefill steps include quantising qI and kI; the decode
    key cache is quantised once beforehand (as it would be when tokens are
    appended) and each step quantises its new queries."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    res = {"note": "optional fp8 (e4m3, per-vector scales) indexer variant; the workload's "
                   "indexer is bf16, so this is reported beside the headline, not as it"}
    bufs = pipeline.alloc_prefill(vl, wl.topk, args.window)
    fp8 = pipeline.alloc_fp8_indexer(wl.total_q, wl.total_k, wl.n_heads_idx, wl.d_idx)
    run = lambda rec: pipeline.prefill(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"],  # noqa: E731
                                       P["v"], out, bufs, lse=lse, stream=stream, record=rec,
                                       fp8=fp8, attn_rows=args.attn_rows)
    log("fp8 indexer: prefill")
    for _ in range(args.warmup):
        run(None)
    torch.cuda.synchronize()
    rec, marks = [], []
    for _ in range(args.steps):
        m0, m1 = ev(), ev()
        m0.record(stream)
        n0 = len(rec)
        run(rec)
        m1.record(stream)
        marks.append((m0, m1, n0))
        torch.cuda.synchronize()
    pre_ms = sum(a.elapsed_time(b) for a, b, _ in marks) / args.steps
    quant_ms = sum(a.elapsed_time(rec[n0][2]["index_scores"][0]) for a, _, n0 in marks) / args.steps
    span = lambda name: sum(e[name][0].elapsed_time(e[name][1]) for _, _, e in rec) / args.steps  # noqa: E731
    idx_ms = span("index_scores")
    pc = prefill_counts(wl)
    tflops = pc["f_idx"] / (idx_ms / 1e3) / 1e12
    res["prefill"] = {
        "ms": round(pre_ms, 3), "tokens_per_s": round(wl.total_q / (pre_ms / 1e3), 1),
        "quantize_ms": round(quant_ms, 3), "index_scores_ms": round(idx_ms, 3),
        "topk_ms": round(span("topk"), 3), "sparse_attn_ms": round(span("sparse_attn"), 3),
        "roofline": {"bound": "mfma", "kernel": "index_scores_fp8 (prefill)",
                     "achieved": round(tflops, 2), "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_FP8_TFLOPS, 4),
                     "avg_launch_ms": round(idx_ms / max(1, len(rec) // args.steps), 3)},
    }
    del bufs, fp8
    if dec is not None:
        wd, vd, D, dout, dlse = dec
        dbufs = pipeline.alloc_decode(vd, wd.n_heads_q, wd.head_dim, wd.topk)
        fp8d = pipeline.alloc_fp8_indexer(wd.total_q, wd.total_k, wd.n_heads_idx, wd.d_idx)
        pipeline.quantize_keys(D["k_idx"], fp8d, stream=stream)
        step = lambda: pipeline.decode(vd, D["q_idx"], None, D["w"], D["q"], D["k"], D["v"],  # noqa: E731
                                       dout, dbufs, lse=dlse, stream=stream, fp8=fp8d)
        log("fp8 indexer: decode")
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        tot = 0.0
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        ms = tot / args.steps
        b_dec, per_q = decode_bytes_fp8(wd)
        gbs = b_dec / (ms / 1e3) / 1e9
        res["decode"] = {"ms": round(ms, 4), "queries_per_s": round(wd.batch / (ms / 1e3), 1),
                         "roofline": {"bound": "hbm", "achieved": round(gbs, 1),
                                      "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                      "frac": round(gbs / PEAK_HBM_GBS, 4),
                                      "bytes_per_query": per_q}}
        del dbufs, fp8d
    torch.cuda.empty_cache()
    return res


def workload_line(torch, pipeline, args, stream, wl):
    """The headline's prefill (same windows, attention launches, one stream)
    on another of the seeded workloads: 32K tokens, or the varlen batch of
    524288 tokens in log-uniform lengths.  Rooflines from the workload's own
    causal and selected pairs (for varlen, the drawn lengths)."""
    import long_context_sparse_score_amd as dsa

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    log(f"workload {wl.name}: generating")
    P, _ = gen_upload(torch, wl, ("q_idx", "k_idx", "w", "q", "k", "v"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    bufs = pipeline.alloc_prefill(vl, wl.topk, args.window)
    out = torch.empty((wl.total_q, wl.n_heads_q, wl.head_dim), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((wl.total_q, wl.n_heads_q), dtype=torch.float32, device="cuda")
    run = lambda rec: pipeline.prefill(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"],  # noqa: E731
                                       P["v"], out, bufs, lse=lse, stream=stream, record=rec,
                                       attn_rows=args.attn_rows)
    for _ in range(args.warmup):
        run(None)
    torch.cuda.synchronize()
    rec, tot = [], 0.0
    for _ in range(args.steps):
        a, b = ev(), ev()
        a.record(stream)
        run(rec)
        b.record(stream)
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    ms = tot / args.steps
    span = lambda name: sum(e[name][0].elapsed_time(e[name][1]) for _, _, e in rec) / args.steps  # noqa: E731
    pc = prefill_counts(wl)
    t_mfma = (pc["f_idx"] + pc["f_attn"]) / (PEAK_BF16_TFLOPS * 1e12) * 1e3
    t_comb = (pc["f_idx"] / (PEAK_BF16_TFLOPS * 1e12) + pc["b_scores"] / (PEAK_HBM_GBS * 1e9)
              + max(pc["f_attn"] / (PEAK_BF16_TFLOPS * 1e12), pc["b_gather"] / (PEAK_HBM_GBS * 1e9))) * 1e3
    idx_ms = span("index_scores")
    tflops = pc["f_idx"] / (idx_ms / 1e3) / 1e12
    res = {"sequences": len(wl.seqlens_q), "tokens": wl.total_q, "max_seqlen": wl.max_seqlen_k,
           "ms": round(ms, 3), "tokens_per_s": round(wl.total_q / (ms / 1e3), 1),
           "index_scores_ms": round(idx_ms, 3), "topk_ms": round(span("topk"), 3),
           "sparse_attn_ms": round(span("sparse_attn"), 3),
           "mfma_roofline_ms": round(t_mfma, 3), "mfma_roofline_frac": round(t_mfma / ms, 4),
           "combined_roofline_ms": round(t_comb, 3), "combined_roofline_frac": round(t_comb / ms, 4),
           "index_scores_roofline": {"bound": "mfma", "achieved": round(tflops, 2),
                                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4)},
           "algorithmic": {k: int(v) for k, v in pc.items()}}
    if len(wl.seqlens_q) > 1:
        res["seqlens"] = list(wl.seqlens_q)
    del P, bufs, out, lse
    torch.cuda.empty_cache()
    return res


def fused_variant(torch, dsa, pipeline, args, stream, wl, vl, P, out, lse, unfused_prefill_ms,
                  unfused_select_ms, dec):
    """The same prefill and decode steps with the indexer and the top-k fused
    (dsa_index_topk: the indexer keeps only candidates above a threshold read
    off a sample of each row, an exact select runs over them, rows it cannot
    settle are recomputed unfused).  Same windows and attention launches as
    the headline; the selection is bitwise the headline's."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    res = {"note": "fused indexer -> top-k (no score rows); same selection, reported beside the "
                   "unfused headline"}
    bufs = pipeline.alloc_prefill(vl, wl.topk, args.window, fused=True)
    run = lambda rec: pipeline.prefill(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"],  # noqa: E731
                                       P["v"], out, bufs, lse=lse, stream=stream, record=rec,
                                       attn_rows=args.attn_rows)
    log("fused indexer -> top-k: prefill")
    for _ in range(args.warmup):
        run(None)
    torch.cuda.synchronize()
    rec, tot = [], 0.0
    for _ in range(args.steps):
        a, b = ev(), ev()
        a.record(stream)
        run(rec)
        b.record(stream)
        torch.cuda.synchronize()
        tot += a.elapsed_time(b)
    pre_ms = tot / args.steps
    span = lambda name: sum(e[name][0].elapsed_time(e[name][1]) for _, _, e in rec) / args.steps  # noqa: E731
    # Candidate counts and fallbacks of every window (an untimed pass).
    counts, fallbacks = [], 0
    window = bufs.window
    for r0 in range(0, wl.total_q, window):
        n = min(window, wl.total_q - r0)
        dsa.dsa_index_topk(vl, P["q_idx"], P["k_idx"], P["w"], bufs.indices[:n], bufs.fused,
                           row_begin=r0, row_count=n)
        off = (n * 4 + 255) // 256 * 256
        counts.append(bufs.fused[:4 * n].view(torch.int32).cpu())
        fallbacks += int(bufs.fused[off:off + 4 * n].view(torch.int32).sum())
    c = torch.cat(counts).double()
    long_rows = c[torch.arange(wl.total_q) + 1 > 10240]
    res["prefill"] = {
        "ms": round(pre_ms, 3), "tokens_per_s": round(wl.total_q / (pre_ms / 1e3), 1),
        "unfused_ms": round(unfused_prefill_ms, 3),
        "index_topk_ms": round(span("index_scores"), 3),
        "unfused_index_scores_plus_topk_ms": round(unfused_select_ms, 3),
        "sparse_attn_ms": round(span("sparse_attn"), 3),
        "candidates_long_rows": {"mean": round(float(long_rows.mean()), 1),
                                 "min": int(long_rows.min()), "max": int(long_rows.max())},
        "fallback_rows": fallbacks,
    }
    del bufs
    if dec is not None:
        wd, vd, D, dout, dlse, unfused_dec_ms, unfused_dec_sel_ms = dec
        dbufs = pipeline.alloc_decode(vd, wd.n_heads_q, wd.head_dim, wd.topk, fused=True)
        step = lambda: pipeline.decode(vd, D["q_idx"], D["k_idx"], D["w"], D["q"], D["k"], D["v"],  # noqa: E731
                                       dout, dbufs, lse=dlse, stream=stream)
        log("fused indexer -> top-k: decode")
        for _ in range(max(1, args.warmup)):
            step()
        torch.cuda.synchronize()
        tot, sel = 0.0, 0.0
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            step()
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
            a, b = ev(), ev()
            a.record(stream)
            dsa.dsa_index_topk(vd, D["q_idx"], D["k_idx"], D["w"], dbufs.indices, dbufs.fused[0])
            b.record(stream)
            torch.cuda.synchronize()
            sel += a.elapsed_time(b)
        ms = tot / args.steps
        res["decode"] = {"ms": round(ms, 4), "queries_per_s": round(wd.batch / (ms / 1e3), 1),
                         "unfused_ms": round(unfused_dec_ms, 4),
                         "index_topk_ms": round(sel / args.steps, 4),
                         "unfused_index_scores_plus_topk_ms": round(unfused_dec_sel_ms, 4)}
        del dbufs
    torch.cuda.empty_cache()
    return res


def kl_variant(torch, dsa, pipeline, args, stream, wl, vl, P):
    """The indexer's dense warm-up step over the whole prefill
    (pipeline.warmup): per 8192-row window the indexer scores, the KL loss
    with its gradient written over the scores (dsa_indexer_kl), and the
    gradient into the indexer's queries, weights and keys
    (dsa_index_scores_backward), each timed by HIP events on the launch
    stream.  The KL computes two dense logit passes per causal pair
    (4 Hq d flops); the backward recomputes the head products twice and runs
    two GEMMs of the same size (8 H_I d_I flops per pair).  A second pass
    times the backward's two kernels apart (dq/dw alone, dk alone)."""
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    pc = prefill_counts(wl)
    H, D = wl.n_heads_idx, wl.d_idx
    kl_flops = pc["pairs"] * 4 * wl.n_heads_q * wl.head_dim
    half_flops = pc["pairs"] * 4 * H * D  # one backward kernel: x again plus one GEMM
    wb = pipeline.alloc_warmup(vl, H, D)
    loss = torch.empty(wl.total_q, dtype=torch.float32, device="cuda")
    dq = torch.empty((wl.total_q, H, D), dtype=torch.float32, device="cuda")
    dw = torch.empty((wl.total_q, H), dtype=torch.float32, device="cuda")
    dk = torch.empty((wl.total_k, D), dtype=torch.float32, device="cuda")
    log("indexer warm-up step: one pass over the prefill")
    rec = []
    a, b = ev(), ev()
    a.record(stream)
    pipeline.warmup(vl, P["q_idx"], P["k_idx"], P["w"], P["q"], P["k"], loss, dq, dw, dk, wb,
                    stream=stream, record=rec)
    b.record(stream)
    torch.cuda.synchronize()
    total = a.elapsed_time(b)
    span = {kind: sum(e[kind][0].elapsed_time(e[kind][1]) for _, _, e in rec)
            for kind in ("index_scores", "indexer_kl", "backward")}
    log("indexer warm-up step: backward kernels timed apart")
    parts = {"dq_dw": 0.0, "dk": 0.0}
    for r0 in range(0, wl.total_q, wb.window):
        n = min(wb.window, wl.total_q - r0)
        sc = wb.scores[:n]
        dsa.dsa_index_scores(vl, P["q_idx"], P["k_idx"], P["w"], sc, row_begin=r0, row_count=n)
        dsa.dsa_indexer_kl(vl, P["q"], P["k"], sc, loss[r0:r0 + n], grad=sc, row_begin=r0,
                           row_count=n)
        for part in ("dq_dw", "dk"):
            e0, e1 = ev(), ev()
            e0.record(stream)
            dsa.dsa_index_scores_backward(
                vl, P["q_idx"], P["k_idx"], P["w"], sc, wb.workspace,
                dq_idx=dq[r0:r0 + n] if part == "dq_dw" else None,
                dw=dw[r0:r0 + n] if part == "dq_dw" else None,
                dk_idx=dk if part == "dk" else None, row_begin=r0, row_count=n)
            e1.record(stream)
            torch.cuda.synchronize()
            parts[part] += e0.elapsed_time(e1)
    del wb, dq, dw, dk
    torch.cuda.empty_cache()

    def roof(kernel, flops, ms):
        tf = flops / (ms / 1e3) / 1e12
        return {"bound": "mfma", "kernel": kernel, "achieved": round(tf, 2),
                "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4)}
    return {
        "window_rows": pipeline.WARMUP_WINDOW, "launches": len(rec),
        "step_ms": round(total, 3),
        "tokens_per_s": round(wl.total_q / (total / 1e3), 1),
        "index_scores_ms": round(span["index_scores"], 3),
        "indexer_kl_ms": round(span["indexer_kl"], 3),
        "backward_ms": round(span["backward"], 3),
        "mean_loss_per_row": round(float(loss.mean()), 5),
        "roofline": dict(roof("indexer_kl", kl_flops, span["indexer_kl"]),
                         flops_per_causal_pair=4 * wl.n_heads_q * wl.head_dim),
        "backward": {
            "ms": round(span["backward"], 3),
            "roofline": dict(roof("index backward (dq/dw + dk)", 2 * half_flops,
                                  span["backward"]),
                             flops_per_causal_pair=8 * H * D),
            "dq_dw_ms": round(parts["dq_dw"], 3),
            "dq_dw_roofline": roof("index_bwd_dq_kernel (+ key transpose)", half_flops,
                                   parts["dq_dw"]),
            "dk_ms": round(parts["dk"], 3),
            "dk_roofline": roof("index_bwd_dk_kernel (+ query transpose)", half_flops,
                                parts["dk"]),
        },
    }


def grouped_variant(torch, dsa, pipeline, args, stream, wl, vl, P, out, lse, iid_attn_ms):
    """Adjacent-query de-duplication (grouped attention, 16 rows per union of
    index sets) against the per-row attention, on prefill_128k_corr: the same
    tensors as the headline prefill except the indexer queries, which share a
    per-block mean.  Both whole prefills are timed; the union sizes come from
    an untimed pass.  The grouped attention on the headline (i.i.d.-query)
    workload is timed too, where the sets barely overlap."""
    import synth

    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    wc = synth.prefill_128k_corr()
    log(f"grouped attention: generating {wc.name} indexer queries")
    qc = upload_bf16(torch, wc.q_idx())
    res = {"workload": f"{wc.name} (indexer query block means of std {wc.query_mean_std})",
           "group_rows": 16}
    modes = {}
    for name, grouped in (("per_row", False), ("grouped", True)):
        bufs = pipeline.alloc_prefill(vl, wl.topk, args.window, grouped=grouped)
        run = lambda rec: pipeline.prefill(vl, qc, P["k_idx"], P["w"], P["q"], P["k"], P["v"],  # noqa: E731
                                           out, bufs, lse=lse, stream=stream, record=rec,
                                           attn_rows=None if grouped else args.attn_rows)
        for _ in range(args.warmup):
            run(None)
        torch.cuda.synchronize()
        rec, tot = [], 0.0
        for _ in range(args.steps):
            a, b = ev(), ev()
            a.record(stream)
            run(rec)
            b.record(stream)
            torch.cuda.synchronize()
            tot += a.elapsed_time(b)
        attn = sum(e["sparse_attn"][0].elapsed_time(e["sparse_attn"][1]) for _, _, e in rec)
        modes[name] = {"prefill_ms": round(tot / args.steps, 3),
                       "tokens_per_s": round(wl.total_q / (tot / args.steps / 1e3), 1),
                       "sparse_attn_ms": round(attn / args.steps, 3)}
        if grouped:
            # Union sizes of every group, one window at a time (untimed).
            counts = []
            window = bufs.scores.shape[0]
            for r0 in range(0, wl.total_q, window):
                n = min(window, wl.total_q - r0)
                dsa.dsa_index_scores(vl, qc, P["k_idx"], P["w"], bufs.scores, row_begin=r0,
                                     row_count=n)
                dsa.dsa_topk(vl, bufs.scores, bufs.indices, row_begin=r0, row_count=n)
                dsa.dsa_sparse_attn_prefill_grouped(vl, P["q"], P["k"], P["v"], bufs.indices, out,
                                                    bufs.grouped, row_begin=r0, row_count=n)
                groups = (n + 15) // 16
                ent = groups * 16 * wl.topk
                off = -(-ent * 4 // 256) * 256 + -(-ent * 2 // 256) * 256
                counts.append(bufs.grouped[off:off + 4 * groups].view(torch.int32).cpu())
            c = torch.cat(counts).double()
            res["unique_kv_per_16_rows"] = {"mean": round(float(c.mean()), 1),
                                            "min": int(c.min()), "max": int(c.max()),
                                            "without_dedup": 16 * wl.topk}
            # The grouped attention on the headline workload's own indices.
            tot_iid = 0.0
            for r0 in range(0, wl.total_q, window):
                n = min(window, wl.total_q - r0)
                dsa.dsa_index_scores(vl, P["q_idx"], P["k_idx"], P["w"], bufs.scores, row_begin=r0,
                                     row_count=n)
                dsa.dsa_topk(vl, bufs.scores, bufs.indices, row_begin=r0, row_count=n)
                a, b = ev(), ev()
                a.record(stream)
                dsa.dsa_sparse_attn_prefill_grouped(vl, P["q"], P["k"], P["v"], bufs.indices, out,
                                                    bufs.grouped, row_begin=r0, row_count=n)
                b.record(stream)
                torch.cuda.synchronize()
                tot_iid += a.elapsed_time(b)
            res["headline_workload_attention_ms"] = {"per_row": round(iid_attn_ms, 3),
                                                     "grouped": round(tot_iid, 3)}
        del bufs
    res.update(modes)
    del qc
    torch.cuda.empty_cache()
    return res


def attainable_peaks(torch, stream):
    """Measured ceilings beside the published peaks: a loop of back-to-back
    bf16 MFMAs on every SIMD (libdsa_calib.so, outside the C ABI; no loads)
    and a plain device-to-device copy.  Under full matrix-core load the chip
    holds an engine clock below the boost clock the published MFMA peak
    assumes, so a kernel's fraction of the attainable figure says how much
    of the achievable throughput it gets."""
    import ctypes

    from long_context_sparse_score_amd import build_lib
    lib = ctypes.CDLL(build_lib.CALIB_PATH)
    lib.dsa_calib_mfma_bf16.argtypes = [ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_void_p]
    lib.dsa_calib_mfma_bf16.restype = ctypes.c_int
    lib.dsa_calib_read.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p,
                                   ctypes.c_void_p]
    lib.dsa_calib_read.restype = ctypes.c_int
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    blocks, iters = cus * 4, 40000            # four 256-thread workgroups per CU
    out = torch.empty(blocks * 256, dtype=torch.float32, device="cuda")
    ev = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    assert lib.dsa_calib_mfma_bf16(iters // 4, blocks, out.data_ptr(), stream.cuda_stream) == 0
    a, b = ev(), ev()
    a.record(stream)
    assert lib.dsa_calib_mfma_bf16(iters, blocks, out.data_ptr(), stream.cuda_stream) == 0
    b.record(stream)
    torch.cuda.synchronize()
    mfma_tflops = blocks * 4 * iters * 16 * 32768 / (a.elapsed_time(b) / 1e3) / 1e12
    src = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    src.fill_(1)
    dst.copy_(src)
    a.record(stream)
    for _ in range(3):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * src.numel() / (a.elapsed_time(b) / 1e3) / 1e9
    del dst
    read = {}
    sink = torch.empty(cus * 16 * 256, dtype=torch.int32, device="cuda")  # one word per thread
    for per_cu in (4, 8, 16):
        nb = cus * per_cu
        assert nb * 256 <= sink.numel()
        assert lib.dsa_calib_read(src.data_ptr(), src.numel(), nb, sink.data_ptr(),
                                  stream.cuda_stream) == 0
        a.record(stream)
        for _ in range(3):
            lib.dsa_calib_read(src.data_ptr(), src.numel(), nb, sink.data_ptr(), stream.cuda_stream)
        b.record(stream)
        torch.cuda.synchronize()
        read[per_cu] = 3 * src.numel() / (a.elapsed_time(b) / 1e3) / 1e9
    read_gbs = max(read.values())
    del src, sink
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": round(mfma_tflops, 1),
            "mfma_frac_of_published": round(mfma_tflops / PEAK_BF16_TFLOPS, 4),
            "copy_GBps": round(copy_gbs, 1),
            "copy_frac_of_published": round(copy_gbs / PEAK_HBM_GBS, 4),
            "read_GBps": round(read_gbs, 1),
            "read_frac_of_published": round(read_gbs / PEAK_HBM_GBS, 4),
            "how": "bf16 MFMA: back-to-back v_mfma_f32_32x32x16_bf16, 4 waves per SIMD, "
                   "4 independent accumulators; copy: 4 GiB device-to-device, bytes read + written; "
                   "read: 4 GiB streamed by 16-byte loads (best of 4, 8, 16 workgroups per CU)"}


def device_info(torch):
    """GPU name and architecture, HIP version; clocks are the driver's (this
    program neither locks nor reads back a fixed clock)."""
    props = torch.cuda.get_device_properties(0)
    return {"name": torch.cuda.get_device_name(0),
            "arch": getattr(props, "gcnArchName", None),
            "compute_units": props.multi_processor_count,
            "hip": torch.version.hip, "torch": torch.__version__, "clocks_locked": False}


def dense_comparator(torch, P, wl, args, sparse_ms):
    """Same-shape dense causal attention (torch SDPA, flash backend only)."""
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel

        q = P["q"].view(1, wl.total_q, wl.n_heads_q, wl.head_dim).transpose(1, 2)
        k = P["k"].view(1, wl.total_k, wl.n_heads_kv, wl.head_dim).transpose(1, 2)
        v = P["v"].view(1, wl.total_k, wl.n_heads_kv, wl.head_dim).transpose(1, 2)
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        f = torch.nn.functional.scaled_dot_product_attention
        with sdpa_kernel([SDPBackend.FLASH_ATTENTION]):
            for _ in range(max(1, args.warmup)):
                f(q, k, v, is_causal=True, enable_gqa=True)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(args.steps):
                f(q, k, v, is_causal=True, enable_gqa=True)
            e1.record()
            torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        flops = wl.total_q * (wl.total_q + 1) / 2 * 4 * wl.n_heads_q * wl.head_dim
        roof_ms = flops / (PEAK_BF16_TFLOPS * 1e12) * 1e3
        return {"kind": "torch SDPA flash backend, causal, GQA", "ms": round(ms, 3),
                "tflops": round(flops / (ms / 1e3) / 1e12, 1),
                "sparse_over_dense_time": round(sparse_ms / ms, 3),
                "dense_mfma_roofline_ms": round(roof_ms, 3),
                "sparse_over_dense_mfma_roofline": round(sparse_ms / roof_ms, 3),
                "note": "sparse_over_dense_time uses the SDPA run as measured; "
                        "sparse_over_dense_mfma_roofline divides by the time dense causal "
                        "attention of this shape would take at the bf16 dense MFMA peak"}
    except Exception as exc:  # the comparator is context, not the product
        return {"kind": "torch SDPA flash backend", "error": repr(exc)[:300]}


if __name__ == "__main__":
    main()
