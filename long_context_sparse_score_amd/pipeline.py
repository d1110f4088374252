"""Orchestration of the DSA hot path over the C ABI (no arithmetic here).

Prefill walks the packed query rows in windows so that the fp32 score buffer
stays bounded: for each window it enqueues dsa_index_scores -> dsa_topk ->
dsa_sparse_attn_prefill.  On one stream the three run in order; with a side
stream the attention of a window runs there while the next window's indexer
runs on the main stream (the indexer is bound by the matrix cores, the
attention by memory, so the two share the chip well).  Decode enqueues the
same three steps for one query per sequence.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import (Varlen, dsa_index_scores, dsa_index_scores_backward,
               dsa_index_scores_backward_workspace_size, dsa_index_scores_fp8, dsa_index_topk,
               dsa_index_topk_workspace_size, dsa_indexer_kl, dsa_quantize_fp8,
               dsa_sparse_attn_decode, dsa_sparse_attn_decode_workspace_size,
               dsa_sparse_attn_prefill, dsa_sparse_attn_prefill_grouped,
               dsa_sparse_attn_prefill_grouped_workspace_size, dsa_topk,
               dsa_topk_workspace_size)


def _torch():
    import torch

    return torch


@dataclass(frozen=True)
class PrefillConfig:
    """Launch shape of a windowed prefill.  BENCH_PREFILL is the one bench.py
    times by default; the full-size parity tests run the same object."""
    window: int = 8192      # query rows per score window (fp32 scores of one window in HBM)
    attn_rows: int = 1024   # rows per attention launch inside a window
    fused: bool = False     # dsa_index_topk instead of dsa_index_scores -> dsa_topk


BENCH_PREFILL = PrefillConfig()


def score_ld(max_seqlen_k: int) -> int:
    """Leading dimension of a score buffer: a multiple of 64 floats (256 B)."""
    return (max_seqlen_k + 63) // 64 * 64


@dataclass
class Fp8Indexer:
    """Indexer inputs as e4m3 codes with one scale per vector (the optional fp8
    indexer)."""
    q_codes: object   # uint8 [total_q, n_heads_idx, d_idx]
    q_scales: object  # fp32 [total_q, n_heads_idx]
    k_codes: object   # uint8 [total_k, d_idx]
    k_scales: object  # fp32 [total_k]


def alloc_fp8_indexer(total_q: int, total_k: int, n_heads_idx: int, d_idx: int,
                      device="cuda") -> Fp8Indexer:
    torch = _torch()
    return Fp8Indexer(
        torch.empty((total_q, n_heads_idx, d_idx), dtype=torch.uint8, device=device),
        torch.empty((total_q, n_heads_idx), dtype=torch.float32, device=device),
        torch.empty((total_k, d_idx), dtype=torch.uint8, device=device),
        torch.empty((total_k,), dtype=torch.float32, device=device))


def quantize_queries(q_idx, fp8: Fp8Indexer, stream=None):
    dsa_quantize_fp8(q_idx, fp8.q_codes, fp8.q_scales, stream=stream)


def quantize_keys(k_idx, fp8: Fp8Indexer, stream=None):
    dsa_quantize_fp8(k_idx, fp8.k_codes, fp8.k_scales, stream=stream)


def _scores(vl, q_idx, k_idx, w, scores, fp8, row_begin, row_count, stream):
    if fp8 is None:
        dsa_index_scores(vl, q_idx, k_idx, w, scores, row_begin=row_begin, row_count=row_count,
                         stream=stream)
    else:
        dsa_index_scores_fp8(vl, fp8.q_codes, fp8.q_scales, fp8.k_codes, fp8.k_scales, w, scores,
                             row_begin=row_begin, row_count=row_count, stream=stream)


@dataclass
class PrefillBuffers:
    scores: object       # fp32 [window, ld] (None when fused)
    indices: object      # int32 [window, topk]
    spare: object = None  # a second int32 [window, topk] for the two-stream schedule
    grouped: object = None  # uint8 workspace of the grouped attention (one per index buffer)
    grouped_spare: object = None
    fused: object = None  # uint8 workspace of dsa_index_topk (fused indexer -> top-k)
    window: int = 0


def alloc_prefill(vl: Varlen, topk: int, window: int, device="cuda", overlap: bool = False,
                  grouped: bool = False, fused: bool = False) -> PrefillBuffers:
    """Buffers of a windowed prefill; `overlap` adds the second index buffer the
    two-stream schedule alternates with; `grouped` selects the grouped attention
    (16 adjacent rows per union of index sets) and adds its workspace; `fused`
    selects dsa_index_topk (no score rows; its workspace instead)."""
    torch = _torch()
    window = max(1, min(window, vl.total_q))
    ld = score_ld(vl.max_seqlen_k)
    idx = lambda: torch.empty((window, topk), dtype=torch.int32, device=device)  # noqa: E731
    gws = lambda: torch.empty(  # noqa: E731
        max(256, dsa_sparse_attn_prefill_grouped_workspace_size(vl, window, topk)),
        dtype=torch.uint8, device=device)
    scores = None if fused else torch.empty((window, ld), dtype=torch.float32, device=device)
    fws = (torch.empty(dsa_index_topk_workspace_size(vl, window, topk), dtype=torch.uint8,
                       device=device) if fused else None)
    return PrefillBuffers(scores, idx(), idx() if overlap else None, gws() if grouped else None,
                          gws() if grouped and overlap else None, fws, window)


def prefill(vl: Varlen, q_idx, k_idx, w, q, k, v, out, bufs: PrefillBuffers, lse=None,
            softmax_scale=None, stream=None, keep_indices=None, side_stream=None, record=None,
            fp8: Fp8Indexer | None = None, attn_rows: int | None = None):
    """Whole prefill path.

    With `fp8` (buffers from alloc_fp8_indexer) the indexer queries and keys
    are first quantised into it and every window's scores come from the fp8
    indexer.

    With `side_stream` (and `bufs.spare`), window i's attention runs on the
    side stream and overlaps window i+1's indexer and top-k on the main
    stream; the top-k of window i waits until the attention of window i-2 has
    finished reading the index buffer they share.  The prefill ends on the
    main stream (`stream`, default the current one) after every window.
    `keep_indices` (int32 [total_q, topk]) receives every window's selection
    (tests).  `record`, a list, receives (row_begin, rows, events) per window,
    events being a dict of (start, end) timing-event pairs around each call:
    "index_scores" and "topk" on the main stream (the top-k pair starts after
    its wait for the index buffer), "sparse_attn" on the stream it runs on
    (starting after its wait for the top-k)."""
    torch = _torch()
    main = torch.cuda.current_stream() if stream is None else stream
    two = side_stream is not None and bufs.spare is not None
    att = side_stream if two else main
    if two:
        side_stream.wait_stream(main)  # inputs written on the main stream
    ibufs = [bufs.indices, bufs.spare] if two else [bufs.indices]
    gbufs = [bufs.grouped, bufs.grouped_spare] if two else [bufs.grouped]
    released = [None, None]  # per index buffer: attention done reading it
    window = bufs.window
    if fp8 is not None and bufs.fused is not None:
        raise ValueError("the fused indexer -> top-k takes bf16 indexer inputs")
    if fp8 is not None:
        quantize_queries(q_idx, fp8, stream=main)
        quantize_keys(k_idx, fp8, stream=main)

    def mark(st):
        if record is None:
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record(st)
        return e

    for i, r0 in enumerate(range(0, vl.total_q, window)):
        n = min(window, vl.total_q - r0)
        ib = ibufs[i % len(ibufs)]
        if bufs.fused is not None:
            # Fused: one call selects the window's indices (no score rows); its
            # time is reported as the indexer's and the top-k pair is empty.
            if two and released[i % 2] is not None:
                main.wait_event(released[i % 2])
            e0 = mark(main)
            dsa_index_topk(vl, q_idx, k_idx, w, ib[:n], bufs.fused, row_begin=r0, row_count=n,
                           stream=main)
            e1 = mark(main)
            t0 = t1 = e1
        else:
            e0 = mark(main)
            _scores(vl, q_idx, k_idx, w, bufs.scores, fp8, r0, n, main)
            e1 = mark(main)
            if two and released[i % 2] is not None:
                main.wait_event(released[i % 2])
            t0 = mark(main)
            dsa_topk(vl, bufs.scores, ib, row_begin=r0, row_count=n, stream=main)
            t1 = mark(main)
        if two:
            ready = torch.cuda.Event()
            ready.record(main)
            att.wait_event(ready)
        a0 = mark(att)
        if bufs.grouped is None:
            # `attn_rows` splits a window's attention into launches of that
            # many rows (same results; a timing knob).
            step = n if attn_rows is None else max(1, attn_rows)
            for j in range(0, n, step):
                m = min(step, n - j)
                dsa_sparse_attn_prefill(vl, q, k, v, ib[j:j + m], out, lse=lse,
                                        softmax_scale=softmax_scale, row_begin=r0 + j, row_count=m,
                                        stream=att)
        else:
            dsa_sparse_attn_prefill_grouped(vl, q, k, v, ib, out, gbufs[i % len(gbufs)], lse=lse,
                                            softmax_scale=softmax_scale, row_begin=r0,
                                            row_count=n, stream=att)
        a1 = mark(att)
        if keep_indices is not None:
            with torch.cuda.stream(att):
                keep_indices[r0:r0 + n].copy_(ib[:n], non_blocking=True)
        if two:
            released[i % 2] = torch.cuda.Event()
            released[i % 2].record(att)
        if record is not None:
            record.append((r0, n, {"index_scores": (e0, e1), "topk": (t0, t1),
                                   "sparse_attn": (a0, a1)}))
    if two:
        main.wait_stream(side_stream)


@dataclass
class DecodeBuffers:
    scores: object          # fp32 [batch, ld] (None when fused)
    indices: object         # int32 [batch, topk]
    groups: list            # (row_begin, row_count) of each row group
    workspaces: list        # per group: uint8 [bytes], decode attention partials
    topk_workspace: object  # uint8 [bytes] or None (the top-k needs none today)
    fused: list = None      # per group: uint8 workspace of dsa_index_topk


def alloc_decode(vl: Varlen, n_heads_q: int, head_dim: int, topk: int, groups: int = 1,
                 device="cuda", fused: bool = False) -> DecodeBuffers:
    """Buffers of a decode step whose batch runs as `groups` contiguous row
    groups; `fused` selects dsa_index_topk for the indexer and top-k."""
    torch = _torch()
    ld = score_ld(vl.max_seqlen_k)
    groups = max(1, min(groups, vl.batch))
    size = -(-vl.batch // groups)
    spans = [(r0, min(size, vl.batch - r0)) for r0 in range(0, vl.batch, size)]
    wss = []
    for _, n in spans:
        ws = dsa_sparse_attn_decode_workspace_size(vl, n_heads_q, head_dim, topk, row_count=n)
        wss.append(torch.empty(max(ws, 256), dtype=torch.uint8, device=device))
    tws = dsa_topk_workspace_size(vl, vl.batch, topk)
    fws = ([torch.empty(dsa_index_topk_workspace_size(vl, n, topk), dtype=torch.uint8,
                        device=device) for _, n in spans] if fused else None)
    return DecodeBuffers(None if fused else torch.empty((vl.batch, ld), dtype=torch.float32,
                                                        device=device),
                         torch.empty((vl.batch, topk), dtype=torch.int32, device=device),
                         spans, wss,
                         torch.empty(tws, dtype=torch.uint8, device=device) if tws else None, fws)


def decode(vl: Varlen, q_idx, k_idx_cache, w, q, k_cache, v_cache, out, bufs: DecodeBuffers,
           lse=None, softmax_scale=None, stream=None, side_stream=None,
           fp8: Fp8Indexer | None = None):
    """One decode step: index scores -> top-k -> sparse attention per row group.

    With `fp8`, the indexer key cache is the one held in fp8.k_codes /
    fp8.k_scales (quantised when its tokens were appended, see quantize_keys;
    k_idx_cache is not read) and the step quantises its new indexer queries.

    The indexer streams the whole key cache and keeps HBM busy; the top-k and
    the attention of a group do not.  With a side stream the groups alternate
    between the two streams and each group's indexer waits only for the
    previous group's indexer, so a group's top-k and attention overlap the
    next group's indexer.  The step ends on `stream` (the current stream by
    default) after every group."""
    torch = _torch()
    main = torch.cuda.current_stream() if stream is None else stream
    streams = [main] if side_stream is None or len(bufs.groups) == 1 else [main, side_stream]
    if fp8 is not None:
        quantize_queries(q_idx, fp8, stream=main)
    if len(streams) > 1:
        side_stream.wait_stream(main)  # inputs written on the main stream
    prev_idx = None
    if fp8 is not None and bufs.fused is not None:
        raise ValueError("the fused indexer -> top-k takes bf16 indexer inputs")
    for i, (r0, n) in enumerate(bufs.groups):
        st = streams[i % len(streams)]
        if prev_idx is not None and len(streams) > 1:
            st.wait_event(prev_idx)
        if bufs.fused is not None:
            dsa_index_topk(vl, q_idx, k_idx_cache, w, bufs.indices[r0:r0 + n], bufs.fused[i],
                           row_begin=r0, row_count=n, stream=st)
        else:
            _scores(vl, q_idx, k_idx_cache, w, bufs.scores[r0:r0 + n], fp8, r0, n, st)
        if len(streams) > 1:
            prev_idx = torch.cuda.Event()
            prev_idx.record(st)
        if bufs.fused is None:
            dsa_topk(vl, bufs.scores[r0:r0 + n], bufs.indices[r0:r0 + n], row_begin=r0,
                     row_count=n, workspace=bufs.topk_workspace, stream=st)
        dsa_sparse_attn_decode(vl, q, k_cache, v_cache, bufs.indices[r0:r0 + n], out,
                               bufs.workspaces[i], lse=lse, softmax_scale=softmax_scale,
                               row_begin=r0, row_count=n, stream=st)
    if len(streams) > 1:
        main.wait_stream(side_stream)


# ---------------------------------------------------------------- warm-up

# Query rows per window of the warm-up step: the KL kernel serves 16 rows per
# workgroup, so 8192 rows fill 512 workgroups (two per CU).
WARMUP_WINDOW = 8192


@dataclass
class WarmupBuffers:
    scores: object     # fp32 [window, ld]: a window's scores, then d loss / d scores over them
    workspace: object  # uint8: dsa_index_scores_backward's workspace for a full window
    window: int


def alloc_warmup(vl: Varlen, n_heads_idx: int, d_idx: int, window: int = WARMUP_WINDOW,
                 device="cuda") -> WarmupBuffers:
    torch = _torch()
    window = max(1, min(window, vl.total_q))
    scores = torch.empty((window, score_ld(vl.max_seqlen_k)), dtype=torch.float32, device=device)
    ws = torch.empty(max(1, dsa_index_scores_backward_workspace_size(vl, n_heads_idx, d_idx,
                                                                     window)),
                     dtype=torch.uint8, device=device)
    return WarmupBuffers(scores, ws, window)


def warmup(vl: Varlen, q_idx, k_idx, w, q, k, loss, dq_idx, dw, dk_idx, bufs: WarmupBuffers,
           softmax_scale=None, stream=None, record=None):
    """The indexer's step of the dense warm-up (page 5 section 1: the rest of
    the model frozen, the indexer trained so that its distribution over
    positions approaches the full attention's, measured by KL divergence).
    Per window of query rows: the indexer scores, the KL loss per row with
    its gradient written over the scores, then that gradient carried into
    the indexer's inputs.  loss (fp32 [total_q]), dq_idx (fp32 [total_q, H,
    d]) and dw (fp32 [total_q, H]) are written; dk_idx (fp32 [total_k, d]) is
    zeroed and then summed over the windows.  `record`, a list, receives
    (row_begin, rows, events) per window with (start, end) event pairs
    "index_scores", "indexer_kl" and "backward"."""
    torch = _torch()
    main = torch.cuda.current_stream() if stream is None else stream

    def mark():
        if record is None:
            return None
        e = torch.cuda.Event(enable_timing=True)
        e.record(main)
        return e

    with torch.cuda.stream(main):
        dk_idx.zero_()
    for r0 in range(0, vl.total_q, bufs.window):
        n = min(bufs.window, vl.total_q - r0)
        sc = bufs.scores[:n]
        e0 = mark()
        dsa_index_scores(vl, q_idx, k_idx, w, sc, row_begin=r0, row_count=n, stream=main)
        e1 = mark()
        dsa_indexer_kl(vl, q, k, sc, loss[r0:r0 + n], grad=sc, softmax_scale=softmax_scale,
                       row_begin=r0, row_count=n, stream=main)
        e2 = mark()
        dsa_index_scores_backward(vl, q_idx, k_idx, w, sc, bufs.workspace,
                                  dq_idx=dq_idx[r0:r0 + n], dw=dw[r0:r0 + n], dk_idx=dk_idx,
                                  row_begin=r0, row_count=n, stream=main)
        e3 = mark()
        if record is not None:
            record.append((r0, n, {"index_scores": (e0, e1), "indexer_kl": (e1, e2),
                                   "backward": (e2, e3)}))
