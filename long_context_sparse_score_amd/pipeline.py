"""Orchestration of the DSA hot path over the C ABI (no arithmetic here).

Prefill walks the packed query rows in windows so that the fp32 score buffer
stays bounded: for each window it enqueues dsa_index_scores -> dsa_topk ->
dsa_sparse_attn_prefill on one stream.  Decode enqueues the same three steps
for one query per sequence.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import (Varlen, dsa_index_scores, dsa_sparse_attn_decode,
               dsa_sparse_attn_decode_workspace_size, dsa_sparse_attn_prefill, dsa_topk,
               dsa_topk_workspace_size)


def _torch():
    import torch

    return torch


def score_ld(max_seqlen_k: int) -> int:
    """Leading dimension of a score buffer: a multiple of 64 floats (256 B)."""
    return (max_seqlen_k + 63) // 64 * 64


@dataclass
class PrefillBuffers:
    scores: object   # fp32 [window, ld]
    indices: object  # int32 [window, topk]


def alloc_prefill(vl: Varlen, topk: int, window: int, device="cuda") -> PrefillBuffers:
    torch = _torch()
    window = max(1, min(window, vl.total_q))
    ld = score_ld(vl.max_seqlen_k)
    return PrefillBuffers(torch.empty((window, ld), dtype=torch.float32, device=device),
                          torch.empty((window, topk), dtype=torch.int32, device=device))


def prefill(vl: Varlen, q_idx, k_idx, w, q, k, v, out, bufs: PrefillBuffers, lse=None,
            softmax_scale=None, stream=None, keep_indices=None):
    """Whole prefill path; `keep_indices` (int32 [total_q, topk]) receives a copy
    of every window's selection when given (tests)."""
    window = bufs.scores.shape[0]
    for r0 in range(0, vl.total_q, window):
        n = min(window, vl.total_q - r0)
        dsa_index_scores(vl, q_idx, k_idx, w, bufs.scores, row_begin=r0, row_count=n,
                         stream=stream)
        dsa_topk(vl, bufs.scores, bufs.indices, row_begin=r0, row_count=n, stream=stream)
        dsa_sparse_attn_prefill(vl, q, k, v, bufs.indices, out, lse=lse,
                                softmax_scale=softmax_scale, row_begin=r0, row_count=n,
                                stream=stream)
        if keep_indices is not None:
            keep_indices[r0:r0 + n].copy_(bufs.indices[:n], non_blocking=True)


@dataclass
class DecodeBuffers:
    scores: object          # fp32 [batch, ld]
    indices: object         # int32 [batch, topk]
    groups: list            # (row_begin, row_count) of each row group
    workspaces: list        # per group: uint8 [bytes], decode attention partials
    topk_workspace: object  # uint8 [bytes] or None (the top-k needs none today)


def alloc_decode(vl: Varlen, n_heads_q: int, head_dim: int, topk: int, groups: int = 1,
                 device="cuda") -> DecodeBuffers:
    """Buffers of a decode step whose batch runs as `groups` contiguous row groups."""
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
    return DecodeBuffers(torch.empty((vl.batch, ld), dtype=torch.float32, device=device),
                         torch.empty((vl.batch, topk), dtype=torch.int32, device=device),
                         spans, wss,
                         torch.empty(tws, dtype=torch.uint8, device=device) if tws else None)


def decode(vl: Varlen, q_idx, k_idx_cache, w, q, k_cache, v_cache, out, bufs: DecodeBuffers,
           lse=None, softmax_scale=None, stream=None, side_stream=None):
    """One decode step: index scores -> top-k -> sparse attention per row group.

    The indexer streams the whole key cache and keeps HBM busy; the top-k and
    the attention of a group do not.  With a side stream the groups alternate
    between the two streams and each group's indexer waits only for the
    previous group's indexer, so a group's top-k and attention overlap the
    next group's indexer.  The step ends on `stream` (the current stream by
    default) after every group."""
    torch = _torch()
    main = torch.cuda.current_stream() if stream is None else stream
    streams = [main] if side_stream is None or len(bufs.groups) == 1 else [main, side_stream]
    if len(streams) > 1:
        side_stream.wait_stream(main)  # inputs written on the main stream
    prev_idx = None
    for i, (r0, n) in enumerate(bufs.groups):
        st = streams[i % len(streams)]
        if prev_idx is not None and len(streams) > 1:
            st.wait_event(prev_idx)
        dsa_index_scores(vl, q_idx, k_idx_cache, w, bufs.scores[r0:r0 + n], row_begin=r0,
                         row_count=n, stream=st)
        if len(streams) > 1:
            prev_idx = torch.cuda.Event()
            prev_idx.record(st)
        dsa_topk(vl, bufs.scores[r0:r0 + n], bufs.indices[r0:r0 + n], row_begin=r0, row_count=n,
                 workspace=bufs.topk_workspace, stream=st)
        dsa_sparse_attn_decode(vl, q, k_cache, v_cache, bufs.indices[r0:r0 + n], out,
                               bufs.workspaces[i], lse=lse, softmax_scale=softmax_scale,
                               row_begin=r0, row_count=n, stream=st)
    if len(streams) > 1:
        main.wait_stream(side_stream)
