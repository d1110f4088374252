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
    workspace: object       # uint8 [bytes], decode attention partials
    topk_workspace: object  # uint8 [bytes] or None, per-segment top-k candidates


def alloc_decode(vl: Varlen, n_heads_q: int, head_dim: int, topk: int,
                 device="cuda") -> DecodeBuffers:
    torch = _torch()
    ld = score_ld(vl.max_seqlen_k)
    ws = dsa_sparse_attn_decode_workspace_size(vl, n_heads_q, head_dim, topk)
    tws = dsa_topk_workspace_size(vl, vl.batch, topk)
    return DecodeBuffers(torch.empty((vl.batch, ld), dtype=torch.float32, device=device),
                         torch.empty((vl.batch, topk), dtype=torch.int32, device=device),
                         torch.empty(max(ws, 256), dtype=torch.uint8, device=device),
                         torch.empty(tws, dtype=torch.uint8, device=device) if tws else None)


def decode(vl: Varlen, q_idx, k_idx_cache, w, q, k_cache, v_cache, out, bufs: DecodeBuffers,
           lse=None, softmax_scale=None, stream=None):
    dsa_index_scores(vl, q_idx, k_idx_cache, w, bufs.scores, row_begin=0, row_count=vl.batch,
                     stream=stream)
    dsa_topk(vl, bufs.scores, bufs.indices, row_begin=0, row_count=vl.batch,
             workspace=bufs.topk_workspace, stream=stream)
    dsa_sparse_attn_decode(vl, q, k_cache, v_cache, bufs.indices, out, bufs.workspace, lse=lse,
                           softmax_scale=softmax_scale, stream=stream)
