"""Python binding of libdsa.so, the MI355X (gfx950) DSA hot path.

Argument marshalling only: every step of the path runs in the HIP kernels of
libdsa.so (see include/dsa.h for the contract of each entry point).  torch
supplies device memory and the stream; nothing here computes.  There is no
fallback: if libdsa.so is missing or fails to load, importing the entry
points raises.

Entry points (same names as the C ABI):
    dsa_index_scores, dsa_topk, dsa_topk_workspace_size,
    dsa_index_topk (+ workspace size; the indexer and top-k fused: no score rows),
    dsa_sparse_attn_prefill, dsa_sparse_attn_decode,
    dsa_sparse_attn_decode_workspace_size,
    dsa_quantize_fp8, dsa_index_scores_fp8 (the optional fp8 indexer),
    dsa_sparse_attn_prefill_grouped (+ workspace size; 16 adjacent rows per
    union of index sets),
    dsa_indexer_kl (the indexer's warm-up KL loss and its score gradient),
    dsa_sparse_attn_decode_noalloc (decode attention with the partials in the
    library's fixed per-GPU scratch, for callers that cannot allocate),
    dsa_check_varlen, dsa_check_indices, dsa_check_scores (device-side
    precondition checks; the entry points also run them when the environment
    variable DSA_CHECK is set to anything but "" or "0")
plus ``Varlen`` (the packed-batch descriptor) and ``DSAError``.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libdsa.so")

EXPORTED = (
    "dsa_status_string", "dsa_last_error", "dsa_index_scores", "dsa_topk_workspace_size",
    "dsa_topk", "dsa_sparse_attn_prefill", "dsa_sparse_attn_decode_workspace_size",
    "dsa_sparse_attn_decode", "dsa_check_varlen", "dsa_check_indices", "dsa_check_scores",
    "dsa_quantize_fp8", "dsa_index_scores_fp8", "dsa_sparse_attn_prefill_grouped_workspace_size",
    "dsa_sparse_attn_prefill_grouped", "dsa_indexer_kl", "dsa_sparse_attn_decode_noalloc",
    "dsa_index_topk_workspace_size", "dsa_index_topk",
    "dsa_index_scores_backward_workspace_size", "dsa_index_scores_backward",
)

DSA_OK = 0
DSA_ERR_INVALID_ARGUMENT = 1
DSA_ERR_UNSUPPORTED = 2
DSA_ERR_WORKSPACE = 3
DSA_ERR_HIP = 4


class DSAError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{_status_name(status)}: {message}")
        self.status = status


class dsa_varlen(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("total_q", ctypes.c_int64),
        ("total_k", ctypes.c_int64),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
    ]


_lib = None


def load_library(path: str = LIB_PATH):
    """Load libdsa.so (raises if it is not built: there is no other path)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"libdsa.so not built at {path}; run "
                          "`python -m long_context_sparse_score_amd.build_lib`")
    lib = ctypes.CDLL(path)
    vp, i32, i64, f32 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_float
    vl = ctypes.POINTER(dsa_varlen)
    sz = ctypes.POINTER(ctypes.c_size_t)
    lib.dsa_status_string.argtypes = [ctypes.c_int]
    lib.dsa_status_string.restype = ctypes.c_char_p
    lib.dsa_last_error.argtypes = []
    lib.dsa_last_error.restype = ctypes.c_char_p
    lib.dsa_index_scores.argtypes = [vl, vp, vp, vp, i32, i32, i64, i64, vp, i64, vp]
    lib.dsa_topk_workspace_size.argtypes = [vl, i64, i32, sz]
    lib.dsa_topk.argtypes = [vl, vp, i64, i64, i64, i32, vp, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_prefill.argtypes = [vl, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, f32,
                                            vp, vp, vp]
    lib.dsa_sparse_attn_decode_workspace_size.argtypes = [vl, i64, i32, i32, i32, sz]
    lib.dsa_sparse_attn_decode.argtypes = [vl, vp, vp, vp, vp, i32, i64, i64, i32, i32, i32, f32,
                                           vp, vp, vp, ctypes.c_size_t, vp]
    lib.dsa_sparse_attn_decode_noalloc.argtypes = [vl, vp, vp, vp, vp, i32, i64, i64, i32, i32,
                                                   i32, f32, vp, vp, vp]
    lib.dsa_index_topk_workspace_size.argtypes = [vl, i64, i32, sz]
    lib.dsa_index_topk.argtypes = [vl, vp, vp, vp, i32, i32, i64, i64, i32, vp, vp,
                                   ctypes.c_size_t, vp]
    lib.dsa_quantize_fp8.argtypes = [vp, i64, i32, vp, vp, vp]
    lib.dsa_index_scores_fp8.argtypes = [vl, vp, vp, vp, vp, vp, i32, i32, i64, i64, vp, i64, vp]
    lib.dsa_sparse_attn_prefill_grouped_workspace_size.argtypes = [vl, i64, i32, sz]
    lib.dsa_sparse_attn_prefill_grouped.argtypes = [vl, vp, vp, vp, vp, i32, i64, i64, i32, i32,
                                                    i32, f32, vp, vp, vp, ctypes.c_size_t, vp]
    lib.dsa_indexer_kl.argtypes = [vl, vp, vp, vp, i64, i64, i64, i32, i32, i32, f32, vp, vp,
                                   i64, vp]
    lib.dsa_index_scores_backward_workspace_size.argtypes = [vl, i32, i32, i64, i32, i32, sz]
    lib.dsa_index_scores_backward.argtypes = [vl, vp, vp, vp, i32, i32, i64, i64, vp, i64, vp, vp,
                                              vp, vp, ctypes.c_size_t, vp]
    lib.dsa_check_varlen.argtypes = [vl, vp]
    lib.dsa_check_indices.argtypes = [vl, vp, i32, i64, i64, vp]
    lib.dsa_check_scores.argtypes = [vl, vp, i64, i64, i64, vp]
    for name in EXPORTED[2:]:
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _status_name(status: int) -> str:
    try:
        return load_library().dsa_status_string(status).decode()
    except ImportError:
        return str(status)


def _check(status: int):
    if status != DSA_OK:
        raise DSAError(status, load_library().dsa_last_error().decode())


# ---- marshalling helpers -----------------------------------------------------

def _torch():
    import torch

    return torch


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _need(t, name, dtype, ndim=None):
    """Type, dtype, rank and contiguity of one tensor argument (the device is
    checked last, by _on_device, after the extents)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise TypeError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise TypeError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _on_device(**tensors):
    for name, t in tensors.items():
        if t is not None and not t.is_cuda:
            raise TypeError(f"{name} must be a device tensor")


# Extent checks: the C ABI addresses every buffer from the packed-batch
# descriptor and the window alone, so an undersized tensor would become an
# out-of-bounds device access.  These raise ValueError before any call.

def _extent(ok: bool, msg: str):
    if not ok:
        raise ValueError(msg)


def _window(vl, row_begin: int, row_count: int):
    _extent(row_begin >= 0 and row_count >= 0 and row_begin + row_count <= vl.total_q,
            f"row window [{row_begin}, {row_begin + row_count}) outside [0, {vl.total_q})")


def _rows(t, name: str, need: int):
    _extent(t.shape[0] >= need, f"{name} has {t.shape[0]} rows, the window needs {need}")


def _shape(t, name: str, want: tuple):
    _extent(tuple(t.shape) == tuple(want), f"{name} has shape {tuple(t.shape)}, expected {want}")


def _score_cols(t, name: str, vl):
    _extent(t.shape[1] >= vl.max_seqlen_k,
            f"{name} has {t.shape[1]} columns, fewer than max_seqlen_k = {vl.max_seqlen_k}")


def _scale(softmax_scale) -> float:
    """None selects the library's default scale (DSA_SCALE_DEFAULT = 0: the C
    ABI applies 1 / sqrt(head_dim)); the binding computes nothing."""
    return 0.0 if softmax_scale is None else float(softmax_scale)


def _stream(stream) -> int:
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


class Varlen:
    """Packed batch: cumulative query / key lengths on the device plus the host
    scalars the C ABI wants."""

    def __init__(self, cu_seqlens_q, cu_seqlens_k, device="cuda"):
        torch = _torch()
        cq = [int(x) for x in cu_seqlens_q]
        ck = [int(x) for x in cu_seqlens_k]
        if len(cq) != len(ck) or len(cq) < 2:
            raise ValueError("cu_seqlens_q and cu_seqlens_k need the same length >= 2")
        self.cu_q_host = cq
        self.cu_k_host = ck
        self.cu_q = torch.tensor(cq, dtype=torch.int32, device=device)
        self.cu_k = torch.tensor(ck, dtype=torch.int32, device=device)
        self.batch = len(cq) - 1
        self.total_q = cq[-1]
        self.total_k = ck[-1]
        self.max_seqlen_q = max(b - a for a, b in zip(cq, cq[1:]))
        self.max_seqlen_k = max(b - a for a, b in zip(ck, ck[1:]))
        self._struct = dsa_varlen(self.batch, self.cu_q.data_ptr(), self.cu_k.data_ptr(),
                                  self.total_q, self.total_k, self.max_seqlen_q, self.max_seqlen_k)

    @property
    def struct(self):
        return ctypes.byref(self._struct)


# ---- entry points ----------------------------------------------------------------

def dsa_index_scores(vl: Varlen, q_idx, k_idx, w, scores, row_begin: int = 0,
                     row_count: int | None = None, stream=None):
    """Indexer scores of rows [row_begin, row_begin + row_count) into scores
    (fp32 [row_count, ld]).  Columns beyond each row's position are untouched."""
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 2)
    _need(w, "w", torch.float32, 2)
    _need(scores, "scores", torch.float32, 2)
    row_count = scores.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    h, d = q_idx.shape[1], q_idx.shape[2]
    _shape(q_idx, "q_idx", (vl.total_q, h, d))
    _shape(k_idx, "k_idx", (vl.total_k, d))
    _shape(w, "w", (vl.total_q, h))
    _rows(scores, "scores", row_count)
    _score_cols(scores, "scores", vl)
    _on_device(q_idx=q_idx, k_idx=k_idx, w=w, scores=scores)
    _check(load_library().dsa_index_scores(
        vl.struct, _ptr(q_idx), _ptr(k_idx), _ptr(w), q_idx.shape[1], q_idx.shape[2], row_begin,
        row_count, _ptr(scores), scores.shape[1], _stream(stream)))


def dsa_index_topk_workspace_size(vl: Varlen, row_count: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_index_topk_workspace_size(vl.struct, row_count, k, ctypes.byref(n)))
    return n.value


def dsa_index_topk(vl: Varlen, q_idx, k_idx, w, indices, workspace, row_begin: int = 0,
                   row_count: int | None = None, stream=None):
    """Fused indexer scores -> top-k (k = indices.shape[1]) of rows
    [row_begin, row_begin + row_count) into indices (int32 [row_count, k]),
    without writing score rows; bitwise what dsa_index_scores -> dsa_topk give."""
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 2)
    _need(w, "w", torch.float32, 2)
    _need(indices, "indices", torch.int32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    row_count = indices.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    h, d = q_idx.shape[1], q_idx.shape[2]
    _shape(q_idx, "q_idx", (vl.total_q, h, d))
    _shape(k_idx, "k_idx", (vl.total_k, d))
    _shape(w, "w", (vl.total_q, h))
    _rows(indices, "indices", row_count)
    _on_device(q_idx=q_idx, k_idx=k_idx, w=w, indices=indices, workspace=workspace)
    _check(load_library().dsa_index_topk(
        vl.struct, _ptr(q_idx), _ptr(k_idx), _ptr(w), h, d, row_begin, row_count,
        indices.shape[1], _ptr(indices), _ptr(workspace), workspace.numel(), _stream(stream)))


def dsa_quantize_fp8(x, codes, scales, stream=None):
    """bf16 x [..., d] -> e4m3 codes (uint8, same shape) and one fp32 scale per
    vector of d values (scales shape x.shape[:-1])."""
    torch = _torch()
    _need(x, "x", torch.bfloat16)
    _need(codes, "codes", torch.uint8)
    _need(scales, "scales", torch.float32)
    d = x.shape[-1]
    if tuple(codes.shape) != tuple(x.shape) or tuple(scales.shape) != tuple(x.shape[:-1]):
        raise ValueError("codes must match x and scales must be x.shape[:-1]")
    _on_device(x=x, codes=codes, scales=scales)
    _check(load_library().dsa_quantize_fp8(_ptr(x), x.numel() // d, d, _ptr(codes), _ptr(scales),
                                           _stream(stream)))


def dsa_index_scores_fp8(vl: Varlen, q_codes, q_scales, k_codes, k_scales, w, scores,
                         row_begin: int = 0, row_count: int | None = None, stream=None):
    """Indexer scores from fp8 codes (q_codes uint8 [total_q, H, d], q_scales
    fp32 [total_q, H], k_codes uint8 [total_k, d], k_scales fp32 [total_k]) for
    rows [row_begin, row_begin + row_count) into scores (fp32 [row_count, ld])."""
    torch = _torch()
    _need(q_codes, "q_codes", torch.uint8, 3)
    _need(q_scales, "q_scales", torch.float32, 2)
    _need(k_codes, "k_codes", torch.uint8, 2)
    _need(k_scales, "k_scales", torch.float32, 1)
    _need(w, "w", torch.float32, 2)
    _need(scores, "scores", torch.float32, 2)
    row_count = scores.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    h, d = q_codes.shape[1], q_codes.shape[2]
    _shape(q_codes, "q_codes", (vl.total_q, h, d))
    _shape(q_scales, "q_scales", (vl.total_q, h))
    _shape(k_codes, "k_codes", (vl.total_k, d))
    _shape(k_scales, "k_scales", (vl.total_k,))
    _shape(w, "w", (vl.total_q, h))
    _rows(scores, "scores", row_count)
    _score_cols(scores, "scores", vl)
    _on_device(q_codes=q_codes, q_scales=q_scales, k_codes=k_codes, k_scales=k_scales, w=w,
               scores=scores)
    _check(load_library().dsa_index_scores_fp8(
        vl.struct, _ptr(q_codes), _ptr(q_scales), _ptr(k_codes), _ptr(k_scales), _ptr(w),
        q_codes.shape[1], q_codes.shape[2], row_begin, row_count, _ptr(scores), scores.shape[1],
        _stream(stream)))


def dsa_topk_workspace_size(vl: Varlen, row_count: int, k: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_topk_workspace_size(vl.struct, row_count, k, ctypes.byref(n)))
    return n.value


def dsa_topk(vl: Varlen, scores, indices, row_begin: int = 0, row_count: int | None = None,
             workspace=None, stream=None):
    """Per-row top-k (k = indices.shape[1]) into indices (int32 [row_count, k])."""
    torch = _torch()
    _need(scores, "scores", torch.float32, 2)
    _need(indices, "indices", torch.int32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    _rows(scores, "scores", row_count)
    _rows(indices, "indices", row_count)
    _score_cols(scores, "scores", vl)
    _on_device(scores=scores, indices=indices, workspace=workspace)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().dsa_topk(
        vl.struct, _ptr(scores), scores.shape[1], row_begin, row_count, indices.shape[1],
        _ptr(indices), _ptr(workspace), ws_bytes, _stream(stream)))


def _attn_extents(vl, q, k, v, indices, out, lse, row_begin, row_count, q_rows=None):
    hq, d = q.shape[1], q.shape[2]
    _window(vl, row_begin, row_count)
    _shape(q, "q", (vl.total_q if q_rows is None else q_rows, hq, d))
    _extent(k.shape[0] == vl.total_k and k.shape[2] == d,
            f"k has shape {tuple(k.shape)}, expected ({vl.total_k}, n_heads_kv, {d})")
    _shape(v, "v", tuple(k.shape))
    _rows(indices, "indices", row_count)
    _shape(out, "out", tuple(q.shape))
    if lse is not None:
        _shape(lse, "lse", (q.shape[0], hq))


def dsa_sparse_attn_prefill(vl: Varlen, q, k, v, indices, out, lse=None, softmax_scale=None,
                            row_begin: int = 0, row_count: int | None = None, stream=None):
    """Sparse GQA attention of rows [row_begin, row_begin + row_count) over
    indices (int32 [row_count, topk]) into out (bf16 [total_q, Hq, d])."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(indices, "indices", torch.int32, 2)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _attn_extents(vl, q, k, v, indices, out, lse, row_begin, row_count)
    _on_device(q=q, k=k, v=v, indices=indices, out=out, lse=lse)
    d = q.shape[2]
    _check(load_library().dsa_sparse_attn_prefill(
        vl.struct, _ptr(q), _ptr(k), _ptr(v), _ptr(indices), indices.shape[1], row_begin,
        row_count, q.shape[1], k.shape[1], d, _scale(softmax_scale), _ptr(out), _ptr(lse),
        _stream(stream)))


def dsa_sparse_attn_prefill_grouped_workspace_size(vl: Varlen, row_count: int, topk: int) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_sparse_attn_prefill_grouped_workspace_size(vl.struct, row_count, topk,
                                                                          ctypes.byref(n)))
    return n.value


def dsa_sparse_attn_prefill_grouped(vl: Varlen, q, k, v, indices, out, workspace, lse=None,
                                    softmax_scale=None, row_begin: int = 0,
                                    row_count: int | None = None, stream=None):
    """dsa_sparse_attn_prefill for groups of 16 adjacent rows served from the
    union of their (ascending) index rows."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(v, "v", torch.bfloat16, 3)
    _need(indices, "indices", torch.int32, 2)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _attn_extents(vl, q, k, v, indices, out, lse, row_begin, row_count)
    _on_device(q=q, k=k, v=v, indices=indices, out=out, lse=lse, workspace=workspace)
    d = q.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().dsa_sparse_attn_prefill_grouped(
        vl.struct, _ptr(q), _ptr(k), _ptr(v), _ptr(indices), indices.shape[1], row_begin,
        row_count, q.shape[1], k.shape[1], d, _scale(softmax_scale), _ptr(out), _ptr(lse),
        _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_indexer_kl(vl: Varlen, q, k, scores, loss, grad=None, softmax_scale=None,
                   row_begin: int = 0, row_count: int | None = None, stream=None):
    """Per-row KL divergence of the indexer's softmax (over the window's
    scores) from the head-averaged dense attention distribution, into loss
    [row_count]; with grad, also d loss / d scores (grad may be scores)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k, "k", torch.bfloat16, 3)
    _need(scores, "scores", torch.float32, 2)
    _need(loss, "loss", torch.float32, 1)
    if grad is not None:
        _need(grad, "grad", torch.float32, 2)
    row_count = scores.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    hq, d = q.shape[1], q.shape[2]
    _shape(q, "q", (vl.total_q, hq, d))
    _extent(k.shape[0] == vl.total_k and k.shape[2] == d,
            f"k has shape {tuple(k.shape)}, expected ({vl.total_k}, n_heads_kv, {d})")
    _rows(scores, "scores", row_count)
    _score_cols(scores, "scores", vl)
    _rows(loss, "loss", row_count)
    if grad is not None:
        _rows(grad, "grad", row_count)
        _score_cols(grad, "grad", vl)
    _on_device(q=q, k=k, scores=scores, loss=loss, grad=grad)
    _check(load_library().dsa_indexer_kl(
        vl.struct, _ptr(q), _ptr(k), _ptr(scores), scores.stride(0), row_begin, row_count,
        q.shape[1], k.shape[1], d, _scale(softmax_scale), _ptr(loss), _ptr(grad),
        0 if grad is None else grad.stride(0), _stream(stream)))


def dsa_index_scores_backward_workspace_size(vl: Varlen, n_heads_idx: int, d_idx: int,
                                             row_count: int, want_dq: bool = True,
                                             want_dk: bool = True) -> int:
    """Workspace bytes of a backward call over row_count rows."""
    n = ctypes.c_size_t(0)
    _check(load_library().dsa_index_scores_backward_workspace_size(
        vl.struct, n_heads_idx, d_idx, row_count, int(want_dq), int(want_dk), ctypes.byref(n)))
    return n.value


def dsa_index_scores_backward(vl: Varlen, q_idx, k_idx, w, grad, workspace, dq_idx=None, dw=None,
                              dk_idx=None, row_begin: int = 0, row_count: int | None = None,
                              stream=None):
    """Gradient of the indexer score for rows [row_begin, row_begin +
    row_count) given grad = d loss / d scores (fp32 [row_count, ld]): writes
    dq_idx (fp32 [row_count, H, d]) and dw (fp32 [row_count, H]) and adds the
    window's share of dk_idx (fp32 [total_k, d]); either group may be None."""
    torch = _torch()
    _need(q_idx, "q_idx", torch.bfloat16, 3)
    _need(k_idx, "k_idx", torch.bfloat16, 2)
    _need(w, "w", torch.float32, 2)
    _need(grad, "grad", torch.float32, 2)
    _need(workspace, "workspace", torch.uint8, 1)
    for t, name, nd in ((dq_idx, "dq_idx", 3), (dw, "dw", 2), (dk_idx, "dk_idx", 2)):
        if t is not None:
            _need(t, name, torch.float32, nd)
    row_count = grad.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    h, d = q_idx.shape[1], q_idx.shape[2]
    _shape(q_idx, "q_idx", (vl.total_q, h, d))
    _shape(k_idx, "k_idx", (vl.total_k, d))
    _shape(w, "w", (vl.total_q, h))
    _rows(grad, "grad", row_count)
    _score_cols(grad, "grad", vl)
    if dq_idx is not None:
        _extent(dq_idx.shape[0] >= row_count and tuple(dq_idx.shape[1:]) == (h, d),
                f"dq_idx has shape {tuple(dq_idx.shape)}, expected ({row_count}, {h}, {d})")
    if dw is not None:
        _extent(dw.shape[0] >= row_count and dw.shape[1] == h,
                f"dw has shape {tuple(dw.shape)}, expected ({row_count}, {h})")
    if dk_idx is not None:
        _shape(dk_idx, "dk_idx", (vl.total_k, d))
    _on_device(q_idx=q_idx, k_idx=k_idx, w=w, grad=grad, workspace=workspace, dq_idx=dq_idx,
               dw=dw, dk_idx=dk_idx)
    _check(load_library().dsa_index_scores_backward(
        vl.struct, _ptr(q_idx), _ptr(k_idx), _ptr(w), h, d, row_begin, row_count, _ptr(grad),
        grad.stride(0), _ptr(dq_idx), _ptr(dw), _ptr(dk_idx), _ptr(workspace), workspace.numel(),
        _stream(stream)))


def dsa_sparse_attn_decode_workspace_size(vl: Varlen, n_heads_q: int, head_dim: int,
                                          topk: int, row_count=None) -> int:
    """Workspace bytes of a decode call over row_count queries (default: all)."""
    n = ctypes.c_size_t(0)
    rc = vl.batch if row_count is None else row_count
    _check(load_library().dsa_sparse_attn_decode_workspace_size(vl.struct, rc, n_heads_q,
                                                                 head_dim, topk, ctypes.byref(n)))
    return n.value


def dsa_sparse_attn_decode(vl: Varlen, q, k_cache, v_cache, indices, out, workspace, lse=None,
                           softmax_scale=None, row_begin=0, row_count=None, stream=None):
    """Sparse GQA attention of one new token per sequence over its indices;
    indices[i] belongs to query row_begin + i."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(indices, "indices", torch.int32, 2)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _attn_extents(vl, q, k_cache, v_cache, indices, out, lse, row_begin, row_count,
                  q_rows=vl.batch)
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, indices=indices, out=out, lse=lse,
               workspace=workspace)
    d = q.shape[2]
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(load_library().dsa_sparse_attn_decode(
        vl.struct, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(indices), indices.shape[1],
        row_begin, row_count, q.shape[1], k_cache.shape[1], d, _scale(softmax_scale), _ptr(out),
        _ptr(lse), _ptr(workspace), ws_bytes, _stream(stream)))


def dsa_sparse_attn_decode_noalloc(vl: Varlen, q, k_cache, v_cache, indices, out, lse=None,
                                   softmax_scale=None, row_begin=0, row_count=None, stream=None):
    """dsa_sparse_attn_decode with the split partials in the library's fixed
    per-GPU scratch (no workspace, nothing allocated; calls that overlap on
    one GPU race on that scratch)."""
    torch = _torch()
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 3)
    _need(indices, "indices", torch.int32, 2)
    _need(out, "out", torch.bfloat16, 3)
    if lse is not None:
        _need(lse, "lse", torch.float32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _attn_extents(vl, q, k_cache, v_cache, indices, out, lse, row_begin, row_count,
                  q_rows=vl.batch)
    _on_device(q=q, k_cache=k_cache, v_cache=v_cache, indices=indices, out=out, lse=lse)
    _check(load_library().dsa_sparse_attn_decode_noalloc(
        vl.struct, _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(indices), indices.shape[1],
        row_begin, row_count, q.shape[1], k_cache.shape[1], q.shape[2], _scale(softmax_scale),
        _ptr(out), _ptr(lse), _stream(stream)))


def dsa_check_varlen(vl: Varlen, stream=None):
    """Device-side check of the packed-batch offsets (waits for the stream)."""
    _check(load_library().dsa_check_varlen(vl.struct, _stream(stream)))


def dsa_check_indices(vl: Varlen, indices, row_begin: int = 0, row_count: int | None = None,
                      stream=None):
    """Device-side check that every row of indices (int32 [row_count, topk]) is
    causal and free of repeats (waits for the stream)."""
    torch = _torch()
    _need(indices, "indices", torch.int32, 2)
    row_count = indices.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    _rows(indices, "indices", row_count)
    _on_device(indices=indices)
    _check(load_library().dsa_check_indices(vl.struct, _ptr(indices), indices.shape[1], row_begin,
                                            row_count, _stream(stream)))


def dsa_check_scores(vl: Varlen, scores, row_begin: int = 0, row_count: int | None = None,
                     stream=None):
    """Device-side check that columns 0..p of every score row are finite
    (waits for the stream)."""
    torch = _torch()
    _need(scores, "scores", torch.float32, 2)
    row_count = scores.shape[0] if row_count is None else row_count
    _window(vl, row_begin, row_count)
    _rows(scores, "scores", row_count)
    _score_cols(scores, "scores", vl)
    _on_device(scores=scores)
    _check(load_library().dsa_check_scores(vl.struct, _ptr(scores), scores.shape[1], row_begin,
                                           row_count, _stream(stream)))


def build(verbose: bool = False) -> str:
    from . import build_lib as _b

    return _b.build(verbose=verbose)
