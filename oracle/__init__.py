"""CPU oracle for the DSA hot path (indexer scores -> top-k -> sparse GQA attention).

TEST INFRASTRUCTURE.  Only the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg may import this package.  The product library
(``long_context_sparse_score_amd``) never imports, links or calls it, and this
package never imports the product library: the two share no code.

The arithmetic lives in ``dsa_oracle.c`` (IEEE double loops, OpenMP over
query rows); this module only marshals numpy arrays into it.  Each function
cites the passage of the pages it follows ("Kwai Keye-VL-2.0 technical report"
summary, page 5, section 1: Lightning Indexer with one shared MQA key per
position, top-2048 selection, attention only over the selected positions,
one index set serving all GQA heads; section 8: deterministic top-k).

Parity status: every function here is pinned by ``tests/test_oracle_pins.py``
against brute force, closed forms, library routines and invariants.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(verbose: bool = False) -> str:
    """Compile dsa_oracle.c with gcc into liboracle.so (always recompiles)."""
    from . import build_lib as _b

    return _b.build(verbose=verbose)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_visible_counts.argtypes = [ctypes.c_int, p, p, i64, p, p]
    lib.oracle_index_scores.argtypes = [ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                        ctypes.c_int, i64, p, p, i64]
    lib.oracle_topk.argtypes = [i64, p, p, i64, ctypes.c_int, p]
    lib.oracle_sparse_attn.argtypes = [ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                       ctypes.c_int, ctypes.c_int, ctypes.c_double,
                                       i64, p, p, ctypes.c_int, p, p]
    lib.oracle_e4m3_value.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_value.restype = ctypes.c_double
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_double]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_quantize_fp8.argtypes = [p, i64, ctypes.c_int, p, p]
    lib.oracle_dequantize_fp8.argtypes = [p, p, i64, ctypes.c_int, p]
    lib.oracle_dequantize_fp8.restype = None
    lib.oracle_index_scores_f64.argtypes = [ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                            ctypes.c_int, i64, p, p, i64]
    lib.oracle_indexer_kl.argtypes = [ctypes.c_int, p, p, p, p, ctypes.c_int, ctypes.c_int,
                                      ctypes.c_int, ctypes.c_double, i64, p, p, i64, p, p]
    lib.oracle_index_scores_backward.argtypes = [ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                                 ctypes.c_int, i64, p, p, i64, p, p, p]
    lib.oracle_index_scores_backward_keys.argtypes = [ctypes.c_int, p, p, p, p, p, ctypes.c_int,
                                                      ctypes.c_int, i64, p, p, i64, p, p]
    for f in (lib.oracle_visible_counts, lib.oracle_index_scores, lib.oracle_topk,
              lib.oracle_sparse_attn, lib.oracle_quantize_fp8, lib.oracle_index_scores_f64,
              lib.oracle_indexer_kl, lib.oracle_index_scores_backward,
              lib.oracle_index_scores_backward_keys):
        f.restype = ctypes.c_int
    _lib = lib
    return lib


def _ptr(a: np.ndarray) -> ctypes.c_void_p:
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=dtype)


def _bf16_bits(a) -> np.ndarray:
    a = np.asarray(a)
    if a.dtype != np.uint16:
        raise TypeError("bf16 tensors are passed as their uint16 bit patterns")
    return np.ascontiguousarray(a)


def visible_counts(cu_q, cu_k, rows) -> np.ndarray:
    """p + 1 for each packed query row (the causal prefix it may attend to)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _c(rows, np.int64)
    out = np.empty(rows.shape[0], np.int64)
    if lib.oracle_visible_counts(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), rows.shape[0],
                                 _ptr(rows), _ptr(out)):
        raise ValueError("a row lies outside every sequence or before its keys")
    return out


def index_scores(cu_q, cu_k, q_idx, k_idx, w, rows, ld=None) -> np.ndarray:
    """Lightning-Indexer scores I[t, s] = sum_h w[t,h] * max(0, qI[t,h] . kI[s]).

    Page 5 section 1 (the scout scores every position with one shared MQA key);
    the weighted-ReLU form is the reading stated in the module header of
    dsa_oracle.c.  Returns float64 [len(rows), ld]; columns beyond the row's
    causal position are NaN.
    """
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    q_idx, k_idx = _bf16_bits(q_idx), _bf16_bits(k_idx)
    w = _c(w, np.float32)
    rows = _c(rows, np.int64)
    n_heads, d = q_idx.shape[1], q_idx.shape[2]
    if k_idx.shape[1] != d or w.shape[1] != n_heads:
        raise ValueError("indexer shapes disagree")
    if ld is None:
        ld = int(np.max(np.diff(cu_k)))
    out = np.empty((rows.shape[0], ld), np.float64)
    if lib.oracle_index_scores(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q_idx),
                               _ptr(k_idx), _ptr(w), n_heads, d, rows.shape[0], _ptr(rows),
                               _ptr(out), ld):
        raise ValueError("invalid row for the varlen layout")
    return out


# ---- fp8 indexer inputs (declared input transform; the pages state no indexer precision)

def e4m3_value(code: int) -> float:
    """Value of an OCP e4m3fn code (bias 7, 3 mantissa bits, no infinities,
    S.1111.111 = NaN)."""
    return _load().oracle_e4m3_value(int(code))


def e4m3_encode(y: float) -> int:
    """Nearest e4m3fn code: round to nearest, ties to even, saturating at 448."""
    return int(_load().oracle_e4m3_encode(float(y)))


def quantize_fp8(x):
    """Per-row fp8 quantisation of bf16 bits x [..., d]: codes (uint8, same
    shape) and scales (float32, shape x.shape[:-1]) with
    inv = 448 / max|x|, code = e4m3(x * inv), scale = max|x| / 448, each step
    in binary32 (all-zero rows: codes 0, scale 0)."""
    lib = _load()
    x = _bf16_bits(x)
    d = x.shape[-1]
    rows = x.size // d
    codes = np.empty(x.shape, np.uint8)
    scales = np.empty(x.shape[:-1], np.float32)
    if lib.oracle_quantize_fp8(_ptr(x), rows, d, _ptr(codes), _ptr(scales)):
        raise ValueError("non-finite input to the fp8 quantisation")
    return codes, scales


def dequantize_fp8(codes, scales) -> np.ndarray:
    """Represented values scale * e4m3_value(code) as float64 (exact)."""
    lib = _load()
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.float32)
    d = codes.shape[-1]
    if scales.shape != codes.shape[:-1]:
        raise ValueError("one scale per row of codes")
    out = np.empty(codes.shape, np.float64)
    lib.oracle_dequantize_fp8(_ptr(codes), _ptr(scales), codes.size // d, d, _ptr(out))
    return out


def index_scores_fp8(cu_q, cu_k, q_codes, q_scales, k_codes, k_scales, w, rows,
                     ld=None) -> np.ndarray:
    """The indexer score of index_scores() (page 5 section 1) evaluated in
    float64 on the values the fp8 inputs represent: queries scale[t, h] *
    value(code) per head, keys scale[s] * value(code)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _c(rows, np.int64)
    n_heads, d = q_codes.shape[1], q_codes.shape[2]
    if k_codes.shape[1] != d or w.shape[1] != n_heads:
        raise ValueError("indexer shapes disagree")
    q_rows = dequantize_fp8(np.asarray(q_codes)[rows], np.asarray(q_scales)[rows])
    k_all = dequantize_fp8(k_codes, k_scales)
    w = _c(w, np.float32)
    if ld is None:
        ld = int(np.max(np.diff(cu_k)))
    out = np.empty((rows.shape[0], ld), np.float64)
    if lib.oracle_index_scores_f64(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q_rows),
                                   _ptr(k_all), _ptr(w), n_heads, d, rows.shape[0], _ptr(rows),
                                   _ptr(out), ld):
        raise ValueError("invalid row for the varlen layout")
    return out


def topk(scores, counts, k: int) -> np.ndarray:
    """Deterministic top-k (page 5 section 1: k best positions per query;
    section 8: deterministic selection).  Order (score desc, position asc),
    output ascending positions padded with -1.  ``scores`` may be float32 or
    float64; float32 values convert to double exactly, so the order is the
    one float32 comparison gives."""
    lib = _load()
    scores = _c(scores, np.float64)
    counts = _c(counts, np.int64)
    out = np.empty((scores.shape[0], k), np.int32)
    if lib.oracle_topk(scores.shape[0], _ptr(counts), _ptr(scores), scores.shape[1], k,
                       _ptr(out)):
        raise ValueError("a row count is outside 1..ld")
    return out


def sparse_attn(cu_q, cu_k, q, k, v, idx, rows, scale: float):
    """Softmax attention of each query head restricted to the row's selected
    positions (page 5 section 1: attention only among the chosen positions;
    GQA head h reads KV head h // (Hq // Hkv), one index set for all heads).
    Returns (out float64 [n, Hq, d], lse float64 [n, Hq])."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    q, k, v = _bf16_bits(q), _bf16_bits(k), _bf16_bits(v)
    idx = _c(idx, np.int32)
    rows = _c(rows, np.int64)
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    if hq % hkv or k.shape != v.shape or k.shape[2] != d:
        raise ValueError("attention shapes disagree")
    n = rows.shape[0]
    out = np.empty((n, hq, d), np.float64)
    lse = np.empty((n, hq), np.float64)
    if lib.oracle_sparse_attn(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q), _ptr(k),
                              _ptr(v), hq, hkv, d, float(scale), n, _ptr(rows), _ptr(idx),
                              idx.shape[1], _ptr(out), _ptr(lse)):
        raise ValueError("invalid row or index outside the causal prefix")
    return out, lse


def indexer_kl(cu_q, cu_k, q, k, scores, rows, scale: float, want_grad: bool = True):
    """Indexer warm-up loss per query row (page 5 section 1, training stages:
    the dense warm-up trains the indexer so that its distribution over
    positions approaches the full attention's, the gap measured by KL
    divergence).  With P = the per-head dense softmax over the visible keys,
    averaged over query heads, and Pi = the softmax of the row's indexer
    scores: loss = KL(P || Pi) and grad = d loss / d I = Pi - P.
    scores: float [n, ld] for the listed rows (columns 0..p used).
    Returns (loss float64 [n], grad float64 [n, ld] or None; grad columns
    past p are 0)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    q, k = _bf16_bits(q), _bf16_bits(k)
    scores = _c(scores, np.float64)
    rows = _c(rows, np.int64)
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    if hq % hkv or k.shape[2] != d:
        raise ValueError("attention shapes disagree")
    n, ld = scores.shape
    if rows.shape[0] != n:
        raise ValueError("one score row per listed row")
    loss = np.empty(n, np.float64)
    grad = np.zeros((n, ld), np.float64) if want_grad else None
    if lib.oracle_indexer_kl(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q), _ptr(k), hq, hkv,
                             d, float(scale), n, _ptr(rows), _ptr(scores), ld, _ptr(loss),
                             _ptr(grad) if want_grad else None):
        raise ValueError("invalid row or score rows shorter than the causal prefix")
    return loss, grad


def _f64(x) -> np.ndarray:
    """bf16 bit patterns (uint16) widened exactly, or real values as float64."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return np.ascontiguousarray(x, dtype=np.float64)


def index_scores_f64(cu_q, cu_k, q_rows, k_idx, w, rows, ld=None) -> np.ndarray:
    """The indexer score of index_scores() on real-valued inputs: q_rows
    [len(rows), H, d] holds the listed rows' queries, k_idx [total_k, d] the
    keys (float64, or bf16 bits widened exactly)."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _c(rows, np.int64)
    q_rows, k_all = _f64(q_rows), _f64(k_idx)
    w = _c(w, np.float32)
    n_heads, d = q_rows.shape[1], q_rows.shape[2]
    if ld is None:
        ld = int(np.max(np.diff(cu_k)))
    out = np.empty((rows.shape[0], ld), np.float64)
    if lib.oracle_index_scores_f64(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q_rows),
                                   _ptr(k_all), _ptr(w), n_heads, d, rows.shape[0], _ptr(rows),
                                   _ptr(out), ld):
        raise ValueError("invalid row for the varlen layout")
    return out


def index_scores_backward(cu_q, cu_k, q_rows, k_idx, w, grad, rows):
    """Backward of the indexer score (page 5 section 1: the dense warm-up
    trains only the indexer, so its loss's gradient reaches the indexer's
    queries, keys and head weights).  grad [len(rows), ld] holds d L / d I
    for the listed rows (columns beyond a row's position are not read);
    q_rows [len(rows), H, d] the listed rows' queries, k_idx [total_k, d] the
    keys (float64, or bf16 bits widened exactly).  The ReLU's derivative is
    1 for x > 0 and 0 otherwise.  Returns (dq float64 [n, H, d], dw float64
    [n, H], dk float64 [total_k, d]); dk sums over the listed rows."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows = _c(rows, np.int64)
    q_rows, k_all = _f64(q_rows), _f64(k_idx)
    w = _c(w, np.float32)
    grad = _c(grad, np.float64)
    n, n_heads, d = q_rows.shape
    if grad.shape[0] != n or rows.shape[0] != n or k_all.shape[1] != d:
        raise ValueError("backward shapes disagree")
    dq = np.empty((n, n_heads, d), np.float64)
    dw = np.empty((n, n_heads), np.float64)
    dk = np.zeros((k_all.shape[0], d), np.float64)
    if lib.oracle_index_scores_backward(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q_rows),
                                        _ptr(k_all), _ptr(w), n_heads, d, n, _ptr(rows),
                                        _ptr(grad), grad.shape[1], _ptr(dq), _ptr(dw), _ptr(dk)):
        raise ValueError("invalid row or gradient rows shorter than the causal prefix")
    return dq, dw, dk


def index_scores_backward_keys(cu_q, cu_k, q_rows, k_idx, w, grad_at, rows, keys):
    """The key gradient of index_scores_backward() at the listed packed keys
    only: grad_at [len(rows), len(keys)] holds d L / d I at (row, key); the
    result dk [len(keys), d] sums over the listed rows that see each key."""
    lib = _load()
    cu_q, cu_k = _c(cu_q, np.int32), _c(cu_k, np.int32)
    rows, keys = _c(rows, np.int64), _c(keys, np.int64)
    q_rows, k_all = _f64(q_rows), _f64(k_idx)
    w = _c(w, np.float32)
    grad_at = _c(grad_at, np.float64)
    n, n_heads, d = q_rows.shape
    if grad_at.shape != (n, keys.shape[0]) or rows.shape[0] != n or k_all.shape[1] != d:
        raise ValueError("backward shapes disagree")
    dk = np.empty((keys.shape[0], d), np.float64)
    if lib.oracle_index_scores_backward_keys(len(cu_q) - 1, _ptr(cu_q), _ptr(cu_k), _ptr(q_rows),
                                             _ptr(k_all), _ptr(w), n_heads, d, n, _ptr(rows),
                                             _ptr(grad_at), keys.shape[0], _ptr(keys), _ptr(dk)):
        raise ValueError("invalid row or key")
    return dk


def dsa_rows(cu_q, cu_k, q_idx, k_idx, w, q, k, v, rows, topk_k: int, scale: float,
             ld=None):
    """The whole path for the given rows: scores -> top-k -> sparse attention.
    Returns dict(scores, counts, idx, out, lse)."""
    counts = visible_counts(cu_q, cu_k, rows)
    s = index_scores(cu_q, cu_k, q_idx, k_idx, w, rows, ld=ld)
    sel = topk(s, counts, topk_k)
    o, l = sparse_attn(cu_q, cu_k, q, k, v, sel, rows, scale)
    return {"scores": s, "counts": counts, "idx": sel, "out": o, "lse": l}
