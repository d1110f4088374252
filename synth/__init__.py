"""Seeded synthetic workloads for the DSA hot path.

This package only draws inputs (see ``synth.c`` for the generator's published
definitions); it holds none of the method's arithmetic.  Both the CPU oracle
and the GPU library are fed from it: the GPU receives uploaded copies, so
both sides see identical bits.

bf16 tensors are returned as their uint16 bit patterns (numpy has no bf16).

Workloads (sizes and distributions; the pages measure on real long-video
data at 128K context with k = 2048, which these stand in for):

* ``prefill_2k_int``: one causal sequence of 2048 tokens, k = 256; attention
  8 query heads / 2 KV heads / dim 64; indexer 4 heads x 64 dims with integer
  qI, kI in [-3, 3] and integer w in [0, 3], so every indexer score is an
  integer and exact in fp32; Q, K, V ~ N(0, 1).
* ``prefill_32k`` / ``prefill_128k``: one causal sequence of 32768 / 131072
  tokens, k = 2048; attention 32 / 4 / 128; indexer 64 x 128.  qI, Q, V ~
  N(0, 1); kI and K are N(0, 1) noise plus a per-256-token-frame mean vector
  with N(0, 0.5^2) entries (independent per frame, and per KV head for K);
  w ~ U(0, 1).
* ``decode_b64_128k``: 64 sequences with 131072 cached tokens each, one new
  query per sequence (the new token already appended); all tensors N(0, 1),
  w ~ U(0, 1).
* ``varlen_512k``: packed prefill of 524288 tokens, lengths log-uniform in
  [4096, 262144] (multiples of 256, drawn in order until the total is reached,
  the last one cut to the remainder); shapes and distributions as
  ``prefill_32k``, plus 8 timestamp-like tokens at the start of every 256-token
  frame whose kI and K are scaled by 2.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass, field, replace

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# Stream ids (one independent counter stream per tensor).
S_QIDX, S_KIDX, S_W, S_Q, S_K, S_V, S_KIDX_MEAN, S_K_MEAN, S_LENGTHS, S_QIDX_MEAN = range(1, 11)


def build(verbose: bool = False) -> str:
    from . import build_lib as _b

    return _b.build(verbose=verbose)


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        build()
    lib = ctypes.CDLL(LIB_PATH)
    u64, i64, p, dbl = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p, ctypes.c_double
    lib.synth_stream_key.argtypes = [u64, u64]
    lib.synth_stream_key.restype = u64
    lib.synth_draw.argtypes = [u64, u64]
    lib.synth_draw.restype = u64
    lib.synth_bf16_from_double.argtypes = [dbl]
    lib.synth_bf16_from_double.restype = ctypes.c_uint16
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, dbl, p]
    lib.synth_normal_f64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_uniform_f32.argtypes = [u64, u64, u64, i64, dbl, dbl, p]
    lib.synth_uniform_f64.argtypes = [u64, u64, u64, i64, dbl, dbl, p]
    lib.synth_int_bf16.argtypes = [u64, u64, u64, i64, i64, i64, p]
    lib.synth_int_f32.argtypes = [u64, u64, u64, i64, i64, i64, p]
    lib.synth_clustered_bf16.argtypes = [u64, u64, u64, ctypes.c_int, p, i64, i64, dbl, i64,
                                         dbl, i64, i64, p]
    for f in (lib.synth_normal_bf16, lib.synth_normal_f64, lib.synth_uniform_f32,
              lib.synth_uniform_f64, lib.synth_int_bf16, lib.synth_int_f32,
              lib.synth_clustered_bf16):
        f.restype = None
    _lib = lib
    return lib


def _ptr(a: np.ndarray):
    return ctypes.c_void_p(a.ctypes.data)


# ---- raw streams -----------------------------------------------------------

def draws(seed: int, stream: int, start: int, count: int) -> np.ndarray:
    """Raw 64-bit SplitMix64 outputs of a stream (for tests of the generator)."""
    lib = _load()
    key = lib.synth_stream_key(seed, stream)
    return np.array([lib.synth_draw(key, start + i) for i in range(count)], dtype=np.uint64)


def normal_bf16(seed, stream, start, count, scale=1.0, out=None) -> np.ndarray:
    out = np.empty(count, np.uint16) if out is None else out
    _load().synth_normal_bf16(seed, stream, start, count, scale, _ptr(out))
    return out


def normal_f64(seed, stream, start, count) -> np.ndarray:
    out = np.empty(count, np.float64)
    _load().synth_normal_f64(seed, stream, start, count, _ptr(out))
    return out


def uniform_f32(seed, stream, start, count, lo=0.0, hi=1.0, out=None) -> np.ndarray:
    out = np.empty(count, np.float32) if out is None else out
    _load().synth_uniform_f32(seed, stream, start, count, lo, hi, _ptr(out))
    return out


def uniform_f64(seed, stream, start, count, lo=0.0, hi=1.0) -> np.ndarray:
    out = np.empty(count, np.float64)
    _load().synth_uniform_f64(seed, stream, start, count, lo, hi, _ptr(out))
    return out


def int_bf16(seed, stream, start, count, lo, hi, out=None) -> np.ndarray:
    out = np.empty(count, np.uint16) if out is None else out
    _load().synth_int_bf16(seed, stream, start, count, lo, hi, _ptr(out))
    return out


def int_f32(seed, stream, start, count, lo, hi, out=None) -> np.ndarray:
    out = np.empty(count, np.float32) if out is None else out
    _load().synth_int_f32(seed, stream, start, count, lo, hi, _ptr(out))
    return out


def bf16_bits_from_float(x) -> np.ndarray:
    """Round float values to bf16 (nearest-even), returning the uint16 bits."""
    f = np.ascontiguousarray(x, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r


def bf16_to_float(bits) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


# ---- workloads -------------------------------------------------------------

def draw_varlen_lengths(seed: int, total: int, lo: int, hi: int, multiple: int = 256):
    """Sequence lengths log-uniform in [lo, hi], rounded to `multiple`, drawn in
    order until `total` tokens are reached; the last length is cut to the
    remainder."""
    lens = []
    acc = 0
    i = 0
    while acc < total:
        u = uniform_f64(seed, S_LENGTHS, i, 1, math.log(lo), math.log(hi))[0]
        n = multiple * int(math.floor(math.exp(u) / multiple + 0.5))
        n = max(multiple, min(n, total - acc))
        lens.append(n)
        acc += n
        i += 1
    return lens


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    seqlens_q: tuple
    seqlens_k: tuple
    n_heads_q: int
    n_heads_kv: int
    head_dim: int
    n_heads_idx: int
    d_idx: int
    topk: int
    integer_indexer: bool = False
    clustered: bool = False
    ts_tokens: int = 0
    block: int = 256
    mean_std: float = 0.5
    ts_scale: float = 2.0
    # > 0: indexer queries get a per-(block, head) mean of this std, shared by
    # the block's tokens, so that adjacent queries select similar positions
    query_mean_std: float = 0.0
    notes: str = field(default="", compare=False)

    # -- layout ---------------------------------------------------------------
    @property
    def batch(self) -> int:
        return len(self.seqlens_q)

    @property
    def cu_q(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens_q)]).astype(np.int32)

    @property
    def cu_k(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens_k)]).astype(np.int32)

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))

    @property
    def max_seqlen_q(self) -> int:
        return int(max(self.seqlens_q))

    @property
    def max_seqlen_k(self) -> int:
        return int(max(self.seqlens_k))

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)

    # -- generation -------------------------------------------------------------
    def _rows(self, rows, per_row: int, fill):
        """Generate rows given as (start, stop) or an index array; `fill(start,
        count, out)` writes `count` elements of the flat stream from `start`."""
        if isinstance(rows, tuple):
            start, stop = rows
            out = np.empty((stop - start) * per_row, dtype=fill.dtype)
            fill(start * per_row, (stop - start) * per_row, out)
            return out
        rows = np.asarray(rows, dtype=np.int64)
        out = np.empty(rows.shape[0] * per_row, dtype=fill.dtype)
        for i, r in enumerate(rows):
            fill(int(r) * per_row, per_row, out[i * per_row:(i + 1) * per_row])
        return out

    def _n(self, rows) -> int:
        return (rows[1] - rows[0]) if isinstance(rows, tuple) else len(rows)

    def q_idx(self, rows=None) -> np.ndarray:
        rows = (0, self.total_q) if rows is None else rows
        per = self.n_heads_idx * self.d_idx
        if self.query_mean_std > 0 and not self.integer_indexer:
            spans = [rows] if isinstance(rows, tuple) else [(int(r), int(r) + 1) for r in rows]
            parts = []
            cu = self.cu_q  # kept alive across the calls
            for a, b in spans:
                out = np.empty((b - a) * per, np.uint16)
                _load().synth_clustered_bf16(self.seed, S_QIDX, S_QIDX_MEAN, self.batch, _ptr(cu),
                                             per, self.block, self.query_mean_std, 0, 1.0, a, b - a,
                                             _ptr(out))
                parts.append(out)
            return np.concatenate(parts).reshape(self._n(rows), self.n_heads_idx, self.d_idx)
        if self.integer_indexer:
            f = _Fill(np.uint16, lambda s, c, o: int_bf16(self.seed, S_QIDX, s, c, -3, 3, o))
        else:
            f = _Fill(np.uint16, lambda s, c, o: normal_bf16(self.seed, S_QIDX, s, c, 1.0, o))
        return self._rows(rows, per, f).reshape(self._n(rows), self.n_heads_idx, self.d_idx)

    def w(self, rows=None) -> np.ndarray:
        rows = (0, self.total_q) if rows is None else rows
        per = self.n_heads_idx
        if self.integer_indexer:
            f = _Fill(np.float32, lambda s, c, o: int_f32(self.seed, S_W, s, c, 0, 3, o))
        else:
            f = _Fill(np.float32, lambda s, c, o: uniform_f32(self.seed, S_W, s, c, 0.0, 1.0, o))
        return self._rows(rows, per, f).reshape(self._n(rows), self.n_heads_idx)

    def q(self, rows=None) -> np.ndarray:
        rows = (0, self.total_q) if rows is None else rows
        per = self.n_heads_q * self.head_dim
        f = _Fill(np.uint16, lambda s, c, o: normal_bf16(self.seed, S_Q, s, c, 1.0, o))
        return self._rows(rows, per, f).reshape(self._n(rows), self.n_heads_q, self.head_dim)

    def _clustered(self, noise_stream, mean_stream, row_len, start_tok, n_tok, out):
        cu = self.cu_k
        _load().synth_clustered_bf16(self.seed, noise_stream, mean_stream, self.batch, _ptr(cu),
                                     row_len, self.block, self.mean_std, self.ts_tokens,
                                     self.ts_scale, start_tok, n_tok, _ptr(out))

    def k_idx(self, tokens=None) -> np.ndarray:
        start, stop = (0, self.total_k) if tokens is None else tokens
        n = stop - start
        out = np.empty(n * self.d_idx, np.uint16)
        if self.integer_indexer:
            int_bf16(self.seed, S_KIDX, start * self.d_idx, n * self.d_idx, -3, 3, out)
        elif self.clustered:
            self._clustered(S_KIDX, S_KIDX_MEAN, self.d_idx, start, n, out)
        else:
            normal_bf16(self.seed, S_KIDX, start * self.d_idx, n * self.d_idx, 1.0, out)
        return out.reshape(n, self.d_idx)

    def k(self, tokens=None) -> np.ndarray:
        start, stop = (0, self.total_k) if tokens is None else tokens
        n = stop - start
        per = self.n_heads_kv * self.head_dim
        out = np.empty(n * per, np.uint16)
        if self.clustered:
            self._clustered(S_K, S_K_MEAN, per, start, n, out)
        else:
            normal_bf16(self.seed, S_K, start * per, n * per, 1.0, out)
        return out.reshape(n, self.n_heads_kv, self.head_dim)

    def v(self, tokens=None) -> np.ndarray:
        start, stop = (0, self.total_k) if tokens is None else tokens
        n = stop - start
        per = self.n_heads_kv * self.head_dim
        out = np.empty(n * per, np.uint16)
        normal_bf16(self.seed, S_V, start * per, n * per, 1.0, out)
        return out.reshape(n, self.n_heads_kv, self.head_dim)


class _Fill:
    def __init__(self, dtype, fn):
        self.dtype = dtype
        self.fn = fn

    def __call__(self, start, count, out):
        self.fn(start, count, out)


def _prefill(name, seed, lens, **kw) -> Workload:
    lens = tuple(int(x) for x in lens)
    return Workload(name=name, seed=seed, seqlens_q=lens, seqlens_k=lens, **kw)


_BIG = dict(n_heads_q=32, n_heads_kv=4, head_dim=128, n_heads_idx=64, d_idx=128, topk=2048)


def prefill_2k_int() -> Workload:
    return _prefill("prefill_2k_int", 1, [2048], n_heads_q=8, n_heads_kv=2, head_dim=64,
                    n_heads_idx=4, d_idx=64, topk=256, integer_indexer=True)


def prefill_32k() -> Workload:
    return _prefill("prefill_32k", 2, [32768], clustered=True, **_BIG)


def prefill_128k() -> Workload:
    return _prefill("prefill_128k", 3, [131072], clustered=True, **_BIG)


def prefill_128k_corr() -> Workload:
    """prefill_128k with correlated indexer queries: a per-(256-token block,
    head) mean of std 8 shared by the block's queries, so that 16 adjacent
    queries select about 7-10 K distinct positions between them (the page's
    figure for real data is about 8000) instead of 19-26 K."""
    return prefill_128k().with_(name="prefill_128k_corr", query_mean_std=8.0)


def decode_b64_128k() -> Workload:
    return Workload(name="decode_b64_128k", seed=4, seqlens_q=(1,) * 64,
                    seqlens_k=(131072,) * 64, **_BIG)


def varlen_512k() -> Workload:
    lens = draw_varlen_lengths(5, 524288, 4096, 262144)
    return _prefill("varlen_512k", 5, lens, clustered=True, ts_tokens=8, **_BIG)


WORKLOADS = {
    "prefill_2k_int": prefill_2k_int,
    "prefill_32k": prefill_32k,
    "prefill_128k": prefill_128k,
    "decode_b64_128k": decode_b64_128k,
    "varlen_512k": varlen_512k,
}


def get(name: str) -> Workload:
    return WORKLOADS[name]()
