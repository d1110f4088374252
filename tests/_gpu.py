"""Helpers shared by the GPU parity tests (host-side marshalling and the
acceptance rules; no arithmetic of the method)."""
from __future__ import annotations

import sys

import numpy as np

import oracle
import synth

# Acceptance bars for bf16 inputs with fp32 accumulation.
ATTN_MAX_ABS = 2e-2
ATTN_MEAN_ABS = 2e-3
TOPK_REL = 1e-3  # disagreements allowed only within this relative band of the k-th score


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev_bf16(bits: np.ndarray):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def to_dev(a: np.ndarray):
    import torch

    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda")


def from_dev_bf16(t) -> np.ndarray:
    import torch

    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def device_workload(wl: synth.Workload, parts=("q_idx", "k_idx", "w", "q", "k", "v")):
    """Generate a workload on the host and upload it.  Returns (host, device)."""
    host, dev = {}, {}
    for p in parts:
        a = getattr(wl, p)()
        host[p] = a
        dev[p] = to_dev(a) if p == "w" else to_dev_bf16(a)
    return host, dev


def sample_rows(total: int, k: int, n_random: int, seed: int):
    """Stratified rows: the first, around k, the last, plus seeded random rows."""
    fixed = {0, 1, k - 2, k - 1, k, k + 1, total // 2, total - 2, total - 1}
    rng = np.random.default_rng(seed)
    rnd = set(rng.integers(0, total, size=n_random).tolist())
    return np.array(sorted(r for r in fixed | rnd if 0 <= r < total), dtype=np.int64)


def check_topk_rows(gpu_idx, ora_idx, ora_scores, counts, k):
    """Top-k acceptance per row.  Returns a bool array: sets identical."""
    same = np.zeros(len(counts), bool)
    for i, cnt in enumerate(counts):
        n = min(k, int(cnt))
        g = gpu_idx[i]
        assert (g[n:] == -1).all(), f"row {i}: padding"
        sel = g[:n]
        assert (sel >= 0).all() and (sel < cnt).all(), f"row {i}: non-causal index"
        assert (np.diff(sel) > 0).all(), f"row {i}: not strictly ascending"
        o = ora_idx[i, :n]
        if np.array_equal(sel, o):
            same[i] = True
            continue
        vis = ora_scores[i, :cnt]
        tau = np.sort(vis)[::-1][n - 1]
        diff = np.setxor1d(sel, o)
        dev = np.abs(vis[diff] - tau)
        assert (dev <= TOPK_REL * abs(tau)).all(), (
            f"row {i}: index disagreement outside the tie band: positions {diff[:8]}, "
            f"|I - tau| = {dev[:8]}, tau = {tau}")
    return same


def check_attn(gpu_out_bits, ora_out, rows_mask=None, what="attention"):
    g = synth.bf16_to_float(gpu_out_bits).astype(np.float64)
    if rows_mask is not None:
        g, o = g[rows_mask], ora_out[rows_mask]
    else:
        o = ora_out
    if g.size == 0:
        return 0.0, 0.0
    err = np.abs(g - o)
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= ATTN_MAX_ABS, f"{what}: max abs error {mx}"
    assert mean <= ATTN_MEAN_ABS, f"{what}: mean abs error {mean}"
    return mx, mean


def check_attn_every_row(wl, host, rows, got_idx, same, got_out_bits, got_lse, ref,
                         what="attention"):
    """Attention and lse on EVERY sampled row.  Where the GPU's index set
    equals the oracle's, the reference is the oracle's own result; where it
    differs (only inside the tie band, checked by check_topk_rows), the
    reference is the oracle's attention over the GPU's own index row, so no
    row goes unchecked.  Returns (max abs, mean abs, rows with the GPU's
    indices)."""
    ref_out = np.array(ref["out"], copy=True)
    ref_lse = np.array(ref["lse"], copy=True)
    diff = np.flatnonzero(~np.asarray(same))
    if len(diff):
        o, l = oracle.sparse_attn(wl.cu_q, wl.cu_k, host["q"], host["k"], host["v"],
                                  np.ascontiguousarray(got_idx[diff]), np.asarray(rows)[diff],
                                  wl.softmax_scale)
        ref_out[diff] = o
        ref_lse[diff] = l
    mx, mean = check_attn(got_out_bits, ref_out, what=what)
    fin = np.isfinite(ref_lse)
    assert (np.isfinite(got_lse) == fin).all(), f"{what}: lse finiteness differs"
    err = np.abs(got_lse[fin] - ref_lse[fin])
    assert err.size == 0 or err.max() <= 2e-3, f"{what}: lse error {err.max()}"
    return mx, mean, len(diff)


def oracle_rows(wl: synth.Workload, host, rows):
    """Oracle scores / top-k / attention for the given packed rows."""
    return oracle.dsa_rows(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"], host["q"],
                           host["k"], host["v"], rows, wl.topk, wl.softmax_scale)
