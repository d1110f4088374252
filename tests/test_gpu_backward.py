"""The indexer backward (dsa_index_scores_backward) through the C ABI against
the oracle's fp64 gradient (page 5 section 1: the dense warm-up trains only
the indexer, so the loss's gradient must reach its queries, keys and head
weights).

Acceptance:
  * integer indexer inputs and an upstream gradient of multiples of 2^-8
    with |G| <= 4/256: every product and partial sum is exact in fp32 and
    every GEMM operand exact in bf16 (G, and w * qI <= 9), so dq, dw and dk
    must equal the oracle's exactly.
  * real-valued (bf16 normal) inputs: a bound derived from the arithmetic.
    dq and dk multiply G [x > 0] (and w qI) rounded to bf16, relative error
    2^-9 each, and accumulate in fp32 over at most a few thousand MFMA steps
    (relative error well below 2^-10 of the sum of magnitudes), so
      |dq - ref| <= |w| (2^-8 sum_s |G| |kI| + flips)
      |dk - ref| <= 2^-7 sum_t |G| sum_h |w| |qI| + flips
      |dw - ref| <= 2^-8 sum_s |G| |x| + 2^-10 sum_s |G| sum_j |qI| |kI|
    (dw = qI . the dq sum before the weight, so it carries the bf16 rounding
    of G and the fp32 accumulation of that sum), where "flips" adds the
    terms whose mask the GPU may decide differently:
    those with |x| within the fp32 dot-product bound d 2^-24 sum_j |qI kI|
    of zero (taken generously as 2^-17 sum_j |qI kI|).
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import device_workload, log, to_dev, to_dev_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402


def positions(wl):
    return np.concatenate([np.arange(L) + (lk - L) for L, lk in zip(wl.seqlens_q, wl.seqlens_k)])


def run_backward(vl, dev, grad_dev, hi, di, windows, want_dq=True, want_dk=True):
    """The backward over the given row windows: dq, dw of every window row,
    dk summed over the windows."""
    total_q = vl.total_q
    dq = torch.full((total_q, hi, di), float("nan"), device="cuda") if want_dq else None
    dw = torch.full((total_q, hi), float("nan"), device="cuda") if want_dq else None
    dk = torch.zeros((vl.total_k, di), device="cuda") if want_dk else None
    for r0, n in windows:
        ws = torch.empty(max(1, dsa.dsa_index_scores_backward_workspace_size(
            vl, hi, di, n, want_dq, want_dk)), dtype=torch.uint8, device="cuda")
        dsa.dsa_index_scores_backward(vl, dev["q_idx"], dev["k_idx"], dev["w"], grad_dev[r0:r0 + n],
                                      ws, dq_idx=None if dq is None else dq[r0:r0 + n],
                                      dw=None if dw is None else dw[r0:r0 + n], dk_idx=dk,
                                      row_begin=r0, row_count=n)
    torch.cuda.synchronize()
    return (None if dq is None else dq.cpu().numpy(), None if dw is None else dw.cpu().numpy(),
            None if dk is None else dk.cpu().numpy())


def windows_of(total, size):
    return [(r0, min(size, total - r0)) for r0 in range(0, total, size)]


def grad_softmax_diff(wl, ld, seed):
    """A realistic upstream gradient: per row, the difference of two softmax
    distributions over the visible keys (sums to zero, like Pi - P)."""
    rng = np.random.default_rng(seed)
    pos = positions(wl)
    g = np.zeros((wl.total_q, ld), np.float32)
    for t, p in enumerate(pos):
        a, b = rng.normal(0, 2, p + 1), rng.normal(0, 2, p + 1)
        ea, eb = np.exp(a - a.max()), np.exp(b - b.max())
        g[t, :p + 1] = (ea / ea.sum() - eb / eb.sum()).astype(np.float32)
    return g


def garbage_beyond(g, wl):
    """Columns past each row's position hold NaN: they must never be read."""
    g = g.copy()
    for t, p in enumerate(positions(wl)):
        g[t, p + 1:] = np.nan
    return g


@pytest.mark.parametrize("hi,di", [(4, 64), (64, 128), (20, 128), (40, 64)])
def test_backward_integer_exact(hi, di):
    """Integer qI, kI (-3..3) and w (0..3), G = multiples of 2^-8 in
    [-4/256, 4/256]: bitwise the oracle's gradients.  Ragged varlen batch,
    windows that split sequences and 4-row blocks."""
    wl = synth.Workload(name="bwd_int", seed=41 + hi, seqlens_q=(700, 1, 333, 1100),
                        seqlens_k=(700, 1, 333, 1100), n_heads_q=8, n_heads_kv=2, head_dim=64,
                        n_heads_idx=hi, d_idx=di, topk=256, integer_indexer=True)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    ld = pipeline.score_ld(vl.max_seqlen_k)
    rng = np.random.default_rng(7)
    g = (rng.integers(-4, 5, (wl.total_q, ld)) / 256.0).astype(np.float32)
    g = garbage_beyond(g, wl)
    dq, dw, dk = run_backward(vl, dev, to_dev(g), hi, di, windows_of(wl.total_q, 601))
    rows = np.arange(wl.total_q)
    q_rows = host["q_idx"].reshape(wl.total_q, hi, di)
    rq, rw, rk = oracle.index_scores_backward(wl.cu_q, wl.cu_k, q_rows, host["k_idx"], host["w"],
                                              np.nan_to_num(g, nan=0.0), rows)
    assert np.array_equal(dq, rq.astype(np.float32)), f"dq: max |diff| {np.abs(dq - rq).max()}"
    assert np.array_equal(dw, rw.astype(np.float32)), f"dw: max |diff| {np.abs(dw - rw).max()}"
    assert np.array_equal(dk, rk.astype(np.float32)), f"dk: max |diff| {np.abs(dk - rk).max()}"


def tolerances(wl, host, g, rows, hi, di):
    """The derived bounds (module docstring) for the listed rows and every key."""
    qf = synth.bf16_to_float(host["q_idx"]).astype(np.float64).reshape(wl.total_q, hi, di)
    kf = synth.bf16_to_float(host["k_idx"]).astype(np.float64)
    w = host["w"].astype(np.float64)
    pos = positions(wl)
    tq = np.zeros((len(rows), hi, di))
    tw = np.zeros((len(rows), hi))
    tk = np.zeros((wl.total_k, di))
    seq_of = np.searchsorted(wl.cu_q, rows, side="right") - 1
    for i, t in enumerate(rows):
        b = seq_of[i]
        k0 = wl.cu_k[b]
        p = pos[t]
        keys = kf[k0:k0 + p + 1]                      # [p+1, d]
        gt = np.abs(g[i, :p + 1].astype(np.float64))  # [p+1]
        x = qf[t] @ keys.T                            # [H, p+1]
        xabs = np.abs(qf[t]) @ np.abs(keys).T         # [H, p+1]
        near = np.abs(x) <= 2.0 ** -17 * xabs
        tq[i] = np.abs(w[t])[:, None] * (2.0 ** -8 * (gt @ np.abs(keys))[None, :]
                                         + (near * gt[None, :]) @ np.abs(keys))
        tw[i] = 2.0 ** -8 * (np.abs(x) @ gt) + 2.0 ** -10 * (xabs @ gt)
        wq = np.abs(w[t])[:, None] * np.abs(qf[t])    # [H, d]
        tk[k0:k0 + p + 1] += 2.0 ** -7 * gt[:, None] * wq.sum(0)[None, :] \
            + (near.T * gt[:, None]) @ wq
    return tq, tw, tk


@pytest.mark.parametrize("grad_kind", ["softmax_diff", "normal"])
def test_backward_real_within_derived_bound(grad_kind):
    """bf16 normal indexer inputs (64 x 128), ragged varlen, NaN beyond each
    row's position: dq, dw, dk within the derived bounds of the oracle."""
    wl = synth.Workload(name="bwd_real", seed=45, seqlens_q=(700, 1, 333, 1100),
                        seqlens_k=(700, 1, 333, 1100), n_heads_q=8, n_heads_kv=2, head_dim=64,
                        n_heads_idx=64, d_idx=128, topk=256)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    ld = pipeline.score_ld(vl.max_seqlen_k)
    if grad_kind == "normal":
        g = np.random.default_rng(8).normal(0, 1, (wl.total_q, ld)).astype(np.float32)
    else:
        g = grad_softmax_diff(wl, ld, 9)
    g = garbage_beyond(g, wl)
    dq, dw, dk = run_backward(vl, dev, to_dev(g), 64, 128, windows_of(wl.total_q, 512))
    rows = np.arange(wl.total_q)
    g0 = np.nan_to_num(g, nan=0.0)
    q_rows = host["q_idx"].reshape(wl.total_q, 64, 128)
    rq, rw, rk = oracle.index_scores_backward(wl.cu_q, wl.cu_k, q_rows, host["k_idx"], host["w"],
                                              g0, rows)
    tq, tw, tk = tolerances(wl, host, g0, rows, 64, 128)
    for name, got, ref, tol in (("dq", dq, rq, tq), ("dw", dw, rw, tw), ("dk", dk, rk, tk)):
        err = np.abs(got.astype(np.float64) - ref)
        assert np.isfinite(got).all(), f"{name}: non-finite values"
        bad = err > tol + 1e-30
        log(f"  {name}: max err {err.max():.3e}, max err / bound {np.max(err / (tol + 1e-30)):.3f}")
        assert not bad.any(), f"{name}: {bad.sum()} entries beyond the bound, first at " \
                              f"{np.argwhere(bad)[0]}"


def test_backward_outputs_independent():
    """dq/dw alone and dk alone equal the combined call; dk accumulates over
    calls (two passes give twice one pass)."""
    wl = synth.Workload(name="bwd_sep", seed=46, seqlens_q=(1500, 600), seqlens_k=(1500, 600),
                        n_heads_q=8, n_heads_kv=2, head_dim=64, n_heads_idx=64, d_idx=128,
                        topk=256, integer_indexer=True)
    _, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    ld = pipeline.score_ld(vl.max_seqlen_k)
    g = to_dev((np.random.default_rng(10).integers(-4, 5, (wl.total_q, ld)) / 256.0)
               .astype(np.float32))
    win = windows_of(wl.total_q, 1024)
    dq, dw, dk = run_backward(vl, dev, g, 64, 128, win)
    dq1, dw1, _ = run_backward(vl, dev, g, 64, 128, win, want_dk=False)
    _, _, dk1 = run_backward(vl, dev, g, 64, 128, win, want_dq=False)
    _, _, dk2 = run_backward(vl, dev, g, 64, 128, win + win, want_dq=False)
    assert np.array_equal(dq, dq1) and np.array_equal(dw, dw1) and np.array_equal(dk, dk1)
    assert np.array_equal(dk2, 2 * dk1)


def test_backward_decode_shape():
    """Decode-shaped batch (one query per sequence, caches of ragged length):
    rows of different sequences share 4-row blocks."""
    lk = [1, 31, 32, 33, 255, 256, 257, 5000]
    wl = synth.Workload(name="bwd_dec", seed=47, seqlens_q=(1,) * len(lk), seqlens_k=tuple(lk),
                        n_heads_q=8, n_heads_kv=2, head_dim=64, n_heads_idx=64, d_idx=128,
                        topk=256, integer_indexer=True)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    ld = pipeline.score_ld(vl.max_seqlen_k)
    g = (np.random.default_rng(11).integers(-4, 5, (wl.total_q, ld)) / 256.0).astype(np.float32)
    g = garbage_beyond(g, wl)
    dq, dw, dk = run_backward(vl, dev, to_dev(g), 64, 128, [(0, wl.total_q)])
    rows = np.arange(wl.total_q)
    q_rows = host["q_idx"].reshape(wl.total_q, 64, 128)
    rq, rw, rk = oracle.index_scores_backward(wl.cu_q, wl.cu_k, q_rows, host["k_idx"], host["w"],
                                              np.nan_to_num(g, nan=0.0), rows)
    assert np.array_equal(dq, rq.astype(np.float32))
    assert np.array_equal(dw, rw.astype(np.float32))
    assert np.array_equal(dk, rk.astype(np.float32))
