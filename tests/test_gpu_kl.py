"""GPU parity of dsa_indexer_kl (the indexer's warm-up KL loss and its score
gradient) against the CPU oracle, through the C ABI.

Tolerances, from the arithmetic: the dense logits are fp32 sums of exact
bf16 products (relative error about d * 2^-24 of sum |q k|), the softmax
statistics fp32 sums; P and Pi then carry relative errors of order 1e-5,
so the per-row loss sum_s P (ln P - ln Pi) is held to 1e-3 (1 + loss) and the
gradient Pi - P to 1e-4 max(P, Pi) + 1e-7 per element."""
import math

import numpy as np
import pytest

import oracle
import synth

from _gpu import device_workload, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402


def small_wl(lq, lk, hq, hkv, d, seed=21):
    return synth.Workload(name="test", seed=seed, seqlens_q=tuple(lq), seqlens_k=tuple(lk),
                          n_heads_q=hq, n_heads_kv=hkv, head_dim=d, n_heads_idx=4, d_idx=64,
                          topk=64, clustered=True)


def check(loss_g, grad_g, loss_o, grad_o, counts, scores):
    dl = np.abs(loss_g - loss_o)
    assert (dl <= 1e-3 * (1 + np.abs(loss_o))).all(), f"loss: worst {dl.max():.3e}"
    for i, n in enumerate(counts):
        g, o = grad_g[i, :n], grad_o[i, :n]
        # the element's scale: max(Pi, P), Pi the softmax of the row's scores
        x = scores[i, :n].astype(np.float64)
        pi = np.exp(x - x.max())
        pi /= pi.sum()
        mag = np.maximum(pi, pi - o)
        bad = np.abs(g - o) > 1e-4 * mag + 1e-7
        assert not bad.any(), f"row {i}: grad off at {np.flatnonzero(bad)[:5]}"
    return float(dl.max())


def run(wl, dev, scores_np, row_begin=0, in_place=False, ld=None):
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    n = scores_np.shape[0]
    ld = ld or scores_np.shape[1]
    sc = torch.zeros((n, ld), dtype=torch.float32, device="cuda")
    sc[:, :scores_np.shape[1]] = to_dev(scores_np.astype(np.float32))
    loss = torch.full((n,), -7.0, dtype=torch.float32, device="cuda")
    grad = sc if in_place else torch.full((n, ld), 5.0, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl(vl, dev["q"], dev["k"], sc, loss, grad=grad, row_begin=row_begin,
                       row_count=n)
    torch.cuda.synchronize()
    return loss.cpu().numpy(), grad.cpu().numpy()


@pytest.mark.parametrize("hq,hkv,d", [(32, 4, 128), (8, 2, 64), (16, 8, 64), (1, 1, 128),
                                      (64, 8, 128), (4, 4, 128), (2, 1, 64)])
def test_kl_matches_oracle_varlen(hq, hkv, d):
    """Sequences of several lengths (a workgroup of 16 rows spans several of
    them), a one-row sequence, rows longer than many key tiles."""
    wl = small_wl([37, 100, 1, 250], [60, 100, 5, 250], hq, hkv, d, seed=hq + d)
    host, dev = device_workload(wl, parts=("q", "k"))
    ld = 256
    rng = np.random.default_rng(hq * 7 + d)
    scores = (rng.standard_normal((wl.total_q, ld)) * 3).astype(np.float32)
    rows = np.arange(wl.total_q)
    log(f"indexer KL hq={hq} hkv={hkv} d={d}")
    loss_g, grad_g = run(wl, dev, scores)
    loss_o, grad_o = oracle.indexer_kl(wl.cu_q, wl.cu_k, host["q"], host["k"],
                                       scores.astype(np.float64), rows, wl.softmax_scale)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    worst = check(loss_g, grad_g, loss_o, grad_o, counts, scores)
    for i, n in enumerate(counts):
        assert (grad_g[i, n:] == 5.0).all()  # columns past p untouched
    log(f"  worst loss error {worst:.2e}, loss range {loss_o.min():.3f}..{loss_o.max():.3f}")


def test_kl_window_in_place_and_zero_target():
    """A window starting mid-sequence, the gradient written over the scores,
    and scores that reproduce the target (ln P), where the loss is ~0."""
    wl = small_wl([300], [300], 8, 2, 128, seed=4)
    host, dev = device_workload(wl, parts=("q", "k"))
    rows = np.arange(120, 300)
    ld = 300
    # ln P from the oracle's own target: zero gradient, zero loss.
    base = np.zeros((len(rows), ld))
    _, g0 = oracle.indexer_kl(wl.cu_q, wl.cu_k, host["q"], host["k"], base, rows,
                              wl.softmax_scale)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    lnp = np.zeros((len(rows), ld))
    for i, n in enumerate(counts):
        P = 1.0 / n - g0[i, :n]          # grad = Pi - P with Pi uniform
        lnp[i, :n] = np.log(P)
    loss_g, grad_g = run(wl, dev, lnp, row_begin=120, in_place=True)
    loss_o, grad_o = oracle.indexer_kl(wl.cu_q, wl.cu_k, host["q"], host["k"],
                                       lnp.astype(np.float32).astype(np.float64), rows,
                                       wl.softmax_scale)
    check(loss_g, grad_g, loss_o, grad_o, counts, lnp.astype(np.float32))
    assert np.abs(loss_g).max() < 1e-4


def test_kl_on_indexer_scores_full_size_sampled():
    """The 128K prefill's last 2048-row window is too long for the oracle
    to redo whole, so whole-window properties are checked on the GPU result
    and sampled rows against the oracle: loss >= 0 (up to rounding), every
    gradient row sums to ~0, and equal rows of the oracle."""
    wl = synth.prefill_128k()
    n = 2048
    r0 = wl.total_q - n
    q, k = wl.q(), wl.k()
    dev = {"q": to_dev_bf16_(q), "k": to_dev_bf16_(k)}
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    ld = wl.total_k
    rng = np.random.default_rng(5)
    sc = torch.randn((n, ld), device="cuda", dtype=torch.float32) * 2
    loss = torch.zeros(n, dtype=torch.float32, device="cuda")
    grad = torch.zeros((n, ld), dtype=torch.float32, device="cuda")
    log("indexer KL on a 2048-row window of the 128K prefill")
    dsa.dsa_indexer_kl(vl, dev["q"], dev["k"], sc, loss, grad=grad, row_begin=r0, row_count=n)
    torch.cuda.synchronize()
    lg = loss.cpu().numpy()
    assert (lg > -1e-4).all()
    gs = grad.sum(dim=1).cpu().numpy()
    assert np.abs(gs).max() < 1e-3
    rows = np.sort(rng.choice(n, size=3, replace=False))
    sel = torch.from_numpy(rows).to("cuda")
    s_np = sc[sel].cpu().numpy().astype(np.float64)
    lo, go = oracle.indexer_kl(wl.cu_q, wl.cu_k, q, k, s_np, rows + r0, wl.softmax_scale)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows + r0)
    check(lg[rows], grad[sel].cpu().numpy(), lo, go, counts, s_np)


def to_dev_bf16_(bits):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.to("cuda").view(torch.bfloat16)


def test_kl_separate_grad_stride_and_checked_scores(monkeypatch):
    """A gradient buffer with its own leading dimension; with DSA_CHECK set,
    a NaN among a row's visible scores is reported before any launch and a
    NaN past the row's position is not."""
    wl = small_wl([70], [90], 8, 2, 64, seed=13)
    host, dev = device_workload(wl, parts=("q", "k"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    n, ld = wl.total_q, 96
    rng = np.random.default_rng(2)
    scores = rng.standard_normal((n, ld)).astype(np.float32)
    sc = to_dev(scores)
    loss = torch.zeros(n, dtype=torch.float32, device="cuda")
    grad = torch.full((n, 100), 3.0, dtype=torch.float32, device="cuda")
    dsa.dsa_indexer_kl(vl, dev["q"], dev["k"], sc, loss, grad=grad)
    torch.cuda.synchronize()
    rows = np.arange(n)
    lo, go = oracle.indexer_kl(wl.cu_q, wl.cu_k, host["q"], host["k"], scores.astype(np.float64),
                               rows, wl.softmax_scale)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    check(loss.cpu().numpy(), grad.cpu().numpy()[:, :ld], lo, go, counts, scores)
    assert (grad.cpu().numpy()[:, ld:] == 3.0).all()
    monkeypatch.setenv("DSA_CHECK", "1")
    bad = scores.copy()
    bad[5, counts[5] + 2] = np.nan          # past row 5's position: never read
    dsa.dsa_indexer_kl(vl, dev["q"], dev["k"], to_dev(bad), loss)
    torch.cuda.synchronize()
    bad[7, 3] = np.nan                      # visible to row 7
    with pytest.raises(dsa.DSAError):
        dsa.dsa_indexer_kl(vl, dev["q"], dev["k"], to_dev(bad), loss)
