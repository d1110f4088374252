"""Pins of the oracle's indexer warm-up loss (oracle.indexer_kl) to facts that
do not come from the oracle itself: the KL divergence of a distribution from
itself is zero, the loss equals a library KL divergence of independently
built distributions, the gradient matches central finite differences of the
loss, softmax shift invariance, and causality.  The reading of the target
(per-head dense softmax averaged over query heads, page 5 section 1 names a
KL divergence to the full attention's distribution and nothing more) is
pinned by a case where only that reading gives zero loss.  CPU only."""
import math

import numpy as np
import pytest
import torch
from scipy.stats import entropy

import oracle
import synth


def bf(x):
    return synth.bf16_bits_from_float(np.asarray(x, np.float32))


def f(bits):
    return synth.bf16_to_float(bits).astype(np.float64)


def _case(seed, lq, lk, hq, hkv, d):
    rng = np.random.default_rng(seed)
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    q = bf(rng.standard_normal((cu_q[-1], hq, d)) * 1.5)
    k = bf(rng.standard_normal((cu_k[-1], hkv, d)) * 1.5)
    return rng, cu_q, cu_k, q, k


def _positions(cu_q, cu_k):
    """(sequence, position) of every packed query row."""
    out = []
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        out += [(b, lk - lq + i) for i in range(lq)]
    return out


def _head_probs(cu_k, q, k, b, t, p, scale):
    """torch CPU softmax (fp64) of every query head's logits over keys 0..p."""
    hq, hkv = q.shape[1], k.shape[1]
    g = hq // hkv
    keys = torch.from_numpy(f(k[cu_k[b]:cu_k[b] + p + 1]))           # [n, hkv, d]
    qq = torch.from_numpy(f(q[t]))                                   # [hq, d]
    z = torch.stack([scale * keys[:, h // g] @ qq[h] for h in range(hq)])  # [hq, n]
    return torch.softmax(z, dim=1).numpy()


def test_kl_is_zero_when_the_indexer_reproduces_the_target():
    """Scores equal to ln P (up to a per-row constant) make Pi = P: zero loss
    and zero gradient.  P is built here with a library softmax, averaging the
    per-head probabilities; averaging the logits instead (another reading)
    would leave a positive loss, which the second half checks."""
    rng, cu_q, cu_k, q, k = _case(3, [6, 9], [6, 13], 4, 2, 8)
    scale = 1 / math.sqrt(8)
    rows = np.arange(cu_q[-1])
    ld = 16
    good = np.zeros((len(rows), ld))
    other = np.zeros((len(rows), ld))
    for i, (b, p) in enumerate(_positions(cu_q, cu_k)):
        a = _head_probs(cu_k, q, k, b, i, p, scale)
        good[i, :p + 1] = np.log(a.mean(axis=0)) + rng.normal()
        other[i, :p + 1] = np.log(a).mean(axis=0)   # mean of log-probabilities
    loss, grad = oracle.indexer_kl(cu_q, cu_k, q, k, good, rows, scale)
    assert np.abs(loss).max() < 1e-12
    assert np.abs(grad).max() < 1e-12
    loss2, _ = oracle.indexer_kl(cu_q, cu_k, q, k, other, rows, scale)
    assert loss2[1:].min() > 1e-6   # row 0 sees one key: every distribution agrees


def test_kl_matches_library_entropy_of_independent_softmaxes():
    rng, cu_q, cu_k, q, k = _case(5, [7, 4, 10], [7, 9, 10], 8, 2, 16)
    scale = 1 / math.sqrt(16)
    rows = np.arange(cu_q[-1])
    ld = 12
    scores = rng.standard_normal((len(rows), ld)) * 3
    loss, grad = oracle.indexer_kl(cu_q, cu_k, q, k, scores, rows, scale)
    for i, (b, p) in enumerate(_positions(cu_q, cu_k)):
        P = _head_probs(cu_k, q, k, b, i, p, scale).mean(axis=0)
        Pi = torch.softmax(torch.from_numpy(scores[i, :p + 1]), dim=0).numpy()
        assert abs(loss[i] - entropy(P, Pi)) < 1e-12
        np.testing.assert_allclose(grad[i, :p + 1], Pi - P, rtol=0, atol=1e-14)
        assert (grad[i, p + 1:] == 0).all()
        assert loss[i] >= 0
        assert abs(grad[i, :p + 1].sum()) < 1e-13


def test_gradient_matches_central_differences():
    rng, cu_q, cu_k, q, k = _case(9, [5], [11], 2, 1, 8)
    scale = 0.3
    rows = np.arange(5)
    ld = 11
    scores = rng.standard_normal((5, ld))
    _, grad = oracle.indexer_kl(cu_q, cu_k, q, k, scores, rows, scale)
    eps = 1e-6
    for i, p in enumerate(range(6, 11)):
        for s in range(p + 1):
            hi, lo = scores.copy(), scores.copy()
            hi[i, s] += eps
            lo[i, s] -= eps
            lh, _ = oracle.indexer_kl(cu_q, cu_k, q, k, hi, rows, scale, want_grad=False)
            ll, _ = oracle.indexer_kl(cu_q, cu_k, q, k, lo, rows, scale, want_grad=False)
            assert abs((lh[i] - ll[i]) / (2 * eps) - grad[i, s]) < 1e-8


def test_shift_invariance_and_causality():
    """A constant added to a row's scores changes nothing; columns past the
    row's position are never read (NaN there leaves the result finite)."""
    rng, cu_q, cu_k, q, k = _case(11, [8], [8], 4, 4, 8)
    scale = 1 / math.sqrt(8)
    rows = np.arange(8)
    scores = rng.standard_normal((8, 8)) * 2
    loss, grad = oracle.indexer_kl(cu_q, cu_k, q, k, scores, rows, scale)
    shifted = scores + rng.standard_normal((8, 1)) * 50
    masked = shifted.copy()
    for t in range(8):
        masked[t, t + 1:] = np.nan
    loss2, grad2 = oracle.indexer_kl(cu_q, cu_k, q, k, masked, rows, scale)
    np.testing.assert_allclose(loss2, loss, rtol=0, atol=1e-12)
    for t in range(8):
        np.testing.assert_allclose(grad2[t, :t + 1], grad[t, :t + 1], rtol=0, atol=1e-14)
    assert loss[0] == 0.0 and grad[0, 0] == 0.0  # one visible key: both distributions are 1


def test_rejects_short_score_rows():
    _, cu_q, cu_k, q, k = _case(1, [4], [4], 1, 1, 8)
    with pytest.raises(ValueError):
        oracle.indexer_kl(cu_q, cu_k, q, k, np.zeros((4, 3)), np.arange(4), 1.0)
