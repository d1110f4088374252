"""Pins of the oracle's indexer backward (oracle.index_scores_backward) to
things other than itself: central differences of the oracle's own forward
score, Euler's identity for the positively homogeneous ReLU score, linearity
in the upstream gradient, the zero gradient, columns past a row's position
never read, and the chain through the warm-up KL loss (page 5 section 1: the
dense warm-up trains only the indexer, so the loss's gradient must reach the
indexer's queries, keys and head weights)."""
import numpy as np

import oracle

CU = np.array([0, 9, 20], np.int32)      # two prefill sequences: 9 and 11 tokens
ROWS = np.arange(20, dtype=np.int64)
H, D = 3, 5
LD = 11


def _case(seed=0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((20, H, D))
    k = rng.standard_normal((20, D))
    w = rng.uniform(-1, 1, (20, H)).astype(np.float32)
    g = rng.standard_normal((20, LD))
    return q, k, w, g


def _loss(q, k, w, g, rows=ROWS):
    """L = sum over rows and visible columns of G * I (the forward is the
    oracle's real-valued indexer score)."""
    s = oracle.index_scores_f64(CU, CU, q[rows], k, w, rows, ld=LD)
    vis = ~np.isnan(s)
    return float(np.sum(np.where(vis, g[: len(rows)] * s, 0.0)))


def test_central_differences_of_the_score():
    q, k, w, g = _case(1)
    dq, dw, dk = oracle.index_scores_backward(CU, CU, q, k, w, g, ROWS)
    eps = 1e-6
    # queries: every coordinate (L is piecewise linear: the difference is exact
    # unless a ReLU kink lies within eps, which random inputs do not hit)
    for idx in np.ndindex(q.shape):
        qp, qm = q.copy(), q.copy()
        qp[idx] += eps
        qm[idx] -= eps
        fd = (_loss(qp, k, w, g) - _loss(qm, k, w, g)) / (2 * eps)
        assert abs(fd - dq[idx]) <= 1e-6 * max(1.0, abs(dq[idx])), idx
    for idx in np.ndindex(k.shape):
        kp, km = k.copy(), k.copy()
        kp[idx] += eps
        km[idx] -= eps
        fd = (_loss(q, kp, w, g) - _loss(q, km, w, g)) / (2 * eps)
        assert abs(fd - dk[idx]) <= 1e-6 * max(1.0, abs(dk[idx])), idx
    # head weights are fp32 inputs: L is linear in them, so a step of 2^-10
    # (exact in fp32 at these magnitudes) gives the derivative up to rounding
    step = np.float32(2.0 ** -10)
    for idx in np.ndindex(w.shape):
        wp, wm = w.copy(), w.copy()
        wp[idx] += step
        wm[idx] -= step
        fd = (_loss(q, k, wp, g) - _loss(q, k, wm, g)) / (2 * float(step))
        assert abs(fd - dw[idx]) <= 1e-9 * max(1.0, abs(dw[idx])), idx


def test_euler_identities():
    """I is positively homogeneous of degree 1 in each head's query and in
    each key (ReLU(a x) = a ReLU(x) for a > 0), so q . dL/dq = w dw per row and
    head, k . dL/dk = sum of G * I over the rows seeing that key, and
    sum_h w dw = sum_s G * I per row."""
    q, k, w, g = _case(2)
    dq, dw, dk = oracle.index_scores_backward(CU, CU, q, k, w, g, ROWS)
    s = oracle.index_scores_f64(CU, CU, q, k, w, ROWS, ld=LD)
    gi = np.where(np.isnan(s), 0.0, g * np.nan_to_num(s))
    np.testing.assert_allclose(np.einsum("thj,thj->th", q, dq), w.astype(np.float64) * dw,
                               rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose((w.astype(np.float64) * dw).sum(axis=1), gi.sum(axis=1),
                               rtol=1e-12, atol=1e-12)
    # key c = position s of sequence b: rows of sequence b with position >= s
    per_key = np.zeros(20)
    for t in range(20):
        b = 0 if t < 9 else 1
        p = t - CU[b]
        per_key[CU[b]:CU[b] + p + 1] += gi[t, :p + 1]
    np.testing.assert_allclose(np.einsum("cj,cj->c", k, dk), per_key, rtol=1e-12, atol=1e-12)


def test_linear_in_the_upstream_gradient_and_zero():
    q, k, w, g1 = _case(3)
    g2 = np.random.default_rng(4).standard_normal(g1.shape)
    a = oracle.index_scores_backward(CU, CU, q, k, w, 2.0 * g1 - 3.0 * g2, ROWS)
    b1 = oracle.index_scores_backward(CU, CU, q, k, w, g1, ROWS)
    b2 = oracle.index_scores_backward(CU, CU, q, k, w, g2, ROWS)
    for x, y1, y2 in zip(a, b1, b2):
        np.testing.assert_allclose(x, 2.0 * y1 - 3.0 * y2, rtol=1e-12, atol=1e-12)
    for x in oracle.index_scores_backward(CU, CU, q, k, w, np.zeros_like(g1), ROWS):
        assert not x.any()


def test_columns_past_the_position_are_not_read():
    q, k, w, g = _case(5)
    pos = np.array([t - (0 if t < 9 else 9) for t in range(20)])
    g_nan = g.copy()
    for t in range(20):
        g_nan[t, pos[t] + 1:] = np.nan
    for x, y in zip(oracle.index_scores_backward(CU, CU, q, k, w, g_nan, ROWS),
                    oracle.index_scores_backward(CU, CU, q, k, w, np.where(np.isnan(g_nan), 0, g),
                                                 ROWS)):
        assert np.isfinite(x).all()
        np.testing.assert_array_equal(x, y)


def test_bf16_inputs_widen_exactly():
    """bf16 bit patterns in, the same result as their exact float64 values."""
    rng = np.random.default_rng(6)
    qb = (rng.integers(0, 1 << 16, (20, H, D)) & 0x3FFF | 0x3C00).astype(np.uint16)  # finite, moderate
    kb = (rng.integers(0, 1 << 16, (20, D)) & 0xBFFF | 0x3C00).astype(np.uint16)
    w = rng.uniform(-1, 1, (20, H)).astype(np.float32)
    g = rng.standard_normal((20, LD))
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)  # noqa: E731
    for x, y in zip(oracle.index_scores_backward(CU, CU, qb, kb, w, g, ROWS),
                    oracle.index_scores_backward(CU, CU, widen(qb), widen(kb), w, g, ROWS)):
        np.testing.assert_array_equal(x, y)


def test_chain_through_the_warm_up_loss():
    """d (sum of KL losses) / d qI = backward(Pi - P): the KL oracle's score
    gradient fed through the indexer backward matches central differences of
    the KL loss itself over the indexer queries and keys."""
    rng = np.random.default_rng(7)
    q_idx, k_idx, w, _ = _case(8)
    # attention inputs (the fixed target P) as bf16 bits
    qa = (rng.standard_normal((20, 4, 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ka = (rng.standard_normal((20, 2, 8)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    scale = 0.35

    def kl_sum(qq, kk):
        s = oracle.index_scores_f64(CU, CU, qq, kk, w, ROWS, ld=LD)
        loss, _ = oracle.indexer_kl(CU, CU, qa, ka, np.nan_to_num(s), ROWS, scale,
                                    want_grad=False)
        return float(loss.sum())

    s = oracle.index_scores_f64(CU, CU, q_idx, k_idx, w, ROWS, ld=LD)
    _, grad = oracle.indexer_kl(CU, CU, qa, ka, np.nan_to_num(s), ROWS, scale)
    dq, _, dk = oracle.index_scores_backward(CU, CU, q_idx, k_idx, w, grad, ROWS)
    eps = 1e-6
    for idx in [(0, 0, 0), (5, 2, 4), (12, 1, 3), (19, 0, 1), (8, 2, 2)]:
        qp, qm = q_idx.copy(), q_idx.copy()
        qp[idx] += eps
        qm[idx] -= eps
        fd = (kl_sum(qp, k_idx) - kl_sum(qm, k_idx)) / (2 * eps)
        assert abs(fd - dq[idx]) <= 1e-6 * max(1.0, abs(dq[idx])), idx
    for idx in [(0, 0), (4, 3), (9, 1), (15, 4), (19, 2)]:
        kp, km = k_idx.copy(), k_idx.copy()
        kp[idx] += eps
        km[idx] -= eps
        fd = (kl_sum(q_idx, kp) - kl_sum(q_idx, km)) / (2 * eps)
        assert abs(fd - dk[idx]) <= 1e-6 * max(1.0, abs(dk[idx])), idx


def test_a_planted_sign_error_is_caught():
    """The central-difference pin fails when the backward's key gradient is
    off by a sign (a mistake planted in the oracle's output, on the CPU)."""
    q, k, w, g = _case(9)
    dq, dw, dk = oracle.index_scores_backward(CU, CU, q, k, w, g, ROWS)
    eps = 1e-6
    idx = tuple(np.argwhere(np.abs(dk) > 1e-3)[0])
    kp, km = k.copy(), k.copy()
    kp[idx] += eps
    km[idx] -= eps
    fd = (_loss(q, kp, w, g) - _loss(q, km, w, g)) / (2 * eps)
    assert abs(fd - (-dk[idx])) > 1e-3


def test_key_restricted_dk_by_central_differences():
    """index_scores_backward_keys at listed keys, for listed rows only (a
    window that starts mid-sequence): central differences of the score sum
    over those rows with respect to each listed key."""
    q, k, w, g = _case(10)
    rows = np.arange(4, 15, dtype=np.int64)           # rows 4..14: both sequences, partial
    keys = np.array([0, 3, 8, 9, 12, 19], np.int64)   # key 19 is seen by no listed row
    pos = np.array([t - (0 if t < 9 else 9) for t in rows])
    seq_k0 = np.array([0 if t < 9 else 9 for t in rows])
    g_rows = g[: len(rows)]   # dL/dI of listed row i (column = local key)
    grad_at = np.array([[g_rows[i, c - seq_k0[i]] if 0 <= c - seq_k0[i] <= pos[i] and
                         (c < 9) == (rows[i] < 9) else 0.0 for c in keys]
                        for i in range(len(rows))])
    dk = oracle.index_scores_backward_keys(CU, CU, q[rows], k, w, grad_at, rows, keys)

    def loss(kk):
        s = oracle.index_scores_f64(CU, CU, q[rows], kk, w, rows, ld=LD)
        return float(np.sum(np.where(np.isnan(s), 0.0, g_rows * np.nan_to_num(s))))

    eps = 1e-6
    for ci, c in enumerate(keys):
        for j in range(D):
            kp, km = k.copy(), k.copy()
            kp[c, j] += eps
            km[c, j] -= eps
            fd = (loss(kp) - loss(km)) / (2 * eps)
            assert abs(fd - dk[ci, j]) <= 1e-6 * max(1.0, abs(dk[ci, j])), (c, j)
    assert not dk[-1].any()
    # the dense backward's key gradient agrees at the listed keys
    _, _, dk_dense = oracle.index_scores_backward(CU, CU, q[rows], k, w, g_rows, rows)
    np.testing.assert_allclose(dk, dk_dense[keys], rtol=1e-12, atol=1e-12)
