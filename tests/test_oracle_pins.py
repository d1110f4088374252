"""Pins for the CPU oracle: each check ties it to something other than itself
(hand-derived values, closed forms, Python big-int arithmetic, numpy/torch
library routines in fp64, brute-force sorts, invariants).  CPU only.

A plausible slip in the oracle -- a dropped ReLU or weight, a sign, a
transposed operand, an off-by-one causal edge, the wrong GQA head mapping, the
wrong tie rule, a missing max-subtraction in the softmax -- fails at least one
test here.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bf(x):
    return synth.bf16_bits_from_float(np.asarray(x, np.float32))


def f(bits):
    return synth.bf16_to_float(bits).astype(np.float64)


# ---------------------------------------------------------------- worked example

def test_worked_example_by_hand():
    ex = json.load(open(os.path.join(GOLDEN, "worked_example_3tok.json")))
    ix = ex["indexer"]
    L = ex["sequence_length"]
    cu = np.array([0, L], np.int32)
    q_idx = np.zeros((L, ix["n_heads"], ix["d"]), np.uint16)
    q_idx[2] = bf(ix["q_idx_row2"])
    w = np.zeros((L, ix["n_heads"]), np.float32)
    w[2] = ix["w_row2"]
    k_idx = bf(ix["k_idx"])
    s = oracle.index_scores(cu, cu, q_idx, k_idx, w, [2])
    assert s[0].tolist() == ix["expected_scores_row2"]

    tk = ex["topk"]
    sel = oracle.topk(s, [3], tk["k"])
    assert sel[0].tolist() == tk["expected_idx_row2"]
    tie = np.array([tk["scores_tie"]], np.float64)
    assert oracle.topk(tie, [4], tk["k_tie"])[0].tolist() == tk["expected_idx_tie"]

    at = ex["attention"]
    q = np.zeros((L, at["n_heads_q"], at["head_dim"]), np.uint16)
    q[2] = bf(at["q_row2"])
    k = bf(at["k"])
    v = bf(at["v"])
    out, lse = oracle.sparse_attn(cu, cu, q, k, v, np.array([at["selected"]], np.int32), [2],
                                  at["scale"])
    assert np.allclose(out[0], at["expected_out_row2"], rtol=0, atol=1e-14)
    assert np.allclose(lse[0] - math.log(2.0), at["expected_lse_row2_minus_ln2"], atol=1e-14)


# ---------------------------------------------------------------- indexer

def test_index_scores_integer_inputs_match_bigint():
    """Integer qI, kI, w (the tiny integer workload's recipe): every score is an
    integer; compare with exact Python integer arithmetic."""
    wl = synth.prefill_2k_int().with_(seqlens_q=(300,), seqlens_k=(300,))
    qi, ki, w = wl.q_idx(), wl.k_idx(), wl.w()
    rows = [0, 1, 17, 150, 299]
    s = oracle.index_scores(wl.cu_q, wl.cu_k, qi, ki, w, rows)
    qi_i = f(qi).astype(np.int64)
    ki_i = f(ki).astype(np.int64)
    w_i = w.astype(np.int64)
    for n, r in enumerate(rows):
        for col in range(r + 1):
            total = 0
            for h in range(wl.n_heads_idx):
                dot = sum(int(a) * int(b) for a, b in zip(qi_i[r, h], ki_i[col]))
                total += int(w_i[r, h]) * max(0, dot)
            assert s[n, col] == total
        assert np.isnan(s[n, r + 1:]).all()


def test_index_scores_basis_vectors_closed_form():
    """qI[h] = +-e_j and one-hot or all-one weights reduce I to a single key
    coordinate: max(0, k[s, j]) and |k[s, j]|."""
    rng = np.random.default_rng(0)
    L, H, d = 40, 3, 8
    k_idx = bf(rng.standard_normal((L, d)))
    kf = f(k_idx)
    cu = np.array([0, L], np.int32)
    q_idx = np.zeros((L, H, d), np.uint16)
    w = np.zeros((L, H), np.float32)
    j = 5
    q_idx[:, 0, j] = bf(1.0)
    q_idx[:, 1, j] = bf(-1.0)
    q_idx[:, 2, 2] = bf(3.0)
    w[:, 0] = 1.0
    s = oracle.index_scores(cu, cu, q_idx, k_idx, w, [L - 1])
    assert np.array_equal(s[0], np.maximum(kf[:, j], 0.0))
    w[:, 1] = 1.0
    s = oracle.index_scores(cu, cu, q_idx, k_idx, w, [L - 1])
    assert np.array_equal(s[0], np.abs(kf[:, j]))
    w[:] = 0.0
    w[:, 2] = 0.25
    s = oracle.index_scores(cu, cu, q_idx, k_idx, w, [L - 1])
    assert np.array_equal(s[0], 0.25 * np.maximum(3.0 * kf[:, 2], 0.0))


def test_index_scores_vs_einsum_varlen():
    """Random real inputs against numpy einsum in fp64, packed varlen with
    Lq < Lk (position offset), every row."""
    rng = np.random.default_rng(1)
    lq, lk = [5, 1, 9], [12, 7, 9]
    H, d = 4, 16
    cu_q = np.concatenate([[0], np.cumsum(lq)]).astype(np.int32)
    cu_k = np.concatenate([[0], np.cumsum(lk)]).astype(np.int32)
    qi = bf(rng.standard_normal((cu_q[-1], H, d)))
    ki = bf(rng.standard_normal((cu_k[-1], d)))
    w = rng.standard_normal((cu_q[-1], H)).astype(np.float32)  # signed weights too
    rows = np.arange(cu_q[-1])
    s = oracle.index_scores(cu_q, cu_k, qi, ki, w, rows, ld=max(lk))
    for b in range(3):
        for i in range(lq[b]):
            r = cu_q[b] + i
            p = lk[b] - lq[b] + i
            keys = f(ki[cu_k[b]:cu_k[b] + p + 1])
            dots = np.einsum("hj,sj->hs", f(qi[r]), keys)
            ref = np.einsum("h,hs->s", w[r].astype(np.float64), np.maximum(dots, 0.0))
            np.testing.assert_allclose(s[r, :p + 1], ref, rtol=1e-12, atol=1e-12)
            assert np.isnan(s[r, p + 1:]).all()


def test_visible_counts_positions():
    cu_q = np.array([0, 3, 4], np.int32)
    cu_k = np.array([0, 5, 105], np.int32)
    assert oracle.visible_counts(cu_q, cu_k, [0, 1, 2, 3]).tolist() == [3, 4, 5, 100]
    with pytest.raises(ValueError):
        oracle.visible_counts(cu_q, cu_k, [4])


# ---------------------------------------------------------------- top-k

def _lexsort_topk(row, n_vis, k):
    keys = row[:n_vis]
    order = np.lexsort((np.arange(n_vis), -keys))  # score desc, then position asc
    sel = np.sort(order[:min(k, n_vis)])
    out = -np.ones(k, np.int32)
    out[:len(sel)] = sel
    return out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_topk_equals_full_sort(seed):
    rng = np.random.default_rng(seed)
    n_rows, ld, k = 40, 300, 64
    scores = rng.integers(-5, 6, size=(n_rows, ld)).astype(np.float64)  # heavy ties
    scores[::3] = rng.standard_normal((len(range(0, n_rows, 3)), ld))
    counts = rng.integers(1, ld + 1, size=n_rows)
    counts[0], counts[1], counts[2] = 1, k, k + 1
    idx = oracle.topk(scores, counts, k)
    for i in range(n_rows):
        assert np.array_equal(idx[i], _lexsort_topk(scores[i], counts[i], k))
        n = min(k, counts[i])
        sel = idx[i, :n]
        assert (idx[i, n:] == -1).all()
        assert (np.diff(sel) > 0).all() and sel[0] >= 0 and sel[-1] < counts[i]


def test_topk_signed_zero_is_a_tie():
    row = np.array([[0.0, -0.0, 0.0, -0.0, -1.0, 2.0]])
    assert oracle.topk(row, [6], 3)[0].tolist() == [0, 1, 5]
    row = np.array([[-0.0, 0.0, -1.0]])
    assert oracle.topk(row, [3], 1)[0].tolist() == [0]


def test_topk_float32_order():
    """float32 scores widen exactly, so the order is float32's."""
    a = np.float32(1.0)
    b = np.nextafter(a, np.float32(2.0))
    row = np.array([[a, b, a, b, a]], np.float32)
    assert oracle.topk(row, [5], 2)[0].tolist() == [1, 3]


# ---------------------------------------------------------------- attention

def _dense_causal_torch(q, k, v, scale):
    """torch CPU scaled_dot_product_attention in fp64 with GQA expansion."""
    qt = torch.from_numpy(f(q)).permute(1, 0, 2)[None]  # [1, Hq, L, d]
    group = q.shape[1] // k.shape[1]
    kt = torch.from_numpy(f(k)).permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
    vt = torch.from_numpy(f(v)).permute(1, 0, 2).repeat_interleave(group, dim=0)[None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                         scale=scale)
    return o[0].permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (8, 1)])
def test_sparse_attn_with_k_ge_L_is_dense_causal(hq, hkv):
    rng = np.random.default_rng(hq * 10 + hkv)
    L, d = 37, 16
    q = bf(rng.standard_normal((L, hq, d)) * 2)
    k = bf(rng.standard_normal((L, hkv, d)) * 2)
    v = bf(rng.standard_normal((L, hkv, d)))
    cu = np.array([0, L], np.int32)
    topk_k = 64
    idx = -np.ones((L, topk_k), np.int32)
    for t in range(L):
        idx[t, :t + 1] = np.arange(t + 1)
    scale = 1.0 / math.sqrt(d)
    out, lse = oracle.sparse_attn(cu, cu, q, k, v, idx, np.arange(L), scale)
    ref = _dense_causal_torch(q, k, v, scale)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-10)
    # lse against a library log-sum-exp of the dense causal logits
    from scipy.special import logsumexp
    group = hq // hkv
    for t in (0, L // 2, L - 1):
        for h in range(hq):
            z = scale * (f(k[:t + 1, h // group]) @ f(q[t, h]))
            assert abs(lse[t, h] - logsumexp(z)) < 1e-10


def test_sparse_attn_full_path_with_k_ge_L_equals_dense():
    """scores -> top-k with k >= L keeps every causal position, so the whole
    oracle path equals dense causal attention."""
    wl = synth.prefill_2k_int().with_(seqlens_q=(50,), seqlens_k=(50,), topk=64)
    r = oracle.dsa_rows(wl.cu_q, wl.cu_k, wl.q_idx(), wl.k_idx(), wl.w(), wl.q(), wl.k(),
                        wl.v(), np.arange(50), wl.topk, wl.softmax_scale)
    ref = _dense_causal_torch(wl.q(), wl.k(), wl.v(), wl.softmax_scale)
    np.testing.assert_allclose(r["out"], ref, rtol=0, atol=1e-10)


def test_sparse_attn_subset_matches_masked_dense():
    """With a strict subset selected, compare with a softmax over exactly the
    selected logits computed by numpy."""
    rng = np.random.default_rng(7)
    L, hq, hkv, d = 64, 6, 3, 8
    q = bf(rng.standard_normal((L, hq, d)))
    k = bf(rng.standard_normal((L, hkv, d)))
    v = bf(rng.standard_normal((L, hkv, d)))
    cu = np.array([0, L], np.int32)
    rows = np.array([10, 40, 63])
    idx = -np.ones((3, 16), np.int32)
    for n, r in enumerate(rows):
        sel = np.sort(rng.choice(r + 1, size=min(9, r + 1), replace=False))
        idx[n, :len(sel)] = sel
    scale = 0.3
    out, lse = oracle.sparse_attn(cu, cu, q, k, v, idx, rows, scale)
    for n, r in enumerate(rows):
        sel = idx[n][idx[n] >= 0]
        for h in range(hq):
            g = h // (hq // hkv)
            z = scale * (f(k[sel, g]) @ f(q[r, h]))
            p = np.exp(z - z.max())
            p /= p.sum()
            np.testing.assert_allclose(out[n, h], p @ f(v[sel, g]), rtol=0, atol=1e-12)


def test_sparse_attn_permutation_and_padding_invariant():
    rng = np.random.default_rng(3)
    L, hq, hkv, d = 30, 4, 2, 8
    q = bf(rng.standard_normal((L, hq, d)) * 3)
    k = bf(rng.standard_normal((L, hkv, d)) * 3)
    v = bf(rng.standard_normal((L, hkv, d)))
    cu = np.array([0, L], np.int32)
    base = np.array([[0, 3, 7, 11, 20, 29, -1, -1]], np.int32)
    perm = np.array([[29, -1, 7, 0, -1, 20, 3, 11]], np.int32)
    o1, l1 = oracle.sparse_attn(cu, cu, q, k, v, base, [29], 0.2)
    o2, l2 = oracle.sparse_attn(cu, cu, q, k, v, perm, [29], 0.2)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_sparse_attn_weights_sum_to_one_and_large_logits():
    """V constant -> O equals the constant (weights sum to 1); logits near 500
    stay finite only if the max is subtracted before exp."""
    L, hq, hkv, d = 10, 2, 1, 4
    q = bf(np.full((L, hq, d), 16.0))
    k = bf(np.full((L, hkv, d), 16.0))
    v = bf(np.full((L, hkv, d), 0.75))
    cu = np.array([0, L], np.int32)
    idx = np.array([[0, 4, 9, -1]], np.int32)
    out, lse = oracle.sparse_attn(cu, cu, q, k, v, idx, [9], 0.5)
    assert np.allclose(out, 0.75, atol=1e-14)
    assert np.allclose(lse, 0.5 * 16 * 16 * 4 + math.log(3.0), atol=1e-9)


def test_sparse_attn_rejects_non_causal_index():
    L = 5
    z = np.zeros((L, 1, 4), np.uint16)
    cu = np.array([0, L], np.int32)
    with pytest.raises(ValueError):
        oracle.sparse_attn(cu, cu, z, z, z, np.array([[0, 3]], np.int32), [2], 1.0)


def test_empty_selection_gives_zero_and_neg_inf():
    L = 4
    z = np.zeros((L, 2, 4), np.uint16)
    cu = np.array([0, L], np.int32)
    out, lse = oracle.sparse_attn(cu, cu, z, z[:, :1], z[:, :1],
                                  np.array([[-1, -1]], np.int32), [1], 1.0)
    assert (out == 0).all() and np.isneginf(lse).all()


# ---------------------------------------------------------------- decode

def test_decode_equals_last_prefill_row():
    """One query at p = N-1 over N cached tokens (decode) equals the last row
    of a causal prefill over the same tokens."""
    wl = synth.prefill_2k_int().with_(seqlens_q=(200,), seqlens_k=(200,), topk=32)
    qi, ki, w, q, k, v = wl.q_idx(), wl.k_idx(), wl.w(), wl.q(), wl.k(), wl.v()
    pre = oracle.dsa_rows(wl.cu_q, wl.cu_k, qi, ki, w, q, k, v, [199], 32, wl.softmax_scale)
    cu_q = np.array([0, 1], np.int32)
    dec = oracle.dsa_rows(cu_q, wl.cu_k, qi[199:], ki, w[199:], q[199:], k, v, [0], 32,
                          wl.softmax_scale)
    assert np.array_equal(pre["idx"], dec["idx"])
    assert np.array_equal(pre["out"], dec["out"])
    assert np.array_equal(pre["scores"], dec["scores"])


# ---------------------------------------------------------------- fp8 indexer inputs

def _torch_e4m3(values):
    """torch's float32 -> float8_e4m3fn conversion (round to nearest even)."""
    t = torch.tensor(np.asarray(values, np.float32)).to(torch.float8_e4m3fn)
    return t.view(torch.uint8).numpy()


def test_e4m3_values_match_torch_and_closed_forms():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = np.array([oracle.e4m3_value(c) for c in range(256)])
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.isnan(got).sum() == 2                       # 0x7f and 0xff only
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])
    assert oracle.e4m3_value(0x7E) == 448.0               # 1.75 * 2^8
    assert oracle.e4m3_value(0x38) == 1.0                 # exponent field 7 = bias
    assert oracle.e4m3_value(0x08) == 2.0 ** -6           # smallest normal
    assert oracle.e4m3_value(0x01) == 2.0 ** -9           # smallest subnormal
    assert oracle.e4m3_value(0xC4) == -3.0                # sign, 1.5 * 2^1


def test_e4m3_encode_rounding_ties_and_saturation():
    finite = [c for c in range(256) if c not in (0x7F, 0xFF)]
    # Every code is its own value's nearest code (the sign of zero kept).
    assert all(oracle.e4m3_encode(oracle.e4m3_value(c)) == c for c in finite)
    vals = sorted({oracle.e4m3_value(c) for c in range(0, 0x7F)})
    mids = [(a + b) / 2 for a, b in zip(vals, vals[1:])]
    probes = []
    for m in mids:
        m32 = np.float32(m)
        probes += [m32, np.nextafter(m32, np.float32(0)), np.nextafter(m32, np.float32(1e9))]
    rng = np.random.default_rng(0)
    probes += list(rng.uniform(-460, 460, 4000).astype(np.float32))
    probes += list((rng.standard_normal(2000) * 0.01).astype(np.float32))
    probes = np.array(probes, np.float32)
    probes = probes[np.abs(probes) < 464]                 # torch turns larger values into NaN
    got = np.array([oracle.e4m3_encode(float(v)) for v in probes], np.uint8)
    assert np.array_equal(got, _torch_e4m3(probes))
    # Ties go to the even mantissa: 1.0625 lies between 1.0 (m=0) and 1.125 (m=1).
    assert oracle.e4m3_encode(1.0625) == 0x38 and oracle.e4m3_encode(1.1875) == 0x3A
    for v in (448.5, 463.9, 470.0, 1e6):
        assert oracle.e4m3_encode(v) == 0x7E and oracle.e4m3_encode(-v) == 0xFE


def test_quantize_fp8_definition_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((40, 128)).astype(np.float32) * rng.uniform(0.01, 30, (40, 1))
    x[3] = 0.0                                            # all-zero row
    x[5, :] = 0.0
    x[5, 17] = -2.5                                       # one non-zero element
    xb = bf(x)
    codes, scales = oracle.quantize_fp8(xb)
    xf = synth.bf16_to_float(xb).astype(np.float32)
    amax = np.abs(xf).max(axis=1)
    for r in range(40):
        if amax[r] == 0:
            assert scales[r] == 0 and not codes[r].any()
            continue
        inv = np.float32(448) / amax[r]                   # binary32 steps, as defined
        assert np.array_equal(codes[r], _torch_e4m3(xf[r] * inv))
        assert scales[r] == amax[r] / np.float32(448)
    assert codes[5, 17] == 0xFE and scales[5] == np.float32(2.5) / np.float32(448)
    # Error bound of the represented values: half a step of 3 mantissa bits
    # (relative 2^-4) above 2^-6 * scale, half of 2^-9 * scale below it,
    # plus the roundings of inv and scale.
    deq = oracle.dequantize_fp8(codes, scales)
    err = np.abs(deq - xf.astype(np.float64))
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, scales[:, None] * 2.0 ** -10) * (1 + 1e-6) + 1e-30
    assert (err <= bound).all()
    assert np.abs(deq).max(axis=1)[amax > 0] == pytest.approx(amax[amax > 0], rel=1e-6)


def test_index_scores_fp8_equals_bf16_scores_on_exact_inputs():
    """Vectors whose every entry is a multiple of 0.5 up to 3.5, each holding a
    +-3.5, quantise losslessly (448 / 3.5 = 128, scale 2^-7): the fp8 score
    must equal the bf16 score exactly."""
    rng = np.random.default_rng(2)
    L, H, d = 70, 5, 64
    grid = np.arange(-7, 8) * 0.5
    q = rng.choice(grid, (L, H, d)).astype(np.float32)
    k = rng.choice(grid, (L, d)).astype(np.float32)
    q[:, :, 0] = 3.5
    k[:, 3] = -3.5
    w = rng.uniform(-1, 2, (L, H)).astype(np.float32)
    cu = np.array([0, 30, 70], np.int32)
    qb, kb = bf(q), bf(k)
    qc, qs = oracle.quantize_fp8(qb)
    kc, ks = oracle.quantize_fp8(kb)
    assert (qs == 2.0 ** -7).all() and (ks == 2.0 ** -7).all()
    rows = np.arange(L)
    ref = oracle.index_scores(cu, cu, qb, kb, w, rows)
    got = oracle.index_scores_fp8(cu, cu, qc, qs, kc, ks, w, rows)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_index_scores_fp8_within_quantisation_bound_of_bf16():
    """Random inputs: |I_fp8 - I| <= sum_h |w_h| (|dq_h| |k^| + |q_h| |dk|)
    (ReLU is 1-Lipschitz, Cauchy-Schwarz on each dot product), and the bound
    is not vacuous (most scores move much less)."""
    rng = np.random.default_rng(3)
    L, H, d = 48, 6, 128
    q = rng.standard_normal((L, H, d)).astype(np.float32)
    k = (rng.standard_normal((L, d)) + rng.standard_normal((1, d))).astype(np.float32)
    w = rng.uniform(0, 1, (L, H)).astype(np.float32)
    cu = np.array([0, L], np.int32)
    qb, kb = bf(q), bf(k)
    qc, qs = oracle.quantize_fp8(qb)
    kc, ks = oracle.quantize_fp8(kb)
    rows = np.arange(L)
    ref = oracle.index_scores(cu, cu, qb, kb, w, rows)
    got = oracle.index_scores_fp8(cu, cu, qc, qs, kc, ks, w, rows)
    qf, kf = f(qb), f(kb)
    qd, kd = oracle.dequantize_fp8(qc, qs), oracle.dequantize_fp8(kc, ks)
    dq = np.linalg.norm(qd - qf, axis=2)                  # [L, H]
    dk = np.linalg.norm(kd - kf, axis=1)                  # [L]
    nq = np.linalg.norm(qf, axis=2)
    nk_hat = np.linalg.norm(kd, axis=1)
    for t in range(L):
        bound = (np.abs(w[t])[:, None] * (dq[t][:, None] * nk_hat[None, :t + 1]
                                          + nq[t][:, None] * dk[None, :t + 1])).sum(axis=0)
        diff = np.abs(got[t, :t + 1] - ref[t, :t + 1])
        assert (diff <= bound * (1 + 1e-9)).all()
        assert np.median(diff) < 0.5 * np.median(bound)
