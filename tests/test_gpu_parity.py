"""GPU parity of the HIP path against the CPU oracle at sizes the oracle
finishes in seconds: several tiles, ragged tails, varlen, edge cases.  Every
call goes through the C ABI (libdsa.so)."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import (check_attn, check_attn_every_row, check_topk_rows, device_workload, from_dev_bf16, log, oracle_rows,
                  to_dev, to_dev_bf16)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402


def varlen_for(wl):
    return dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())


def small_wl(lq, lk, hq=8, hkv=2, d=64, hi=4, di=64, topk=256, integer=False, clustered=False,
             seed=11):
    return synth.Workload(name="test", seed=seed, seqlens_q=tuple(lq), seqlens_k=tuple(lk),
                          n_heads_q=hq, n_heads_kv=hkv, head_dim=d, n_heads_idx=hi, d_idx=di,
                          topk=topk, integer_indexer=integer, clustered=clustered)


# ---------------------------------------------------------------- top-k alone

def _topk_case(scores_rows, cu_q, cu_k, k, ld):
    """Run dsa_topk on host-made fp32 scores; compare bit-exactly with the
    oracle's selection on the same fp32 values (decided in fp32 on both sides)."""
    vl = dsa.Varlen(cu_q, cu_k)
    rows = np.arange(cu_q[-1])
    counts = oracle.visible_counts(np.array(cu_q, np.int32), np.array(cu_k, np.int32), rows)
    s_dev = to_dev(scores_rows.astype(np.float32))
    idx = torch.full((len(rows), k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(vl, s_dev, idx)
    torch.cuda.synchronize()
    ref = oracle.topk(scores_rows.astype(np.float32), counts, k)
    got = idx.cpu().numpy()
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]} differ; first: got {got[bad[0]][:12]} ref {ref[bad[0]][:12]}"


@pytest.mark.parametrize("case", ["normal", "ties", "signed_zero", "integers"])
def test_topk_single_sequence(case):
    rng = np.random.default_rng({"normal": 1, "ties": 2, "signed_zero": 3, "integers": 4}[case])
    L, k = 9000, 256
    ld = 9024
    if case == "normal":
        s = rng.standard_normal((L, ld))
    elif case == "ties":
        s = np.round(rng.standard_normal((L, ld)) * 2) / 2
    elif case == "signed_zero":
        s = rng.standard_normal((L, ld))
        s[:, ::3] = 0.0
        s[:, 1::3] = -0.0
        s[:, 2::7] = -1.5
    else:
        s = rng.integers(0, 3, size=(L, ld)).astype(np.float64)
    rows = np.r_[0:300, 4000:4100, 8700:9000]
    sub = s[rows]
    # only these rows: a varlen layout where each sampled row keeps its position
    cu_q = [0]
    cu_k = [0]
    for r in rows:
        cu_q.append(cu_q[-1] + 1)
        cu_k.append(cu_k[-1] + int(r) + 1)
    log(f"topk {case}: {len(rows)} rows, k={k}")
    _topk_case(sub, cu_q, cu_k, k, ld)


def test_topk_k2048_long_rows_and_boundaries():
    rng = np.random.default_rng(5)
    k = 2048
    lens = [1, 2047, 2048, 2049, 4095, 4096, 4097, 8191, 8192, 8193, 12289, 40000, 131072]
    ld = 131072
    s = rng.standard_normal((len(lens), ld)).astype(np.float32)
    s[3, :] = np.round(s[3, :])          # heavy ties in a row just above k
    s[11, :] = rng.integers(0, 2, size=ld)  # two-valued row: ties decide everything
    s[12, 60000:70000] = 7.0              # a tie block far above the rest
    cu_q = list(range(len(lens) + 1))
    cu_k = np.concatenate([[0], np.cumsum(lens)]).tolist()
    log("topk long rows")
    _topk_case(s, cu_q, cu_k, k, ld)


def test_topk_survivors_crowd_one_segment():
    """Regression: survivors concentrated in one quarter of every 1024-score
    step (block-structured scores) fill one wave's candidate segment while the
    total is still below k; the selection must stay exact."""
    rng = np.random.default_rng(11)
    k = 2048
    lens = [9000, 12106, 20000, 40000, 131072]
    ld = 131072
    s = rng.standard_normal((len(lens), ld)).astype(np.float32)
    hot = (np.arange(ld) % 1024) < 256
    s[:, hot] += 6.0
    s[1, (np.arange(ld) % 1024) >= 768] += 3.0  # two crowded quarters
    cu_q = list(range(len(lens) + 1))
    cu_k = np.concatenate([[0], np.cumsum(lens)]).tolist()
    log("topk crowded segments")
    _topk_case(s, cu_q, cu_k, k, ld)


@pytest.mark.parametrize("k", [1, 7, 64, 1000, 2048])
def test_topk_various_k_varlen(k):
    rng = np.random.default_rng(k)
    lq = [1, 7, 300, 5]
    lk = [9000, 2100, 300, 5]
    ld = 9000
    total_q = sum(lq)
    s = (rng.standard_normal((total_q, ld)) * 3).astype(np.float32)
    s[::2] = np.round(s[::2])
    cu_q = np.concatenate([[0], np.cumsum(lq)]).tolist()
    cu_k = np.concatenate([[0], np.cumsum(lk)]).tolist()
    log(f"topk varlen k={k}")
    _topk_case(s, cu_q, cu_k, k, ld)


@pytest.mark.parametrize("k,case", [(2048, "normal"), (2048, "integers"), (1000, "normal"),
                                    (7, "ties")])
def test_topk_few_long_rows_both_configurations(k, case):
    """Few long rows (decode-like, one query per sequence) run the wide
    configuration (four 16-byte loads per thread and step, 8192 candidates);
    the same rows inside a batch of more than 512 rows run the narrow one.
    Both must equal the oracle exactly; row lengths are ragged (shorter than
    k, one step, not a multiple of a step, the longest)."""
    rng = np.random.default_rng(k + len(case))
    lk = [131072, 20000, 16385, 9000, 2048, 100, 65539, 50001, 2049, 131071]
    B = len(lk)
    ld = 131072
    s = np.empty((B, ld), np.float32)
    for b in range(B):
        if case == "normal":
            row = rng.standard_normal(ld) * 2
        elif case == "integers":
            row = rng.integers(-40, 41, ld)
        else:  # heavy ties: a handful of values
            row = rng.integers(0, 3, ld) * 0.5
        s[b] = row.astype(np.float32)
    ref = oracle.topk(s, np.array(lk, np.int64), k)
    # wide: the ten rows alone
    vl = dsa.Varlen(list(range(B + 1)), np.concatenate([[0], np.cumsum(lk)]).tolist())
    wide = torch.full((B, k), -7, dtype=torch.int32, device="cuda")
    log(f"topk few long rows k={k} {case}")
    dsa.dsa_topk(vl, to_dev(s), wide)
    # narrow: 600 one-position rows first, then the same ten rows
    pad = 600
    lk2 = [1] * pad + lk
    vl2 = dsa.Varlen(list(range(B + pad + 1)), np.concatenate([[0], np.cumsum(lk2)]).tolist())
    s2 = torch.zeros((B + pad, ld), dtype=torch.float32, device="cuda")
    s2[pad:] = to_dev(s)
    narrow = torch.full((B + pad, k), -9, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(vl2, s2, narrow)
    torch.cuda.synchronize()
    got = wide.cpu().numpy()
    bad = np.nonzero((got != ref).any(axis=1))[0]
    assert bad.size == 0, f"wide configuration: rows {bad[:5]} differ"
    assert torch.equal(narrow[pad:], wide)
    assert (narrow[:pad, 0] == 0).all() and (narrow[:pad, 1:] == -1).all()


def _sampled_positions(n, pieces):
    """Positions read by the start-threshold sample of a row of n scores when
    the sample takes `pieces` 16-byte pieces spread over the row (piece i at
    floor(i n / pieces), rounded down to a multiple of 4)."""
    at = (np.arange(pieces, dtype=np.int64) * n // pieces) & ~3
    return np.unique((at[:, None] + np.arange(4)[None, :]).ravel())


@pytest.mark.parametrize("pieces", [1024, 256])
def test_topk_sample_threshold_too_high_restarts(pieces):
    """Rows whose largest scores sit exactly where the start-threshold sample
    reads (1024 pieces: the few-rows configuration, 512 threads x 2; 256: the
    many-rows one): the sampled threshold then admits far fewer than k scores
    and the row has to be streamed again from threshold zero.  The result
    must still equal the oracle exactly.  (Should the sampling rule change,
    the test still checks exactness; only this path may go unexercised.)"""
    rng = np.random.default_rng(100 + pieces)
    k = 2048
    lk = [131072, 65536, 40000, 20000]
    ld = 131072
    s = (rng.standard_normal((len(lk), ld)) * 0.1).astype(np.float32)
    for b, n in enumerate(lk):
        hot = _sampled_positions(n, pieces)
        s[b, hot] = 100.0 + rng.permutation(len(hot)).astype(np.float32)
    log(f"topk restart rows, {pieces} sample pieces")
    if pieces == 1024:
        cu_q = list(range(len(lk) + 1))
        cu_k = np.concatenate([[0], np.cumsum(lk)]).tolist()
        _topk_case(s, cu_q, cu_k, k, ld)
    else:
        # the many-rows configuration: 600 one-position rows before them
        pad = 600
        lk2 = [1] * pad + lk
        s2 = np.zeros((pad + len(lk), ld), np.float32)
        s2[pad:] = s
        cu_q = list(range(len(lk2) + 1))
        cu_k = np.concatenate([[0], np.cumsum(lk2)]).tolist()
        _topk_case(s2, cu_q, cu_k, k, ld)


@pytest.mark.parametrize("pieces,band", [(1024, (120, 300)), (512, (60, 150))])
def test_topk_restart_from_a_deeper_sample_rank(pieces, band):
    """Rows where the sampled start threshold admits fewer than k scores but
    a threshold four times deeper in the same sample admits enough: the
    sampled elements carry distinct large values (so the sample's order is
    known), and 3000 other positions carry values between the sample's
    band[0]-th and band[1]-th largest -- below the first threshold (rank
    about 49 of 2048 samples in the many-rows configuration, 97 of 4096 in
    the few-rows one, at n = 131072) and above the restart's (four times
    that rank).  The row is then streamed a second time from the deeper
    threshold rather than from zero; the result must equal the oracle
    exactly.  (Should the sampling rule change, the test still checks
    exactness; only this path may go unexercised.)"""
    rng = np.random.default_rng(300 + pieces)
    k = 2048
    lk = [131072, 120000]
    ld = 131072
    s = (rng.standard_normal((len(lk), ld)) * 0.1).astype(np.float32)
    for b, n in enumerate(lk):
        hot = _sampled_positions(n, pieces)
        h = len(hot)
        s[b, hot] = 100.0 + rng.permutation(h).astype(np.float32)  # rank r: 100 + h - r
        cold = np.setdiff1d(np.arange(n), hot)
        warm = rng.choice(cold, 3000, replace=False)
        lo, hi = 100.0 + h - band[1], 100.0 + h - band[0]
        s[b, warm] = (lo + 0.5 + (hi - lo - 1.0) * rng.random(3000)).astype(np.float32)
    log(f"topk restart from a deeper sample rank, {pieces} sample pieces")
    if pieces == 1024:
        cu_q = list(range(len(lk) + 1))
        cu_k = np.concatenate([[0], np.cumsum(lk)]).tolist()
        _topk_case(s, cu_q, cu_k, k, ld)
    else:
        pad = 600
        lk2 = [1] * pad + lk
        s2 = np.zeros((pad + len(lk), ld), np.float32)
        s2[pad:] = s
        cu_q = list(range(len(lk2) + 1))
        cu_k = np.concatenate([[0], np.cumsum(lk2)]).tolist()
        _topk_case(s2, cu_q, cu_k, k, ld)


def test_topk_row_window():
    """A window of rows inside the packed batch writes only its own rows."""
    rng = np.random.default_rng(9)
    L, k, ld = 3000, 128, 3008
    s = rng.standard_normal((L, ld)).astype(np.float32)
    vl = dsa.Varlen([0, L], [0, L])
    r0, n = 1000, 700
    win = to_dev(s[r0:r0 + n])
    idx = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(vl, win, idx, row_begin=r0, row_count=n)
    counts = np.arange(r0, r0 + n) + 1
    ref = oracle.topk(s[r0:r0 + n], counts, k)
    assert np.array_equal(idx.cpu().numpy(), ref)


# ---------------------------------------------------------------- indexer alone

def test_index_scores_integer_inputs_exact():
    """Integer-valued inputs (2048-token workload): every score is an integer
    and the GPU must reproduce the oracle bit for bit."""
    wl = synth.prefill_2k_int()
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = varlen_for(wl)
    ld = pipeline.score_ld(wl.max_seqlen_k)
    scores = torch.full((wl.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    log("index_scores prefill_2k_int")
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], scores)
    got = scores.cpu().numpy().astype(np.float64)
    ref = oracle.index_scores(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"],
                              np.arange(wl.total_q), ld=ld)
    causal = ~np.isnan(ref)
    assert np.array_equal(got[causal], ref[causal])
    assert np.isnan(got[~causal]).all()  # untouched beyond each row's position


@pytest.mark.parametrize("hi,di", [(64, 128), (40, 64), (4, 128), (33, 64)])
def test_index_scores_real_valued_bound(hi, di):
    """Real-valued inputs: |I_gpu - I_oracle| <= 2e-5 * sum_h |w_h| sum_j |q_hj k_j|
    (fp32 accumulation of exact bf16 products over d_idx, then over heads)."""
    wl = small_wl([300, 77, 1, 130], [300, 500, 129, 130], hi=hi, di=di, clustered=True,
                  seed=hi + di)
    host, dev = device_workload(wl, ("q_idx", "k_idx"))
    w = synth.uniform_f32(99, 1, 0, wl.total_q * hi, -1.0, 1.0).reshape(wl.total_q, hi)
    vl = varlen_for(wl)
    ld = pipeline.score_ld(wl.max_seqlen_k)
    scores = torch.full((wl.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    log(f"index_scores real H={hi} d={di}")
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], to_dev(w), scores)
    got = scores.cpu().numpy().astype(np.float64)
    rows = np.arange(wl.total_q)
    ref = oracle.index_scores(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], w, rows, ld=ld)
    qf = synth.bf16_to_float(host["q_idx"]).astype(np.float64)
    kf = synth.bf16_to_float(host["k_idx"]).astype(np.float64)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    for r in rows:
        b = np.searchsorted(wl.cu_q, r, side="right") - 1
        n = counts[r]
        keys = kf[wl.cu_k[b]:wl.cu_k[b] + n]
        bound = np.abs(w[r]).astype(np.float64) @ (np.abs(qf[r]) @ np.abs(keys).T)
        err = np.abs(got[r, :n] - ref[r, :n])
        assert (err <= 2e-5 * bound + 1e-30).all(), f"row {r}: {err.max()} vs {bound[err.argmax()]}"
        assert np.isnan(got[r, n:]).all()


# Cache lengths for the decode-shaped indexer: it streams each (row, key
# chunk) in groups of four 32-key tiles and then a tail of 0-3 tiles.  With
# 512-key chunks these give every tail on rows of 1-7 tiles and on the last
# chunk of chunked rows (992: 15 tiles, 1057: 2, 1120: 3, 1568: 1).
DECODE_TAIL_LENGTHS = [1, 32, 33, 64, 96, 97, 128, 200, 224, 992, 1000, 1057, 1120, 1568, 1600,
                       2047]


@pytest.mark.parametrize("hi,di", [(64, 128), (4, 64)])
def test_index_scores_decode_stream_every_tail(hi, di):
    """One query per sequence (the per-wave streaming indexer) on integer
    inputs: every score is an exact integer, so the kernel must reproduce the
    oracle bit for bit whatever the tile count modulo four."""
    lk = DECODE_TAIL_LENGTHS
    wl = small_wl([1] * len(lk), lk, hi=hi, di=di, integer=True, seed=44 + hi)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = varlen_for(wl)
    ld = pipeline.score_ld(wl.max_seqlen_k)
    scores = torch.full((wl.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    log(f"index_scores decode tails H={hi} d={di}")
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], scores)
    got = scores.cpu().numpy().astype(np.float64)
    ref = oracle.index_scores(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"],
                              np.arange(wl.total_q), ld=ld)
    causal = ~np.isnan(ref)
    assert causal.sum() == sum(lk)
    assert np.array_equal(got[causal], ref[causal])
    assert np.isnan(got[~causal]).all()


def test_index_scores_row_window_and_empty():
    wl = small_wl([700], [700], hi=64, di=128, seed=3)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = varlen_for(wl)
    ld = 704
    win = torch.full((100, ld), float("nan"), dtype=torch.float32, device="cuda")
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], win, row_begin=600,
                         row_count=100)
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], win, row_begin=0, row_count=0)
    ref = oracle.index_scores(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"],
                              np.arange(600, 700), ld=ld)
    got = win.cpu().numpy().astype(np.float64)
    ok = ~np.isnan(ref)
    assert np.allclose(got[ok], ref[ok], rtol=1e-4, atol=1e-3)
    assert np.isnan(got[~ok]).all()


# ---------------------------------------------------------------- attention alone

@pytest.mark.parametrize("hq,hkv,d", [(8, 2, 64), (32, 4, 128), (16, 1, 128), (8, 8, 64)])
def test_sparse_attn_prefill_given_indices(hq, hkv, d):
    """Attention over oracle-chosen indices (including -1 padding, k >= L rows
    and varlen) against the oracle's fp64 attention."""
    wl = small_wl([200, 33, 1, 64], [200, 50, 1, 300], hq=hq, hkv=hkv, d=d, hi=8, di=64,
                  topk=96, clustered=True, seed=hq + d)
    host, dev = device_workload(wl)
    rows = np.arange(wl.total_q)
    ref = oracle_rows(wl, host, rows)
    vl = varlen_for(wl)
    idx = to_dev(ref["idx"])
    out = torch.zeros((wl.total_q, hq, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((wl.total_q, hq), dtype=torch.float32, device="cuda")
    log(f"attn prefill hq={hq} hkv={hkv} d={d}")
    dsa.dsa_sparse_attn_prefill(vl, dev["q"], dev["k"], dev["v"], idx, out, lse=lse)
    torch.cuda.synchronize()
    check_attn(from_dev_bf16(out), ref["out"])
    assert np.allclose(lse.cpu().numpy(), ref["lse"], rtol=0, atol=2e-3)


def test_sparse_attn_shuffled_and_invalid_slots(monkeypatch):
    """Index order does not matter; -1 and out-of-range slots are empty; a row
    with no valid slot gives zeros and -inf.  The same call under DSA_CHECK
    (which reads out-of-range entries as empty slots for attention) is
    accepted and bitwise equal; the default scale (softmax_scale=None, the C
    ABI's DSA_SCALE_DEFAULT) is bitwise the explicit 1/sqrt(d)."""
    wl = small_wl([64], [64], hq=8, hkv=2, d=128, topk=32, seed=4)
    host, dev = device_workload(wl)
    rng = np.random.default_rng(0)
    idx = -np.ones((64, 40), np.int32)
    for t in range(64):
        sel = rng.permutation(t + 1)[:min(t + 1, 30)]
        idx[t, :len(sel)] = sel
        idx[t, 35] = t + 5  # beyond the causal position: an empty slot
        rng.shuffle(idx[t])
    idx[10] = -1
    rows = np.arange(64)
    clean = np.where((idx >= 0) & (idx <= rows[:, None]), idx, -1)
    ref_out, ref_lse = oracle.sparse_attn(wl.cu_q, wl.cu_k, host["q"], host["k"], host["v"], clean,
                                          rows, wl.softmax_scale)
    vl = varlen_for(wl)
    out = torch.full((64, 8, 128), 3.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((64, 8), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attn_prefill(vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out, lse=lse)
    torch.cuda.synchronize()
    check_attn(from_dev_bf16(out), ref_out)
    l = lse.cpu().numpy()
    assert np.isneginf(l[10]).all()
    ok = np.arange(64) != 10
    assert np.allclose(l[ok], ref_lse[ok], atol=2e-3)
    out2 = torch.zeros_like(out)
    lse2 = torch.zeros_like(lse)
    dsa.dsa_sparse_attn_prefill(vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out2, lse=lse2,
                                softmax_scale=float(np.float32(1) / np.sqrt(np.float32(128))))
    monkeypatch.setenv("DSA_CHECK", "1")
    out3 = torch.zeros_like(out)
    dsa.dsa_sparse_attn_prefill(vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out3)
    monkeypatch.delenv("DSA_CHECK")
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse, lse2)
    assert torch.equal(out.view(torch.int16), out3.view(torch.int16))


# ---------------------------------------------------------------- whole path

def test_prefill_2k_int_end_to_end():
    """The integer 2048-token workload through index_scores -> topk -> attention
    in two row windows: scores and indices exact, attention within tolerance."""
    wl = synth.prefill_2k_int()
    host, dev = device_workload(wl)
    vl = varlen_for(wl)
    bufs = pipeline.alloc_prefill(vl, wl.topk, window=1024)
    out = torch.zeros((wl.total_q, wl.n_heads_q, wl.head_dim), dtype=torch.bfloat16,
                      device="cuda")
    lse = torch.zeros((wl.total_q, wl.n_heads_q), dtype=torch.float32, device="cuda")
    keep = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    log("prefill_2k_int end to end")
    pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"], out,
                     bufs, lse=lse, keep_indices=keep)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    ref = oracle_rows(wl, host, rows)
    assert np.array_equal(keep.cpu().numpy(), ref["idx"])
    mx, mean = check_attn(from_dev_bf16(out), ref["out"])
    log(f"  attention max abs {mx:.3e} mean abs {mean:.3e}")
    assert np.allclose(lse.cpu().numpy(), ref["lse"], atol=2e-3)


@pytest.mark.parametrize("groups", [1, 3])
def test_decode_small_varlen(groups):
    """Decode (one query per sequence, p = Lk - 1) with ragged cache lengths,
    including caches shorter than k; with groups > 1 the batch runs as row
    groups alternating between two streams (ragged last group)."""
    lk = [1, 100, 2048, 2049, 5000, 9000, 300]
    wl = small_wl([1] * len(lk), lk, hq=32, hkv=4, d=128, hi=64, di=128, topk=2048, seed=21)
    host, dev = device_workload(wl)
    vl = varlen_for(wl)
    bufs = pipeline.alloc_decode(vl, wl.n_heads_q, wl.head_dim, wl.topk, groups=groups)
    out = torch.zeros((wl.batch, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((wl.batch, 32), dtype=torch.float32, device="cuda")
    log(f"decode small varlen, {groups} group(s)")
    side = torch.cuda.Stream() if groups > 1 else None
    pipeline.decode(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"], out,
                    bufs, lse=lse, side_stream=side)
    torch.cuda.synchronize()
    rows = np.arange(wl.batch)
    ref = oracle_rows(wl, host, rows)
    got_idx = bufs.indices.cpu().numpy()
    same = check_topk_rows(got_idx, ref["idx"], ref["scores"], ref["counts"], wl.topk)
    check_attn_every_row(wl, host, rows, got_idx, same, from_dev_bf16(out), lse.cpu().numpy(), ref)


def test_bitwise_repeatable():
    wl = small_wl([1500, 700], [1500, 700], hq=32, hkv=4, d=128, hi=64, di=128, topk=512,
                  clustered=True, seed=8)
    host, dev = device_workload(wl)
    vl = varlen_for(wl)
    outs = []
    # Three one-stream runs, then two with each window's attention on a side
    # stream (overlapping the next window's indexer): all bitwise equal.
    # A sixth run splits every window's attention into launches of 300 rows.
    for rep in range(6):
        two = rep in (3, 4)
        bufs = pipeline.alloc_prefill(vl, wl.topk, window=800 if rep != 4 else 256, overlap=two)
        out = torch.zeros((wl.total_q, 32, 128), dtype=torch.bfloat16, device="cuda")
        keep = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
        pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"],
                         out, bufs, keep_indices=keep,
                         side_stream=torch.cuda.Stream() if two else None,
                         attn_rows=300 if rep == 5 else None)
        torch.cuda.synchronize()
        outs.append((from_dev_bf16(out), keep.cpu().numpy()))
    for o, i in outs[1:]:
        assert np.array_equal(o, outs[0][0])
        assert np.array_equal(i, outs[0][1])
