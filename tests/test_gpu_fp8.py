"""GPU parity of the optional fp8 indexer (e4m3 codes, one scale per vector)
against the CPU oracle: quantisation bit for bit, scores exact on
integer-valued codes and within the fp32 accumulation bound otherwise, the
whole prefill and decode paths with the top-k tie-band rule.  Every call goes
through the C ABI (libdsa.so)."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import (check_attn, check_attn_every_row, check_topk_rows, device_workload, from_dev_bf16,
                  log, to_dev,
                  to_dev_bf16)

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402


def small_wl(lq, lk, hq=8, hkv=2, d=64, hi=4, di=64, topk=256, clustered=False, seed=11):
    return synth.Workload(name="test", seed=seed, seqlens_q=tuple(lq), seqlens_k=tuple(lk),
                          n_heads_q=hq, n_heads_kv=hkv, head_dim=d, n_heads_idx=hi, d_idx=di,
                          topk=topk, integer_indexer=False, clustered=clustered)


def varlen_for(wl):
    return dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())


def upload_fp8(codes, scales):
    return to_dev(codes), to_dev(scales.astype(np.float32))


# ---------------------------------------------------------------- quantisation

@pytest.mark.parametrize("d", [128, 64])
def test_quantize_fp8_bit_exact(d):
    """Codes and scales equal the oracle's on rows of every magnitude, rows of
    zeros, single non-zero rows, subnormal codes and exact rounding ties."""
    rows = 1001  # not a multiple of the vectors a wave handles per step
    rng = np.random.default_rng(d)
    x = rng.standard_normal((rows, d)) * np.exp(rng.uniform(-9, 9, (rows, 1)))
    x[5] = 0.0
    x[6] = 0.0
    x[6, 3] = -0.75
    x[7] = rng.standard_normal(d) * 1e-3
    x[7, 0] = 40.0                       # most of the row lands on subnormal codes
    # amax 3.5 makes inv = 128 exactly: 17 * 2^-11 * 128 = 1.0625 and
    # 19 * 2^-11 * 128 = 1.1875 are midpoints between e4m3 values.
    x[8] = 0.0
    x[8, :4] = [3.5, 17 * 2.0 ** -11, 19 * 2.0 ** -11, -17 * 2.0 ** -11]
    xb = synth.bf16_bits_from_float(x.astype(np.float32))
    ref_c, ref_s = oracle.quantize_fp8(xb)
    codes = torch.full((rows, d), 0x55, dtype=torch.uint8, device="cuda")
    scales = torch.full((rows,), -1.0, dtype=torch.float32, device="cuda")
    log(f"quantize_fp8 {rows} x {d}")
    dsa.dsa_quantize_fp8(to_dev_bf16(xb), codes, scales)
    torch.cuda.synchronize()
    got_c, got_s = codes.cpu().numpy(), scales.cpu().numpy()
    bad = np.nonzero((got_c != ref_c).any(axis=1))[0]
    assert bad.size == 0, f"rows {bad[:5]}: got {got_c[bad[0]][:8]} ref {ref_c[bad[0]][:8]}"
    assert np.array_equal(got_s.view(np.uint32), ref_s.view(np.uint32))
    assert ref_c[8, 1] == 0x38 and ref_c[8, 2] == 0x3A and ref_c[8, 3] == 0xB8


# ---------------------------------------------------------------- scores

def integer_fp8_inputs(wl, seed):
    """Codes of integers -3..3 with power-of-two scales and integer weights:
    every score is an exact integer in fp32."""
    rng = np.random.default_rng(seed)
    enc = np.array([oracle.e4m3_encode(v) for v in range(-3, 4)], np.uint8)
    qc = enc[rng.integers(0, 7, (wl.total_q, wl.n_heads_idx, wl.d_idx))]
    kc = enc[rng.integers(0, 7, (wl.total_k, wl.d_idx))]
    qs = (2.0 ** rng.integers(-2, 3, (wl.total_q, wl.n_heads_idx))).astype(np.float32)
    ks = (2.0 ** rng.integers(-2, 3, wl.total_k)).astype(np.float32)
    w = rng.integers(0, 4, (wl.total_q, wl.n_heads_idx)).astype(np.float32)
    return qc, qs, kc, ks, w


@pytest.mark.parametrize("case", ["prefill", "varlen", "decode"])
def test_index_scores_fp8_integer_codes_exact(case):
    """Exact integer scores bit for bit, through the prefill kernel (several
    LDS stages), the per-wave path of workgroups straddling sequences, and
    the decode kernel; then the top-k of those scores equals the oracle's."""
    if case == "prefill":
        wl = small_wl([700], [700], hi=64, di=128, seed=1)
    elif case == "varlen":
        wl = small_wl([300, 77, 1, 130], [300, 500, 129, 130], hi=33, di=64, seed=2)
    else:
        wl = small_wl([1] * 5, [1, 100, 2048, 2049, 5000], hi=64, di=128, topk=2048, seed=3)
    qc, qs, kc, ks, w = integer_fp8_inputs(wl, seed=len(case))
    vl = varlen_for(wl)
    ld = pipeline.score_ld(wl.max_seqlen_k)
    scores = torch.full((wl.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    log(f"index_scores_fp8 integer codes: {case}")
    dsa.dsa_index_scores_fp8(vl, to_dev(qc), to_dev(qs), to_dev(kc), to_dev(ks), to_dev(w), scores)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    ref = oracle.index_scores_fp8(wl.cu_q, wl.cu_k, qc, qs, kc, ks, w, rows, ld=ld)
    got = scores.cpu().numpy().astype(np.float64)
    causal = ~np.isnan(ref)
    assert np.array_equal(got[causal], ref[causal])
    assert np.isnan(got[~causal]).all()
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    sel = torch.full((wl.total_q, wl.topk), -7, dtype=torch.int32, device="cuda")
    dsa.dsa_topk(vl, scores, sel)
    torch.cuda.synchronize()
    assert np.array_equal(sel.cpu().numpy(), oracle.topk(ref, counts, wl.topk))


@pytest.mark.parametrize("hi,di", [(64, 128), (40, 64), (4, 128), (33, 64)])
def test_index_scores_fp8_real_valued_bound(hi, di):
    """Real-valued inputs quantised by the oracle: |I_gpu - I_oracle| <=
    2e-5 * sum_h |w_h| sum_j |q^_hj k^_j| on the represented values (exact
    code products summed in fp32, then the fp32 weighting and head sum)."""
    wl = small_wl([300, 77, 1, 130], [300, 500, 129, 130], hi=hi, di=di, clustered=True,
                  seed=hi + di)
    q_idx, k_idx = wl.q_idx(), wl.k_idx()
    w = synth.uniform_f32(98, 1, 0, wl.total_q * hi, -1.0, 1.0).reshape(wl.total_q, hi)
    qc, qs = oracle.quantize_fp8(q_idx)
    kc, ks = oracle.quantize_fp8(k_idx)
    vl = varlen_for(wl)
    ld = pipeline.score_ld(wl.max_seqlen_k)
    scores = torch.full((wl.total_q, ld), float("nan"), dtype=torch.float32, device="cuda")
    log(f"index_scores_fp8 real H={hi} d={di}")
    dsa.dsa_index_scores_fp8(vl, to_dev(qc), to_dev(qs), to_dev(kc), to_dev(ks), to_dev(w), scores)
    torch.cuda.synchronize()
    got = scores.cpu().numpy().astype(np.float64)
    rows = np.arange(wl.total_q)
    ref = oracle.index_scores_fp8(wl.cu_q, wl.cu_k, qc, qs, kc, ks, w, rows, ld=ld)
    qd, kd = oracle.dequantize_fp8(qc, qs), oracle.dequantize_fp8(kc, ks)
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    for r in rows:
        b = np.searchsorted(wl.cu_q, r, side="right") - 1
        n = counts[r]
        keys = kd[wl.cu_k[b]:wl.cu_k[b] + n]
        bound = np.abs(w[r]).astype(np.float64) @ (np.abs(qd[r]) @ np.abs(keys).T)
        err = np.abs(got[r, :n] - ref[r, :n])
        assert (err <= 2e-5 * bound + 1e-30).all(), f"row {r}: {err.max()} vs {bound[err.argmax()]}"
        assert np.isnan(got[r, n:]).all()


# ---------------------------------------------------------------- whole path

def fp8_oracle_rows(wl, host, rows):
    """The oracle path on the fp8-represented indexer inputs."""
    qc, qs = oracle.quantize_fp8(host["q_idx"])
    kc, ks = oracle.quantize_fp8(host["k_idx"])
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    s = oracle.index_scores_fp8(wl.cu_q, wl.cu_k, qc, qs, kc, ks, host["w"], rows)
    sel = oracle.topk(s, counts, wl.topk)
    o, l = oracle.sparse_attn(wl.cu_q, wl.cu_k, host["q"], host["k"], host["v"], sel, rows,
                              wl.softmax_scale)
    return {"scores": s, "counts": counts, "idx": sel, "out": o, "lse": l}


def test_prefill_fp8_end_to_end_varlen():
    """Quantise -> fp8 scores -> top-k -> attention over a clustered varlen
    batch in row windows: indices within the tie band of the oracle's fp8
    scores, attention within tolerance on rows whose sets agree."""
    wl = small_wl([1500, 700, 9], [1500, 700, 9], hq=32, hkv=4, d=128, hi=64, di=128,
                  topk=512, clustered=True, seed=8)
    host, dev = device_workload(wl)
    vl = varlen_for(wl)
    bufs = pipeline.alloc_prefill(vl, wl.topk, window=800)
    fp8 = pipeline.alloc_fp8_indexer(wl.total_q, wl.total_k, wl.n_heads_idx, wl.d_idx)
    out = torch.zeros((wl.total_q, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((wl.total_q, 32), dtype=torch.float32, device="cuda")
    keep = torch.full((wl.total_q, wl.topk), -7, dtype=torch.int32, device="cuda")
    log("prefill fp8 indexer, varlen")
    pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"], out,
                     bufs, lse=lse, keep_indices=keep, fp8=fp8)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    ref = fp8_oracle_rows(wl, host, rows)
    got_idx = keep.cpu().numpy()
    same = check_topk_rows(got_idx, ref["idx"], ref["scores"], ref["counts"], wl.topk)
    mx, mean, nd = check_attn_every_row(wl, host, rows, got_idx, same, from_dev_bf16(out),
                                        lse.cpu().numpy(), ref)
    log(f"  {same.sum()} of {len(rows)} rows identical ({nd} checked on the GPU's own indices); "
        f"attention max {mx:.2e} mean {mean:.2e}")


def test_decode_fp8_small_varlen():
    lk = [1, 100, 2048, 2049, 5000, 9000, 300]
    wl = small_wl([1] * len(lk), lk, hq=32, hkv=4, d=128, hi=64, di=128, topk=2048, seed=21)
    host, dev = device_workload(wl)
    vl = varlen_for(wl)
    bufs = pipeline.alloc_decode(vl, wl.n_heads_q, wl.head_dim, wl.topk)
    fp8 = pipeline.alloc_fp8_indexer(wl.total_q, wl.total_k, wl.n_heads_idx, wl.d_idx)
    pipeline.quantize_keys(dev["k_idx"], fp8)  # the cache, quantised when it was filled
    out = torch.zeros((wl.batch, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((wl.batch, 32), dtype=torch.float32, device="cuda")
    log("decode fp8 indexer, small varlen")
    pipeline.decode(vl, dev["q_idx"], None, dev["w"], dev["q"], dev["k"], dev["v"], out, bufs,
                    lse=lse, fp8=fp8)
    torch.cuda.synchronize()
    rows = np.arange(wl.batch)
    ref = fp8_oracle_rows(wl, host, rows)
    got_idx = bufs.indices.cpu().numpy()
    same = check_topk_rows(got_idx, ref["idx"], ref["scores"], ref["counts"], wl.topk)
    check_attn_every_row(wl, host, rows, got_idx, same, from_dev_bf16(out), lse.cpu().numpy(), ref)
