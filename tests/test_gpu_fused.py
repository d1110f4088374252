"""The fused indexer -> top-k (dsa_index_topk) through the C ABI.

It must return exactly what dsa_index_scores -> dsa_topk return on the same
inputs (the same kernel arithmetic makes the scores, the same tie rule picks
among them), and therefore meet the oracle's acceptance rules: bit-exact on
integer indexer inputs, the 1e-3 tie band of the k-th score otherwise.  The
sampled threshold only decides how many candidates a row keeps; inputs built
to defeat it (sampled keys far above or far below the rest) must send rows to
the exact fallback and still give the same selection.
"""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check_topk_rows, device_workload, log, to_dev_bf16

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402

SAMPLE_STRIDE = 64  # every 64th key is sampled for rows up to 262144 keys


def wl_of(lq, lk, hi=64, di=128, topk=2048, integer=False, clustered=True, seed=31):
    return synth.Workload(name="fused", seed=seed, seqlens_q=tuple(lq), seqlens_k=tuple(lk),
                          n_heads_q=8, n_heads_kv=2, head_dim=64, n_heads_idx=hi, d_idx=di,
                          topk=topk, integer_indexer=integer, clustered=clustered)


def unfused(vl, dev, k, window):
    ld = pipeline.score_ld(vl.max_seqlen_k)
    scores = torch.empty((window, ld), dtype=torch.float32, device="cuda")
    out = torch.full((vl.total_q, k), -7, dtype=torch.int32, device="cuda")
    for r0 in range(0, vl.total_q, window):
        n = min(window, vl.total_q - r0)
        dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], scores, row_begin=r0,
                             row_count=n)
        dsa.dsa_topk(vl, scores, out[r0:r0 + n], row_begin=r0, row_count=n)
    return out


def fused(vl, dev, k, window):
    """Returns (indices, candidate counts, fallback flags) of every row."""
    ws = torch.empty(dsa.dsa_index_topk_workspace_size(vl, window, k), dtype=torch.uint8,
                     device="cuda")
    out = torch.full((vl.total_q, k), -7, dtype=torch.int32, device="cuda")
    counts, flags = [], []
    for r0 in range(0, vl.total_q, window):
        n = min(window, vl.total_q - r0)
        off = (n * 4 + 255) // 256 * 256  # the flags follow the counts, 256-byte aligned
        dsa.dsa_index_topk(vl, dev["q_idx"], dev["k_idx"], dev["w"], out[r0:r0 + n], ws,
                           row_begin=r0, row_count=n)
        counts.append(ws[:4 * n].view(torch.int32).clone())
        flags.append(ws[off:off + 4 * n].view(torch.int32).clone())
    torch.cuda.synchronize()
    return out, torch.cat(counts).cpu().numpy(), torch.cat(flags).cpu().numpy()


def oracle_select(wl, host, rows):
    """The oracle's indexer scores and top-k of the given packed rows."""
    counts = oracle.visible_counts(wl.cu_q, wl.cu_k, rows)
    sc = oracle.index_scores(wl.cu_q, wl.cu_k, host["q_idx"], host["k_idx"], host["w"], rows)
    return {"scores": sc, "counts": counts, "idx": oracle.topk(sc, counts, wl.topk)}


def positions(wl):
    return np.concatenate([np.arange(L) + (lk - L) for L, lk in zip(wl.seqlens_q, wl.seqlens_k)])


@pytest.mark.parametrize("window", [2048, 700])
def test_fused_integer_2k_exact(window):
    """prefill_2k_int: rows are shorter than a candidate list, so every score
    is a candidate; indices bit-exact against the oracle and the unfused path."""
    wl = synth.prefill_2k_int()
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    got, counts, flags = fused(vl, dev, wl.topk, window)
    ref = unfused(vl, dev, wl.topk, window)
    assert torch.equal(got, ref)
    rows = np.arange(wl.total_q)
    ora = oracle_select(wl, host, rows)
    assert np.array_equal(got.cpu().numpy(), ora["idx"])
    assert (counts == positions(wl) + 1).all() and (flags == 0).all()


@pytest.mark.parametrize("di,hi", [(128, 64), (64, 4)])
def test_fused_long_rows_match_unfused_and_oracle(di, hi):
    """Rows up to 20000 keys (beyond a list's 10240, so the sampled threshold
    is used) in a varlen batch whose workgroups straddle sequences, in windows
    that split sequences: bitwise the unfused selection; sampled rows against
    the oracle."""
    wl = wl_of([20000, 3000, 12000, 1], [20000, 3000, 12000, 1], hi=hi, di=di, seed=32 + di)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    got, counts, flags = fused(vl, dev, wl.topk, 4096)
    ref = unfused(vl, dev, wl.topk, 4096)
    assert torch.equal(got, ref)
    long_rows = positions(wl) + 1 > 10240
    log(f"  long rows: {long_rows.sum()}, candidates mean {counts[long_rows].mean():.0f} "
        f"min {counts[long_rows].min()} max {counts[long_rows].max()}, "
        f"fallbacks {int(flags.sum())}")
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([[0, 2047, 2048, 19999, 20000, 22999, 23000, 34999, 35000],
                                     rng.integers(0, wl.total_q, 40)]))
    ora = oracle_select(wl, host, rows)
    check_topk_rows(got[torch.from_numpy(rows).cuda()].cpu().numpy(), ora["idx"], ora["scores"],
                    ora["counts"], wl.topk)


def _crafted(scale_sampled):
    """Keys at sampled positions (multiples of 64) scaled by scale_sampled:
    0 makes every sampled score 0 (the threshold admits every score, so long
    lists overflow); a large factor makes the sampled scores tower over the
    rest (too few candidates).  Either way the rows must fall back."""
    wl = wl_of([16384, 5000], [16384, 5000], seed=35, clustered=False)
    ki = synth.bf16_to_float(wl.k_idx()).astype(np.float32)
    ki[::SAMPLE_STRIDE] *= scale_sampled
    ki[16384::SAMPLE_STRIDE] = synth.bf16_to_float(wl.k_idx())[16384::SAMPLE_STRIDE]
    bits = (ki.view(np.uint32) >> 16).astype(np.uint16)
    assert (synth.bf16_to_float(bits) == ki).all()  # exact in bf16 (power-of-two scale or 0)
    dev = {"q_idx": to_dev_bf16(wl.q_idx()), "k_idx": to_dev_bf16(bits),
           "w": torch.from_numpy(wl.w()).cuda()}
    return wl, dev


@pytest.mark.parametrize("scale", [0.0, 64.0])
def test_fused_fallback_when_the_sample_misleads(scale):
    wl, dev = _crafted(scale)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    got, counts, flags = fused(vl, dev, wl.topk, 2048)
    ref = unfused(vl, dev, wl.topk, 2048)
    assert torch.equal(got, ref)
    long_rows = positions(wl) + 1 > 10240  # only in the first sequence, the crafted one
    assert flags[long_rows].all(), f"{(flags[long_rows] == 0).sum()} misled rows did not fall back"
    if scale == 0.0:
        assert (counts[long_rows] > 10240).all()
    else:
        assert (counts[long_rows] < wl.topk).all()
    assert (flags[~long_rows] == 0).all()


def test_fused_decode_small_varlen_and_groups():
    """Decode (one query per sequence): ragged caches around k and the list
    size, fused against unfused, and the pipeline's fused decode with two row
    groups on two streams."""
    lk = [1, 100, 2048, 2049, 10240, 10241, 70000, 131072]
    wl = synth.Workload(name="fused_dec", seed=36, seqlens_q=(1,) * len(lk), seqlens_k=tuple(lk),
                        n_heads_q=32, n_heads_kv=4, head_dim=128, n_heads_idx=64, d_idx=128,
                        topk=2048)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w", "q", "k", "v"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    got, counts, flags = fused(vl, dev, wl.topk, wl.batch)
    ref = unfused(vl, dev, wl.topk, wl.batch)
    assert torch.equal(got, ref)
    log(f"  decode candidates {counts.tolist()}, fallbacks {flags.tolist()}")
    for groups in (1, 2):
        bufs = pipeline.alloc_decode(vl, wl.n_heads_q, wl.head_dim, wl.topk, groups=groups,
                                     fused=True)
        ubufs = pipeline.alloc_decode(vl, wl.n_heads_q, wl.head_dim, wl.topk, groups=groups)
        outs = []
        for b in (bufs, ubufs):
            out = torch.zeros((wl.batch, 32, 128), dtype=torch.bfloat16, device="cuda")
            pipeline.decode(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"],
                            dev["v"], out, b, side_stream=torch.cuda.Stream() if groups > 1 else None)
            outs.append(out)
        torch.cuda.synchronize()
        assert torch.equal(bufs.indices, ubufs.indices)
        assert torch.equal(outs[0].view(torch.int16), outs[1].view(torch.int16))


def test_fused_decode_stream_every_tail():
    """Candidate mode of the per-wave streaming indexer on integer inputs,
    with cache lengths that end a row or its last key chunk in every tail of
    0-3 tiles after the groups of four: the fused selection equals the
    unfused one and the oracle's (ties to the lower position)."""
    lk = [1, 32, 33, 64, 96, 97, 128, 200, 224, 992, 1000, 1057, 1120, 1568, 1600, 2047]
    wl = synth.Workload(name="fused_dec_tails", seed=45, seqlens_q=(1,) * len(lk),
                        seqlens_k=tuple(lk), n_heads_q=8, n_heads_kv=2, head_dim=64,
                        n_heads_idx=64, d_idx=128, topk=64, integer_indexer=True)
    host, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    log("fused decode tails")
    got, counts, flags = fused(vl, dev, wl.topk, wl.batch)
    ref = unfused(vl, dev, wl.topk, wl.batch)
    assert torch.equal(got, ref)
    ora = oracle_select(wl, host, np.arange(wl.batch))
    check_topk_rows(got.cpu().numpy(), ora["idx"], ora["scores"], ora["counts"], wl.topk)


def test_fused_prefill_pipeline_equals_unfused():
    """The whole prefill (windows, attention launches) fused and unfused:
    bitwise equal outputs and indices."""
    wl = wl_of([14000, 2500], [14000, 2500], seed=37)
    wl = synth.Workload(**{**wl.__dict__, "n_heads_q": 32, "n_heads_kv": 4, "head_dim": 128})
    host, dev = device_workload(wl)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    res = []
    for f in (True, False):
        bufs = pipeline.alloc_prefill(vl, wl.topk, 3000, fused=f)
        out = torch.zeros((wl.total_q, 32, 128), dtype=torch.bfloat16, device="cuda")
        keep = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
        pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"],
                         out, bufs, keep_indices=keep, attn_rows=1000)
        res.append((out, keep))
    torch.cuda.synchronize()
    assert torch.equal(res[0][1], res[1][1])
    assert torch.equal(res[0][0].view(torch.int16), res[1][0].view(torch.int16))


def test_fused_repeatable():
    wl = wl_of([30000], [30000], seed=38)
    _, dev = device_workload(wl, ("q_idx", "k_idx", "w"))
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    a, ca, _ = fused(vl, dev, wl.topk, 2048)
    b, cb, _ = fused(vl, dev, wl.topk, 2048)
    assert torch.equal(a, b)
    assert np.array_equal(ca, cb)
