"""Host-side logic of bench.py (no GPU): the algorithmic counts the rooflines
divide by, the stratified oracle sample, the traffic record check and the
one-GPU guard.  The counts are checked against brute-force enumeration of
the causal pairs and selected pairs they stand for."""
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import synth  # noqa: E402


def _brute(wl):
    pairs = sel = 0
    for lq, lk in zip(wl.seqlens_q, wl.seqlens_k):
        for i in range(lq):
            p = lk - lq + i
            pairs += p + 1
            sel += min(wl.topk, p + 1)
    return pairs, sel


@pytest.mark.parametrize("lens", [(2048,), (300, 1, 2048, 700), (5000,)])
def test_prefill_counts_match_enumeration(lens):
    wl = synth.prefill_2k_int().with_(seqlens_q=lens, seqlens_k=lens)
    c = bench.prefill_counts(wl)
    pairs, sel = _brute(wl)
    assert c["pairs"] == pairs and c["selected"] == sel
    assert c["f_idx"] == pairs * 2 * wl.n_heads_idx * wl.d_idx
    assert c["f_attn"] == sel * 4 * wl.n_heads_q * wl.head_dim
    assert c["b_gather"] == sel * 2 * wl.n_heads_kv * wl.head_dim * 2  # K and V rows, bf16
    assert c["b_scores"] == pairs * 8  # fp32 written once, read once


def test_window_flops_sum_to_the_prefill():
    wl = synth.prefill_2k_int().with_(seqlens_q=(5000,), seqlens_k=(5000,))
    total = sum(bench.window_flops(wl, r0, min(1024, 5000 - r0)) for r0 in range(0, 5000, 1024))
    assert total == bench.prefill_counts(wl)["f_idx"]


def test_headline_counts_closed_form():
    """131072 causal rows, k = 2048: L(L+1)/2 pairs; the first k rows select
    p + 1 positions, the rest k."""
    wl = synth.prefill_128k()
    c = bench.prefill_counts(wl)
    L, k = 131072, 2048
    assert c["pairs"] == L * (L + 1) // 2
    assert c["selected"] == k * (k + 1) // 2 + (L - k) * k
    assert c["f_idx"] == 140738562097152  # 16384 flops per causal pair


def test_decode_bytes_per_query():
    """64 x 131072 decode: the indexer's key stream (256 B a key), 2048 K and V
    rows of 4 heads x 128 (4 KiB a position), the score round trip (8 B a
    key), the index round trip, qI, w, q and out."""
    wd = synth.decode_b64_128k()
    total, per = bench.decode_bytes(wd)
    N, k = 131072, 2048
    expect = N * 256 + k * 2 * 4 * 128 * 2 + N * 8 + k * 8 + 64 * 128 * 2 + 64 * 4 + 2 * 32 * 128 * 2
    assert per == expect and total == 64 * expect


def test_stratified_rows():
    rows = bench.stratified_rows(131072, 2048, 1024, seed=0)
    assert np.all(np.diff(rows) > 0)
    assert rows[0] == 0 and rows[-1] == 131071
    assert {2047, 2048} <= set(rows.tolist())
    assert 1024 <= len(rows) <= 1028
    edges = np.linspace(0, 131072, 1025).astype(np.int64)
    hits = np.histogram(rows, bins=edges)[0]
    assert (hits >= 1).all()  # one row from every stratum


def test_counter_traffic_requires_the_measured_source_and_window(tmp_path, monkeypatch):
    src = tmp_path / "kernel.hip"
    src.write_bytes(b"kernel v1")
    import hashlib

    rec = {"source_sha256": hashlib.sha256(b"kernel v1").hexdigest(), "window_rows": 8192,
           "fetch_bytes_per_dispatch": 10.0, "write_bytes_per_dispatch": 5.0}
    (tmp_path / "rec.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.counter_traffic("kernel.hip", "rec.json", 8192) == 15
    assert bench.counter_traffic("kernel.hip", "rec.json", 2048) is None
    src.write_bytes(b"kernel v2")
    assert bench.counter_traffic("kernel.hip", "rec.json", 8192) is None
    assert bench.counter_traffic("kernel.hip", "missing.json", 8192) is None


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
