"""Device-side precondition checks (dsa_check_* and the DSA_CHECK flag): every
kind of bad metadata, index list and score row is reported with the first
offending sequence or row, valid inputs pass, and checked entry points give
the same results as unchecked ones.  Bad inputs go only to the check kernels
(or to entry points whose kernels treat them as defined cases)."""
import numpy as np
import pytest

import synth

from _gpu import device_workload, from_dev_bf16, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402


@pytest.fixture(autouse=True)
def _checks_off_by_default(monkeypatch):
    monkeypatch.delenv("DSA_CHECK", raising=False)


def expect_invalid(fn, *args, match, **kw):
    with pytest.raises(dsa.DSAError) as e:
        fn(*args, **kw)
    assert e.value.status == dsa.DSA_ERR_INVALID_ARGUMENT
    assert match in str(e.value), str(e.value)


# Three sequences: 2 queries over 4 keys each (host fields stay these).
CU_Q = [0, 2, 4, 6]
CU_K = [0, 4, 8, 12]


@pytest.mark.parametrize("which,bad,match", [
    ("q", [1, 2, 4, 6], "must be 0"),
    ("k", [0, 4, 3, 12], "decrease at sequence 1"),
    ("k", [0, 4, 5, 12], "sequence 1 has more queries than keys"),
    ("q", [0, 1, 4, 6], "sequence 1 is longer than max_seqlen"),
    ("k", [0, 4, 8, 11], "differs from total"),
])
def test_check_varlen_reports_the_first_bad_sequence(which, bad, match):
    vl = dsa.Varlen(CU_Q, CU_K)
    log(f"check_varlen {which}={bad}")
    dsa.dsa_check_varlen(vl)
    (vl.cu_q if which == "q" else vl.cu_k).copy_(torch.tensor(bad, dtype=torch.int32))
    expect_invalid(dsa.dsa_check_varlen, vl, match=match)


def causal_index_rows(cu_q, cu_k, topk, seed):
    """Valid index rows: a random set of distinct causal positions per query
    row, shuffled, padded with -1."""
    rng = np.random.default_rng(seed)
    rows = []
    for b in range(len(cu_q) - 1):
        lq, lk = cu_q[b + 1] - cu_q[b], cu_k[b + 1] - cu_k[b]
        for i in range(lq):
            p = lk - lq + i
            sel = rng.choice(p + 1, size=min(topk - 2, p + 1), replace=False).astype(np.int32)
            row = np.full(topk, -1, np.int32)
            row[:len(sel)] = sel
            rng.shuffle(row)
            rows.append(row)
    return np.stack(rows)


def test_check_indices_range_and_repeats():
    cu_q, cu_k = [0, 50, 80], [0, 50, 100]
    vl = dsa.Varlen(cu_q, cu_k)
    idx = causal_index_rows(cu_q, cu_k, 24, seed=3)
    log("check_indices on 80 rows")
    dsa.dsa_check_indices(vl, to_dev(idx))

    bad = idx.copy()
    bad[37, 5] = 38                      # row 37 sees positions 0..37
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(bad), match="row 37: an index")
    bad = idx.copy()
    bad[60, 0] = -2                      # neither -1 nor a position
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(bad), match="row 60: an index")
    bad = idx.copy()
    j = int(np.nonzero(bad[12] >= 0)[0][0])
    k = int(np.nonzero(bad[12] == -1)[0][0])
    bad[12, k] = bad[12, j]              # a repeat in place of padding
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(bad), match="row 12 lists a position twice")
    bad[3, 0] = 99                       # an earlier row wins the report
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(bad), match="row 3: an index")

    # A window: rows 40..79 only; the report names the packed row.
    win = idx[40:].copy()
    dsa.dsa_check_indices(vl, to_dev(win), row_begin=40)
    win[25, 1] = 200
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(win), row_begin=40, match="row 65: an index")
    # Packed row 60 is local query 10 of sequence 1: p = 50 - 30 + 10 = 30.
    win = idx[40:].copy()
    win[20, 0] = 31
    expect_invalid(dsa.dsa_check_indices, vl, to_dev(win), row_begin=40, match="row 60: an index")


def test_check_indices_repeats_beyond_the_first_bitmap_span():
    """One query over 600000 keys: repeats are found in the first and in a
    later span of the duplicate bitmap (262144 positions per pass)."""
    vl = dsa.Varlen([0, 1], [0, 600000])
    rng = np.random.default_rng(5)
    row = np.sort(rng.choice(600000, size=2047, replace=False)).astype(np.int32)
    idx = np.concatenate([row, [-1]]).astype(np.int32)[None, :]
    dsa.dsa_check_indices(vl, to_dev(idx))
    for pos in (7, 300001, 599999):
        bad = idx.copy()
        bad[0, :2] = pos
        expect_invalid(dsa.dsa_check_indices, vl, to_dev(bad), match="row 0 lists a position twice")


def test_check_scores_only_reads_the_causal_columns():
    cu = [0, 40, 100]
    vl = dsa.Varlen(cu, cu)
    rows = []
    for b in range(2):
        for i in range(cu[b + 1] - cu[b]):
            r = np.random.default_rng(i).standard_normal(64).astype(np.float32)
            r[i + 1:] = np.nan                # beyond p: never read
            rows.append(r)
    s = np.stack(rows)
    dsa.dsa_check_scores(vl, to_dev(s))
    for val, row, col in ((np.nan, 20, 20), (np.inf, 70, 3), (-np.inf, 99, 59)):
        bad = s.copy()
        bad[row, col] = val
        expect_invalid(dsa.dsa_check_scores, vl, to_dev(bad), match=f"row {row}: a score")
    bad = s.copy()
    bad[50, 5] = np.nan
    expect_invalid(dsa.dsa_check_scores, vl, to_dev(bad[40:]), row_begin=40,
                   match="row 50: a score")


def test_checked_entry_points_match_unchecked_and_stop_on_bad_input(monkeypatch):
    wl = synth.prefill_2k_int()
    host, dev = device_workload(wl)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())

    def run():
        bufs = pipeline.alloc_prefill(vl, wl.topk, window=1024)
        out = torch.zeros((wl.total_q, wl.n_heads_q, wl.head_dim), dtype=torch.bfloat16,
                          device="cuda")
        keep = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
        pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"],
                         out, bufs, keep_indices=keep)
        torch.cuda.synchronize()
        return from_dev_bf16(out), keep.cpu().numpy()

    log("prefill_2k_int unchecked, then with DSA_CHECK=1")
    plain = run()
    monkeypatch.setenv("DSA_CHECK", "1")
    checked = run()
    assert np.array_equal(plain[0], checked[0])
    assert np.array_equal(plain[1], checked[1])

    # A repeated index: the checked call fails and writes nothing.
    idx = plain[1][:64].copy()
    idx[10, 1] = idx[10, 0]
    out = torch.full((wl.total_q, wl.n_heads_q, wl.head_dim), 5.0, dtype=torch.bfloat16,
                     device="cuda")
    expect_invalid(dsa.dsa_sparse_attn_prefill, vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out,
                   row_count=64, match="row 10 lists a position twice")
    torch.cuda.synchronize()
    assert bool((out == 5.0).all())

    # A NaN score among the causal columns: dsa_topk fails and writes nothing.
    scores = np.random.default_rng(1).standard_normal((8, wl.total_k)).astype(np.float32)
    scores[6, 3] = np.nan
    sel = torch.full((8, wl.topk), -7, dtype=torch.int32, device="cuda")
    expect_invalid(dsa.dsa_topk, vl, to_dev(scores), sel, match="row 6: a score")
    torch.cuda.synchronize()
    assert bool((sel == -7).all())

    # DSA_CHECK=0 is off: the same list runs (a repeat is a defined case for
    # the kernel, it simply counts twice).
    monkeypatch.setenv("DSA_CHECK", "0")
    dsa.dsa_sparse_attn_prefill(vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out, row_count=64)
    torch.cuda.synchronize()
    assert not bool((out[:64] == 5.0).all())
