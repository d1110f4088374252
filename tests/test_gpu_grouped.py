"""GPU parity of the grouped prefill attention (16 adjacent rows served from
the union of their index sets) against the CPU oracle's per-row attention,
and of the union itself against numpy on the same index rows.  Every call
goes through the C ABI (libdsa.so)."""
import numpy as np
import pytest

import oracle
import synth

from _gpu import check_attn, device_workload, from_dev_bf16, log, oracle_rows, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - collected on CPU-only hosts
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402

GROUP = 16


def small_wl(lq, lk, hq, hkv, d, topk, qstd=0.0, seed=11, hi=8, di=64):
    return synth.Workload(name="test", seed=seed, seqlens_q=tuple(lq), seqlens_k=tuple(lk),
                          n_heads_q=hq, n_heads_kv=hkv, head_dim=d, n_heads_idx=hi, d_idx=di,
                          topk=topk, clustered=True, query_mean_std=qstd)


def run_grouped(wl, dev, idx, row_begin=0, row_count=None):
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    row_count = idx.shape[0] if row_count is None else row_count
    nbytes = dsa.dsa_sparse_attn_prefill_grouped_workspace_size(vl, row_count, wl.topk)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    out = torch.full((wl.total_q, wl.n_heads_q, wl.head_dim), 7.0, dtype=torch.bfloat16,
                     device="cuda")
    lse = torch.zeros((wl.total_q, wl.n_heads_q), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attn_prefill_grouped(vl, dev["q"], dev["k"], dev["v"], to_dev(idx), out, ws,
                                        lse=lse, row_begin=row_begin, row_count=row_count)
    torch.cuda.synchronize()
    return out, lse, ws


def workspace_counts(ws, row_count, topk):
    """The per-group union sizes at the end of the workspace (keys int32 and
    masks uint16 regions, each rounded up to 256 bytes, then one int32 per group)."""
    groups = (row_count + GROUP - 1) // GROUP
    n = groups * GROUP * topk
    off = -(-n * 4 // 256) * 256 + -(-n * 2 // 256) * 256
    raw = ws[off:off + 4 * groups].cpu().numpy()
    return raw.view(np.int32)


def gray_rank(b):
    """Inverse Gray code of b (prefix XOR of its bits)."""
    r = 0
    while b:
        r ^= b
        b >>= 1
    return r


def check_union_order(ws, row_count, topk, groups_keys, waves):
    """Every group's union in the workspace: exactly the distinct packed keys
    of its rows with the right 16-bit row masks, ordered by the Gray rank of
    the wave byte (bit w: one of rows w 16/waves .. (w + 1) 16/waves - 1 owns
    the key), ties in ascending key order.  groups_keys[g][r] is the array of
    packed keys of row r of group g."""
    groups = (row_count + GROUP - 1) // GROUP
    n = groups * GROUP * topk
    keys_all = ws[:n * 4].cpu().numpy().view(np.int32)
    moff = -(-n * 4 // 256) * 256
    masks_all = ws[moff:moff + n * 2].cpu().numpy().view(np.uint16)
    counts = workspace_counts(ws, row_count, topk)
    rpw = GROUP // waves
    for g in range(groups):
        own = {}
        for r, ks in enumerate(groups_keys[g]):
            for x in ks.tolist():
                own[x] = own.get(x, 0) | (1 << r)
        c = int(counts[g])
        assert c == len(own), f"group {g}: {c} != {len(own)}"
        got_k = keys_all[g * GROUP * topk:g * GROUP * topk + c]
        got_m = masks_all[g * GROUP * topk:g * GROUP * topk + c]

        def bucket(m):
            b = 0
            for w in range(waves):
                if (m >> (w * rpw)) & ((1 << rpw) - 1):
                    b |= 1 << w
            return gray_rank(b)

        want = sorted(own, key=lambda x: (bucket(own[x]), x))
        np.testing.assert_array_equal(got_k, np.array(want, np.int32), err_msg=f"group {g}")
        np.testing.assert_array_equal(got_m, np.array([own[x] for x in want], np.uint16))


@pytest.mark.parametrize("hq,hkv,d", [(32, 4, 128), (8, 1, 128), (8, 2, 64), (8, 8, 64),
                                      (8, 4, 128), (16, 2, 64), (32, 8, 64), (4, 4, 128)])
def test_grouped_matches_oracle_varlen(hq, hkv, d):
    """Groups straddling sequences, a partial last group, rows shorter than k
    (-1 padding), 1, 2, 4 and 8 query heads per KV head."""
    wl = small_wl([37, 100, 1, 250], [60, 100, 5, 250], hq, hkv, d, topk=64, qstd=3.0,
                  seed=hq + d)
    host, dev = device_workload(wl)
    rows = np.arange(wl.total_q)
    ref = oracle_rows(wl, host, rows)
    log(f"grouped attention hq={hq} hkv={hkv} d={d}")
    out, lse, ws = run_grouped(wl, dev, ref["idx"])
    mx, mean = check_attn(from_dev_bf16(out), ref["out"])
    log(f"  max abs {mx:.2e} mean abs {mean:.2e}")
    assert np.allclose(lse.cpu().numpy(), ref["lse"], atol=2e-3)
    # The unions: distinct packed keys over each group's rows, their masks
    # and their order.
    cu_k = wl.cu_k
    seq = np.searchsorted(wl.cu_q, rows, side="right") - 1
    packed = [cu_k[seq[r]] + ref["idx"][r][ref["idx"][r] >= 0] for r in rows]
    check_union_order(ws, wl.total_q, wl.topk,
                      [packed[g:g + GROUP] for g in range(0, len(rows), GROUP)], hq // hkv)


def test_grouped_row_window_and_long_rows():
    """A window that starts mid-sequence (groups are formed from row_begin),
    rows longer than one union span (8192 keys) and k = 2048."""
    wl = small_wl([9000], [9000], 32, 4, 128, topk=2048, qstd=4.0, seed=5, hi=16, di=64)
    host, dev = device_workload(wl)
    rows = np.arange(8700, 9000)
    ref = oracle_rows(wl, host, rows)
    log("grouped attention, window of 300 rows at 8700 over 9000 keys")
    out, lse, ws = run_grouped(wl, dev, ref["idx"], row_begin=8700, row_count=300)
    got = from_dev_bf16(out)[8700:9000]
    mx, mean = check_attn(got, ref["out"])
    log(f"  max abs {mx:.2e} mean abs {mean:.2e}")
    assert np.allclose(lse.cpu().numpy()[8700:9000], ref["lse"], atol=2e-3)
    untouched = from_dev_bf16(out)[:8700]
    assert (untouched == 0x40E0).all()  # 7.0 in bf16: rows outside the window stay
    packed = [ref["idx"][i][ref["idx"][i] >= 0] for i in range(300)]
    check_union_order(ws, 300, wl.topk, [packed[g:g + GROUP] for g in range(0, 300, GROUP)], 8)


def test_grouped_any_row_order_and_long_lists():
    """Index rows in any order give the same union and bitwise the same
    output (the union's order depends on the sets only), also for k = 3000,
    more entries per row than the union pass holds at once, whose rows here
    see about 40000 keys: more than one 32768-key span of the union pass."""
    wl = small_wl([40000], [40000], 32, 4, 128, topk=3000, qstd=4.0, seed=21, hi=16, di=64)
    host, dev = device_workload(wl)
    r0 = 39900
    rows = np.arange(r0, r0 + 100)
    ref = oracle_rows(wl, host, rows)
    log("grouped attention, k = 3000, rows 39900..39999, ascending then shuffled index rows")
    out_a, lse_a, ws = run_grouped(wl, dev, ref["idx"], row_begin=r0, row_count=100)
    mx, mean = check_attn(from_dev_bf16(out_a)[r0:r0 + 100], ref["out"])
    log(f"  max abs {mx:.2e} mean abs {mean:.2e}")
    packed = [ref["idx"][i][ref["idx"][i] >= 0] for i in range(100)]
    check_union_order(ws, 100, wl.topk, [packed[g:g + GROUP] for g in range(0, 100, GROUP)], 8)
    rng = np.random.default_rng(0)
    shuffled = np.stack([rng.permutation(r) for r in ref["idx"]])
    out_b, lse_b, ws_b = run_grouped(wl, dev, shuffled, row_begin=r0, row_count=100)
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    check_union_order(ws_b, 100, wl.topk, [packed[g:g + GROUP] for g in range(0, 100, GROUP)], 8)


def test_grouped_equals_per_row_pipeline_end_to_end():
    """The prefill pipeline with the grouped attention against the oracle on a
    correlated-query clustered workload (indices from the GPU top-k)."""
    wl = small_wl([1500, 700], [1500, 700], 32, 4, 128, topk=512, qstd=4.0, seed=8, hi=64,
                  di=128)
    host, dev = device_workload(wl)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    bufs = pipeline.alloc_prefill(vl, wl.topk, window=800, grouped=True)
    out = torch.zeros((wl.total_q, 32, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((wl.total_q, 32), dtype=torch.float32, device="cuda")
    keep = torch.zeros((wl.total_q, wl.topk), dtype=torch.int32, device="cuda")
    pipeline.prefill(vl, dev["q_idx"], dev["k_idx"], dev["w"], dev["q"], dev["k"], dev["v"], out,
                     bufs, lse=lse, keep_indices=keep)
    torch.cuda.synchronize()
    rows = np.arange(wl.total_q)
    sel = keep.cpu().numpy()
    ref_out, ref_lse = oracle.sparse_attn(wl.cu_q, wl.cu_k, host["q"], host["k"], host["v"], sel,
                                          rows, wl.softmax_scale)
    mx, mean = check_attn(from_dev_bf16(out), ref_out)
    log(f"  pipeline grouped: max abs {mx:.2e} mean abs {mean:.2e}")
    assert np.allclose(lse.cpu().numpy(), ref_lse, atol=2e-3)
