"""The decode attention entry point that allocates nothing
(dsa_sparse_attn_decode_noalloc: split partials in the library's fixed
per-GPU scratch) against dsa_sparse_attn_decode with a caller workspace,
through the C ABI: bitwise equal on two calls in a row, the second with a
smaller batch and shorter caches, so the scratch holds the first call's
partials when the second starts."""
import numpy as np
import pytest

import synth

from _gpu import device_workload, log, to_dev

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("needs a GPU", allow_module_level=True)

import long_context_sparse_score_amd as dsa  # noqa: E402
from long_context_sparse_score_amd import pipeline  # noqa: E402


def _case(lk, topk, seed):
    wl = synth.Workload(name="noalloc", seed=seed, seqlens_q=(1,) * len(lk), seqlens_k=tuple(lk),
                        n_heads_q=32, n_heads_kv=4, head_dim=128, n_heads_idx=64, d_idx=128,
                        topk=topk, integer_indexer=False, clustered=False)
    _, dev = device_workload(wl)
    vl = dsa.Varlen(wl.cu_q.tolist(), wl.cu_k.tolist())
    bufs = pipeline.alloc_decode(vl, wl.n_heads_q, wl.head_dim, wl.topk)
    dsa.dsa_index_scores(vl, dev["q_idx"], dev["k_idx"], dev["w"], bufs.scores)
    dsa.dsa_topk(vl, bufs.scores, bufs.indices)
    return wl, vl, dev, bufs


def _both(wl, vl, dev, bufs):
    shape = (wl.batch, wl.n_heads_q, wl.head_dim)
    ref = torch.full(shape, 7.0, dtype=torch.bfloat16, device="cuda")
    ref_lse = torch.zeros((wl.batch, wl.n_heads_q), dtype=torch.float32, device="cuda")
    got = torch.full(shape, -7.0, dtype=torch.bfloat16, device="cuda")
    got_lse = torch.ones((wl.batch, wl.n_heads_q), dtype=torch.float32, device="cuda")
    dsa.dsa_sparse_attn_decode(vl, dev["q"], dev["k"], dev["v"], bufs.indices, ref,
                               bufs.workspaces[0], lse=ref_lse)
    dsa.dsa_sparse_attn_decode_noalloc(vl, dev["q"], dev["k"], dev["v"], bufs.indices, got,
                                       lse=got_lse)
    torch.cuda.synchronize()
    return ref, ref_lse, got, got_lse


def test_noalloc_decode_matches_workspace_decode_twice():
    first = _case([9000, 2049, 131072, 300] * 16, 2048, seed=41)   # 64 queries, split partials
    log("no-alloc decode: 64 queries, caches up to 131072")
    r1 = _both(*first)
    second = _case([5000, 700, 2100], 2048, seed=42)              # smaller: 3 queries
    log("no-alloc decode: 3 queries")
    r2 = _both(*second)
    for ref, ref_lse, got, got_lse in (r1, r2):
        assert torch.equal(ref.view(torch.int16), got.view(torch.int16))
        assert torch.equal(ref_lse, got_lse)
    # the second call's rows went through the split path too (partials in the scratch)
    ws = dsa.dsa_sparse_attn_decode_workspace_size(second[1], 32, 128, 2048)
    assert ws > 0
