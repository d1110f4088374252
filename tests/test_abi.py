"""The C ABI of libdsa.so without a GPU: the library loads, exports every
declared entry point, and rejects bad arguments on the host before any launch."""
import ctypes
import os
import re
import subprocess

import pytest

import long_context_sparse_score_amd as dsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dsa.h")

FAKE = 0x7F0000000000  # a 256-byte aligned address; never dereferenced on these paths


@pytest.fixture(autouse=True)
def _no_device_checks(monkeypatch):
    """The calls below must stop on the host: device-side checking stays off."""
    monkeypatch.delenv("DSA_CHECK", raising=False)


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\*?(dsa_\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("dsa_index_scores", "dsa_topk", "dsa_sparse_attn_prefill",
              "dsa_sparse_attn_decode"):
        assert n in names
    assert set(names) == set(dsa.EXPORTED)


def test_library_exports_every_declared_symbol():
    out = subprocess.run(["nm", "-D", "--defined-only", dsa.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared_functions():
        assert name in exported, name
    lib = dsa.load_library()
    for name in declared_functions():
        assert hasattr(lib, name)


def test_library_is_gfx950_only():
    """The embedded offload bundle names gfx950 and no other GPU target."""
    blob = open(dsa.LIB_PATH, "rb").read()
    targets = set(re.findall(rb"amdgcn-amd-amdhsa-+(gfx[0-9a-z]+)", blob))
    assert targets == {b"gfx950"}


def test_status_strings():
    lib = dsa.load_library()
    assert lib.dsa_status_string(0) == b"DSA_OK"
    assert lib.dsa_status_string(3) == b"DSA_ERR_WORKSPACE"
    assert lib.dsa_status_string(99) == b"DSA_ERR_UNKNOWN"


def vl(batch=1, total_q=100, total_k=100, max_q=100, max_k=100, cu=FAKE):
    return dsa.dsa_varlen(batch, cu, cu + 256, total_q, total_k, max_q, max_k)


def call_scores(v, q=FAKE, k=FAKE, w=FAKE, heads=64, d=128, rb=0, rc=10, s=FAKE, ld=128):
    lib = dsa.load_library()
    return lib.dsa_index_scores(ctypes.byref(v), q, k, w, heads, d, rb, rc, s, ld, None)


def test_index_scores_validation():
    lib = dsa.load_library()
    I, U = dsa.DSA_ERR_INVALID_ARGUMENT, dsa.DSA_ERR_UNSUPPORTED
    assert call_scores(vl(), rc=0) == dsa.DSA_OK  # empty window: no launch
    assert lib.dsa_index_scores(None, FAKE, FAKE, FAKE, 64, 128, 0, 1, FAKE, 128, None) == I
    assert call_scores(vl(batch=0)) == I
    assert call_scores(vl(cu=0)) == I
    assert call_scores(vl(), q=None) == I
    assert call_scores(vl(), q=FAKE + 2) == I          # bf16 must be 16-byte aligned
    assert call_scores(vl(), s=FAKE + 4) == I          # scores 16-byte aligned
    assert call_scores(vl(), ld=96) == I               # ld < max_seqlen_k
    assert call_scores(vl(), ld=102) == I              # ld multiple of 4
    assert call_scores(vl(), rb=95, rc=10) == I        # window beyond total_q
    assert call_scores(vl(), rb=-1) == I
    assert call_scores(vl(), d=96) == U
    assert call_scores(vl(), heads=65) == U
    assert call_scores(vl(), heads=0) == U
    assert b"d_idx" in lib.dsa_last_error() or True
    assert call_scores(vl(), d=96) == U and b"d_idx 96" in lib.dsa_last_error()


def test_topk_validation():
    lib = dsa.load_library()
    v = vl()
    n = ctypes.c_size_t(123)
    assert lib.dsa_topk_workspace_size(ctypes.byref(v), 10, 2048, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.dsa_topk_workspace_size(ctypes.byref(v), 10, 4096, ctypes.byref(n)) == \
        dsa.DSA_ERR_UNSUPPORTED
    args = lambda **kw: dict(dict(s=FAKE, ld=128, rb=0, rc=10, k=64, idx=FAKE), **kw)

    def call(**kw):
        a = args(**kw)
        return lib.dsa_topk(ctypes.byref(v), a["s"], a["ld"], a["rb"], a["rc"], a["k"], a["idx"],
                            None, 0, None)
    assert call(rc=0) == dsa.DSA_OK
    assert call(k=0) == dsa.DSA_ERR_UNSUPPORTED
    assert call(k=2049) == dsa.DSA_ERR_UNSUPPORTED
    assert call(idx=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(idx=FAKE + 2) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(s=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(ld=64) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(rb=91) == dsa.DSA_ERR_INVALID_ARGUMENT


def test_topk_needs_no_workspace():
    """Every call shape reports 0 workspace bytes (few long rows included), and
    a NULL workspace is accepted."""
    lib = dsa.load_library()
    n = ctypes.c_size_t(123)
    dec = vl(batch=64, total_q=64, total_k=64 * 131072, max_q=1, max_k=131072)
    assert lib.dsa_topk_workspace_size(ctypes.byref(dec), 64, 2048, ctypes.byref(n)) == 0
    assert n.value == 0
    pre = vl(total_q=131072, total_k=131072, max_q=131072, max_k=131072)
    assert lib.dsa_topk_workspace_size(ctypes.byref(pre), 8192, 2048, ctypes.byref(n)) == 0
    assert n.value == 0


def test_attention_validation():
    lib = dsa.load_library()
    v = vl()

    def pre(hq=32, hkv=4, d=128, topk=2048, scale=0.088, q=FAKE, out=FAKE, lse=None, rc=5):
        return lib.dsa_sparse_attn_prefill(ctypes.byref(v), q, FAKE, FAKE, FAKE, topk, 0, rc, hq,
                                           hkv, d, scale, out, lse, None)
    assert pre(rc=0) == dsa.DSA_OK
    assert pre(hq=30) == dsa.DSA_ERR_INVALID_ARGUMENT      # not a multiple of hkv
    assert pre(d=96) == dsa.DSA_ERR_UNSUPPORTED
    assert pre(hkv=16, hq=32) == dsa.DSA_ERR_UNSUPPORTED   # more than 8 KV heads
    assert pre(hq=68, hkv=4) == dsa.DSA_ERR_UNSUPPORTED    # group of 17
    assert pre(topk=0) == dsa.DSA_ERR_UNSUPPORTED
    assert pre(topk=5000) == dsa.DSA_ERR_UNSUPPORTED
    assert pre(scale=float("nan")) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert pre(q=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert pre(out=FAKE + 8) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert pre(lse=FAKE + 2) == dsa.DSA_ERR_INVALID_ARGUMENT

    dv = vl(batch=64, total_q=64, total_k=64 * 1000, max_q=1, max_k=1000)
    need = ctypes.c_size_t(0)
    assert lib.dsa_sparse_attn_decode_workspace_size(ctypes.byref(dv), 64, 32, 128, 2048,
                                                     ctypes.byref(need)) == 0
    assert need.value > 0
    half = ctypes.c_size_t(0)
    assert lib.dsa_sparse_attn_decode_workspace_size(ctypes.byref(dv), 32, 32, 128, 2048,
                                                     ctypes.byref(half)) == 0
    assert 0 < half.value
    assert lib.dsa_sparse_attn_decode_workspace_size(ctypes.byref(dv), 65, 32, 128, 2048,
                                                     ctypes.byref(half)) == \
        dsa.DSA_ERR_INVALID_ARGUMENT                      # more rows than the batch

    def dec(ws=FAKE, ws_bytes=None, vv=dv, rb=0, rc=64):
        b = need.value if ws_bytes is None else ws_bytes
        return lib.dsa_sparse_attn_decode(ctypes.byref(vv), FAKE, FAKE, FAKE, FAKE, 2048, rb, rc,
                                          32, 4, 128, 0.088, FAKE, None, ws, b, None)
    assert dec(ws=None) == dsa.DSA_ERR_WORKSPACE
    assert dec(ws_bytes=need.value - 1) == dsa.DSA_ERR_WORKSPACE
    assert dec(ws=FAKE + 64) == dsa.DSA_ERR_WORKSPACE       # 256-byte alignment
    assert dec(vv=vl()) == dsa.DSA_ERR_INVALID_ARGUMENT     # more than one query per sequence
    assert dec(rb=40, rc=30) == dsa.DSA_ERR_INVALID_ARGUMENT  # window past the batch
    assert dec(rb=10, rc=0, ws=None) == dsa.DSA_OK            # empty window: nothing to do

    # A sequence whose K (or V) rows pass 2 GiB: the kernels address one
    # sequence with 32-bit byte offsets, so the host refuses it (3M tokens x
    # 4 KV heads x 128 x 2 bytes = 3 GB), even for an empty prefill window.
    big = vl(batch=1, total_q=1, total_k=3_000_000, max_q=1, max_k=3_000_000)
    assert lib.dsa_sparse_attn_prefill(ctypes.byref(big), FAKE, FAKE, FAKE, FAKE, 2048, 0, 0, 32,
                                       4, 128, 0.088, FAKE, None, None) == dsa.DSA_ERR_UNSUPPORTED
    assert dec(vv=big, rc=1) == dsa.DSA_ERR_UNSUPPORTED
    ok_size = vl(batch=1, total_q=1, total_k=2_000_000, max_q=1, max_k=2_000_000)  # 2.05e9 bytes
    assert lib.dsa_sparse_attn_prefill(ctypes.byref(ok_size), FAKE, FAKE, FAKE, FAKE, 2048, 0, 0,
                                       32, 4, 128, 0.088, FAKE, None, None) == dsa.DSA_OK


def test_varlen_struct_layout():
    assert ctypes.sizeof(dsa.dsa_varlen) == 48
    assert dsa.dsa_varlen.cu_seqlens_q.offset == 8
    assert dsa.dsa_varlen.total_q.offset == 24
    assert dsa.dsa_varlen.max_seqlen_k.offset == 44


def test_check_entry_points_validate_on_the_host():
    """The device-side checks reject bad descriptors, windows and pointers on
    the host, before any HIP call."""
    lib = dsa.load_library()
    I = dsa.DSA_ERR_INVALID_ARGUMENT
    v = vl()
    assert lib.dsa_check_varlen(None, None) == I
    assert lib.dsa_check_varlen(ctypes.byref(vl(batch=0)), None) == I
    assert lib.dsa_check_varlen(ctypes.byref(vl(cu=0)), None) == I
    assert lib.dsa_check_indices(ctypes.byref(v), None, 64, 0, 10, None) == I
    assert lib.dsa_check_indices(ctypes.byref(v), FAKE + 2, 64, 0, 10, None) == I
    assert lib.dsa_check_indices(ctypes.byref(v), FAKE, 0, 0, 10, None) == I
    assert lib.dsa_check_indices(ctypes.byref(v), FAKE, 64, 95, 10, None) == I
    assert b"row window" in lib.dsa_last_error()
    assert lib.dsa_check_scores(ctypes.byref(v), None, 128, 0, 10, None) == I
    assert lib.dsa_check_scores(ctypes.byref(v), FAKE, 96, 0, 10, None) == I
    assert lib.dsa_check_scores(ctypes.byref(v), FAKE, 128, -1, 10, None) == I


def test_checked_calls_still_reject_bad_arguments_on_the_host(monkeypatch):
    """With DSA_CHECK on, host validation still comes first: these calls fail
    before the device-side checks would run."""
    monkeypatch.setenv("DSA_CHECK", "1")
    lib = dsa.load_library()
    assert call_scores(vl(), d=96) == dsa.DSA_ERR_UNSUPPORTED
    assert lib.dsa_topk(ctypes.byref(vl()), FAKE, 64, 0, 10, 64, FAKE, None, 0, None) == \
        dsa.DSA_ERR_INVALID_ARGUMENT
    assert lib.dsa_sparse_attn_prefill(ctypes.byref(vl()), FAKE, FAKE, FAKE, FAKE, 0, 0, 5, 32, 4,
                                       128, 0.088, FAKE, None, None) == dsa.DSA_ERR_UNSUPPORTED


def test_fp8_entry_points_validate_on_the_host():
    lib = dsa.load_library()
    I, U = dsa.DSA_ERR_INVALID_ARGUMENT, dsa.DSA_ERR_UNSUPPORTED
    q = lib.dsa_quantize_fp8
    assert q(FAKE, 0, 128, FAKE, FAKE, None) == dsa.DSA_OK          # nothing to do
    assert q(None, 10, 128, FAKE, FAKE, None) == I
    assert q(FAKE + 2, 10, 128, FAKE, FAKE, None) == I
    assert q(FAKE, 10, 128, FAKE + 8, FAKE, None) == I              # codes 16-byte aligned
    assert q(FAKE, 10, 128, FAKE, FAKE + 2, None) == I
    assert q(FAKE, -1, 128, FAKE, FAKE, None) == I
    assert q(FAKE, 10, 96, FAKE, FAKE, None) == U

    def s8(v=None, qc=FAKE, qs=FAKE, kc=FAKE, ks=FAKE, w=FAKE, heads=64, d=128, rb=0, rc=10,
           sc=FAKE, ld=128):
        v = vl() if v is None else v
        return lib.dsa_index_scores_fp8(ctypes.byref(v), qc, qs, kc, ks, w, heads, d, rb, rc, sc,
                                        ld, None)
    assert s8(rc=0) == dsa.DSA_OK
    assert s8(qc=FAKE + 8) == I
    assert s8(kc=None) == I
    assert s8(ks=FAKE + 1) == I
    assert s8(w=None) == I
    assert s8(ld=96) == I
    assert s8(rb=95) == I
    assert s8(d=32) == U
    assert s8(heads=65) == U
    # One sequence's key codes beyond 2 GiB: 20M keys x 128 bytes.
    big = vl(total_q=1, total_k=20_000_000, max_q=1, max_k=20_000_000)
    assert s8(v=big, rc=1, ld=20_000_000) == U


def test_index_scores_key_extent_limit():
    """The bf16 indexer addresses one sequence's keys with 32-bit offsets:
    9M keys x 128 x 2 bytes pass 2 GiB and are refused on the host."""
    big = vl(total_q=1, total_k=9_000_000, max_q=1, max_k=9_000_000)
    assert call_scores(big, rc=1, ld=9_000_000) == dsa.DSA_ERR_UNSUPPORTED
    ok_size = vl(total_q=1, total_k=8_000_000, max_q=1, max_k=8_000_000)
    assert call_scores(ok_size, rc=0, ld=8_000_000) == dsa.DSA_OK


def test_grouped_attention_validation():
    lib = dsa.load_library()
    v = vl(total_q=100, total_k=100, max_q=100, max_k=100)
    n = ctypes.c_size_t(0)
    assert lib.dsa_sparse_attn_prefill_grouped_workspace_size(ctypes.byref(v), 100, 2048,
                                                              ctypes.byref(n)) == 0
    assert n.value > 0
    need = n.value
    assert lib.dsa_sparse_attn_prefill_grouped_workspace_size(ctypes.byref(v), 0, 2048,
                                                              ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.dsa_sparse_attn_prefill_grouped_workspace_size(ctypes.byref(v), 101, 2048,
                                                              ctypes.byref(n)) == \
        dsa.DSA_ERR_INVALID_ARGUMENT

    def call(ws=FAKE, ws_bytes=None, vv=v, rc=100, hq=32, hkv=4, topk=2048):
        b = need if ws_bytes is None else ws_bytes
        return lib.dsa_sparse_attn_prefill_grouped(ctypes.byref(vv), FAKE, FAKE, FAKE, FAKE, topk,
                                                   0, rc, hq, hkv, 128, 0.088, FAKE, None, ws, b,
                                                   None)
    assert call(rc=0, ws=None) == dsa.DSA_OK
    assert call(ws=None) == dsa.DSA_ERR_WORKSPACE
    assert call(ws_bytes=need - 1) == dsa.DSA_ERR_WORKSPACE
    assert call(ws=FAKE + 64) == dsa.DSA_ERR_WORKSPACE
    assert call(hq=30) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(hq=24, hkv=8) == dsa.DSA_ERR_UNSUPPORTED   # 3 query heads per KV head
    assert call(hq=64, hkv=4) == dsa.DSA_ERR_UNSUPPORTED   # 16 query heads per KV head
    assert call(topk=5000) == dsa.DSA_ERR_UNSUPPORTED
    # all K rows beyond 2 GiB (the grouped kernels use one 32-bit offset space)
    big = vl(total_q=100, total_k=3_000_000, max_q=100, max_k=3_000_000)
    assert call(vv=big) == dsa.DSA_ERR_UNSUPPORTED


def test_indexer_kl_validation():
    """Host-side checks of dsa_indexer_kl (no kernel is launched: every call
    below fails before, or has an empty window)."""
    lib = dsa.load_library()
    v = vl(total_q=100, total_k=100, max_q=100, max_k=100)

    def call(q=FAKE, scores=FAKE, ld=128, loss=FAKE, grad=None, ld_grad=0, rc=100, hq=32, hkv=4,
             d=128, scale=0.088):
        return lib.dsa_indexer_kl(ctypes.byref(v), q, FAKE, scores, ld, 0, rc, hq, hkv, d, scale,
                                  loss, grad, ld_grad, None)
    assert call(rc=0) == dsa.DSA_OK
    assert call(q=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(scores=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(loss=None) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(ld=96) == dsa.DSA_ERR_INVALID_ARGUMENT           # < max_seqlen_k
    assert call(grad=FAKE, ld_grad=64) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(grad=FAKE, ld_grad=132) == dsa.DSA_ERR_INVALID_ARGUMENT  # in place, other ld
    assert call(hq=24, hkv=8) == dsa.DSA_ERR_UNSUPPORTED         # not a power of two
    assert call(hq=128, hkv=8) == dsa.DSA_ERR_UNSUPPORTED
    assert call(d=96) == dsa.DSA_ERR_UNSUPPORTED
    assert call(scale=float("nan")) == dsa.DSA_ERR_INVALID_ARGUMENT
    assert call(scale=-0.1) == dsa.DSA_ERR_UNSUPPORTED


# ---- binding extent checks (host only: CPU tensors, the device check comes last)

def _bf(*shape):
    import torch

    return torch.zeros(shape, dtype=torch.bfloat16)


def _f32(*shape):
    import torch

    return torch.zeros(shape, dtype=torch.float32)


def _i32(*shape):
    import torch

    return torch.zeros(shape, dtype=torch.int32)


def _cpu_varlen(cq=(0, 40, 100), ck=(0, 40, 100)):
    return dsa.Varlen(cq, ck, device="cpu")


def _expect(fn, exc=ValueError):
    with pytest.raises(exc):
        fn()


def test_binding_index_scores_extents():
    v = _cpu_varlen()
    good = dict(q_idx=_bf(100, 4, 64), k_idx=_bf(100, 64), w=_f32(100, 4), scores=_f32(16, 64))
    call = lambda **kw: dsa.dsa_index_scores(v, **{**good, **kw}, row_begin=80)  # noqa: E731
    _expect(lambda: call(), TypeError)                     # extents fine: stops at the device check
    _expect(lambda: call(q_idx=_bf(99, 4, 64)))            # q_idx rows != total_q
    _expect(lambda: call(k_idx=_bf(100, 128)))             # key width != d_idx
    _expect(lambda: call(k_idx=_bf(90, 64)))               # k_idx rows != total_k
    _expect(lambda: call(w=_f32(100, 3)))                  # w heads != n_heads_idx
    _expect(lambda: call(scores=_f32(16, 32)))             # fewer columns than max_seqlen_k
    _expect(lambda: dsa.dsa_index_scores(v, **good, row_begin=90))          # window past total_q
    _expect(lambda: dsa.dsa_index_scores(v, **good, row_begin=0, row_count=17))  # > scores rows


def test_binding_topk_extents():
    v = _cpu_varlen()
    call = lambda s, i, **kw: dsa.dsa_topk(v, s, i, **kw)  # noqa: E731
    _expect(lambda: call(_f32(8, 64), _i32(8, 16)), TypeError)
    _expect(lambda: call(_f32(8, 64), _i32(8, 16), row_count=9))
    _expect(lambda: call(_f32(4, 64), _i32(8, 16)))
    _expect(lambda: call(_f32(8, 59), _i32(8, 16)))    # fewer columns than max_seqlen_k (60)
    _expect(lambda: call(_f32(8, 64), _i32(8, 16), row_begin=95))


def test_binding_attention_extents():
    v = _cpu_varlen()
    good = dict(q=_bf(100, 8, 64), k=_bf(100, 2, 64), v=_bf(100, 2, 64), indices=_i32(10, 32),
                out=_bf(100, 8, 64), lse=_f32(100, 8))
    call = lambda **kw: dsa.dsa_sparse_attn_prefill(v, **{**good, **kw})  # noqa: E731
    _expect(lambda: call(), TypeError)
    _expect(lambda: call(q=_bf(50, 8, 64)))
    _expect(lambda: call(k=_bf(99, 2, 64)))
    _expect(lambda: call(v=_bf(100, 4, 64)))
    _expect(lambda: call(out=_bf(100, 8, 32)))
    _expect(lambda: call(lse=_f32(100, 4)))
    _expect(lambda: call(row_count=11))
    _expect(lambda: call(row_begin=95))
    ws = torch_u8(1024)
    _expect(lambda: dsa.dsa_sparse_attn_prefill_grouped(v, **{**good, "q": _bf(10, 8, 64)},
                                                        workspace=ws))
    _expect(lambda: dsa.dsa_sparse_attn_prefill_grouped(v, **good, workspace=ws), TypeError)


def torch_u8(n):
    import torch

    return torch.zeros(n, dtype=torch.uint8)


def test_binding_decode_extents():
    v = _cpu_varlen((0, 1, 2), (0, 300, 700))
    good = dict(q=_bf(2, 8, 64), k_cache=_bf(700, 2, 64), v_cache=_bf(700, 2, 64),
                indices=_i32(2, 32), out=_bf(2, 8, 64), workspace=torch_u8(1024))
    call = lambda **kw: dsa.dsa_sparse_attn_decode(v, **{**good, **kw})  # noqa: E731
    _expect(lambda: call(), TypeError)
    _expect(lambda: call(q=_bf(3, 8, 64)))
    _expect(lambda: call(k_cache=_bf(600, 2, 64)))
    _expect(lambda: call(indices=_i32(1, 32), row_count=2))
    _expect(lambda: call(lse=_f32(2, 4)))


def test_binding_kl_and_check_extents():
    v = _cpu_varlen()
    good = dict(q=_bf(100, 8, 64), k=_bf(100, 2, 64), scores=_f32(10, 64), loss=_f32(10))
    call = lambda **kw: dsa.dsa_indexer_kl(v, **{**good, **kw})  # noqa: E731
    _expect(lambda: call(), TypeError)
    _expect(lambda: call(loss=_f32(9)))
    _expect(lambda: call(grad=_f32(9, 64)))
    _expect(lambda: call(grad=_f32(10, 32)))
    _expect(lambda: call(k=_bf(100, 2, 32)))
    _expect(lambda: dsa.dsa_check_indices(v, _i32(10, 32), row_count=11))
    _expect(lambda: dsa.dsa_check_scores(v, _f32(10, 64), row_begin=95))
    _expect(lambda: dsa.dsa_check_scores(v, _f32(10, 64)), TypeError)


def test_binding_passes_no_computed_scale(monkeypatch):
    """With softmax_scale=None the binding hands the library its default
    sentinel (0) and computes nothing; the library applies 1 / sqrt(d)."""
    assert dsa._scale(None) == 0.0
    assert dsa._scale(0.25) == 0.25
    src = open(os.path.join(ROOT, "long_context_sparse_score_amd", "__init__.py")).read()
    assert "** -0.5" not in src and "math.sqrt" not in src and "** 0.5" not in src
    assert "#define DSA_SCALE_DEFAULT 0.0f" in open(HEADER).read()


def test_noalloc_decode_validation_and_limit():
    """The no-alloc decode rejects bad arguments and partials beyond its
    fixed 16 MiB scratch on the host, before touching any device."""
    lib = dsa.load_library()
    U, I = dsa.DSA_ERR_UNSUPPORTED, dsa.DSA_ERR_INVALID_ARGUMENT

    def call(batch=64, hq=32, hkv=4, d=128, topk=2048, q=FAKE, rc=None):
        v = vl(batch=batch, total_q=batch, total_k=batch * 1000, max_q=1, max_k=1000)
        return lib.dsa_sparse_attn_decode_noalloc(ctypes.byref(v), q, FAKE, FAKE, FAKE, topk, 0,
                                                  batch if rc is None else rc, hq, hkv, d, 0.0,
                                                  FAKE, None, None)

    # 64 rows x 4 splits x 128 heads x 130 x 4 B = 17.0 MB > 16 MiB
    assert call(hq=128, hkv=8) == U
    assert b"fixed scratch" in lib.dsa_last_error()
    assert call(q=None) == I
    assert call(rc=65) == I
    assert call(hq=30, hkv=4) == I
    assert call(rc=0) == dsa.DSA_OK  # empty window: nothing enqueued, no device touched


def test_index_topk_validation():
    """dsa_index_topk rejects bad arguments, a missing or small workspace,
    and unsupported k on the host; its workspace size grows with the rows."""
    lib = dsa.load_library()
    I, U, W = dsa.DSA_ERR_INVALID_ARGUMENT, dsa.DSA_ERR_UNSUPPORTED, dsa.DSA_ERR_WORKSPACE
    v = vl(total_q=100, total_k=100, max_q=100, max_k=100)
    n = ctypes.c_size_t(0)
    assert lib.dsa_index_topk_workspace_size(ctypes.byref(v), 10, 64, ctypes.byref(n)) == 0
    small = n.value
    assert lib.dsa_index_topk_workspace_size(ctypes.byref(v), 20, 64, ctypes.byref(n)) == 0
    assert n.value > small > 0
    assert lib.dsa_index_topk_workspace_size(ctypes.byref(v), 10, 4096, ctypes.byref(n)) == U
    assert lib.dsa_index_topk_workspace_size(ctypes.byref(v), 101, 64, ctypes.byref(n)) == I

    def call(q=FAKE, k=64, rc=10, ws=FAKE, wsb=1 << 40, heads=64, d=128, idx=FAKE):
        return lib.dsa_index_topk(ctypes.byref(v), q, FAKE, FAKE, heads, d, 0, rc, k, idx, ws, wsb,
                                  None)

    assert call(rc=0) == dsa.DSA_OK
    assert call(q=None) == I
    assert call(q=FAKE + 2) == I
    assert call(idx=None) == I
    assert call(k=0) == U and call(k=2049) == U
    assert call(d=96) == U and call(heads=65) == U
    assert call(ws=None) == W
    assert call(wsb=small - 1) == W
    assert call(ws=FAKE + 16) == W  # not 256-byte aligned


def test_index_backward_validation():
    """dsa_index_scores_backward rejects bad arguments, a missing or small
    workspace and unsupported shapes on the host; the workspace covers only
    the outputs asked for."""
    lib = dsa.load_library()
    I, U, W = dsa.DSA_ERR_INVALID_ARGUMENT, dsa.DSA_ERR_UNSUPPORTED, dsa.DSA_ERR_WORKSPACE
    v = vl(total_q=100, total_k=100, max_q=100, max_k=100)
    n = ctypes.c_size_t(0)

    def size(rows=10, dq=1, dk=1, heads=64, d=128):
        assert lib.dsa_index_scores_backward_workspace_size(ctypes.byref(v), heads, d, rows, dq,
                                                            dk, ctypes.byref(n)) == 0
        return n.value
    both, only_dq, only_dk = size(), size(dk=0), size(dq=0)
    assert both == only_dq + only_dk and only_dq > 0 and only_dk > 0
    assert size(rows=20, dq=0) > only_dk
    assert lib.dsa_index_scores_backward_workspace_size(ctypes.byref(v), 65, 128, 10, 1, 1,
                                                        ctypes.byref(n)) == U
    assert lib.dsa_index_scores_backward_workspace_size(ctypes.byref(v), 64, 128, 101, 1, 1,
                                                        ctypes.byref(n)) == I

    def call(q=FAKE, grad=FAKE, ld=128, dq=FAKE, dw=FAKE, dk=FAKE, rc=10, ws=FAKE, wsb=1 << 40,
             heads=64, d=128):
        return lib.dsa_index_scores_backward(ctypes.byref(v), q, FAKE, FAKE, heads, d, 0, rc, grad,
                                             ld, dq, dw, dk, ws, wsb, None)

    assert call(rc=0) == dsa.DSA_OK
    assert call(q=None) == I and call(q=FAKE + 2) == I
    assert call(grad=None) == I and call(grad=FAKE + 2) == I
    assert call(ld=99) == I                                      # < max_seqlen_k
    assert call(dw=None) == I and call(dq=None) == I             # one without the other
    assert call(dq=None, dw=None, dk=None) == I                  # nothing to compute
    assert call(dk=FAKE + 2) == I
    assert call(d=96) == U and call(heads=65) == U and call(heads=0) == U
    assert call(ws=None) == W
    assert call(wsb=both - 1) == W
    assert call(dk=None, wsb=only_dq) != W                       # only what is asked for
    assert call(ws=FAKE + 16) == W                               # not 256-byte aligned


def test_binding_backward_extents():
    v = _cpu_varlen()
    q, k, w, g = _bf(100, 64, 128), _bf(100, 128), _f32(100, 64), _f32(100, 100)
    ws = torch_u8(64)
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, _f32(100, 59), ws, dk_idx=_f32(100, 128)))
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, g, ws, dk_idx=_f32(99, 128)))
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, g, ws, dq_idx=_f32(100, 64, 64),
                                                  dw=_f32(100, 64)))
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, g, ws, dq_idx=_f32(100, 64, 128),
                                                  dw=_f32(100, 32)))
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, g[:50], ws, dk_idx=_f32(100, 128),
                                                  row_count=100))
    # shapes right: only the device check is left
    _expect(lambda: dsa.dsa_index_scores_backward(v, q, k, w, g, ws, dk_idx=_f32(100, 128)),
            TypeError)


def torch_u8(n):
    import torch

    return torch.zeros(n, dtype=torch.uint8)
