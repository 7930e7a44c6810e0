"""The C ABI library loads, exports every entry point include/sa.h declares, and rejects
invalid calls on the host before any launch (CPU only: no call here reaches a kernel)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sa.h")

from block_sparse_attention_estimate_amd import _lib  # noqa: E402


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libsa.so is not built (run __graft_entry__.build())")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(sa_\w+)", out))
    for n in names:
        assert n in exported, n
        assert getattr(lib, n) is not None


def test_status_strings(lib):
    for st in range(9):
        assert lib.sa_status_string(st) != b"unknown status"
    assert lib.sa_status_string(0) == b"ok"
    assert lib.sa_status_string(9) == b"unknown status"


def test_debug_build_exports_the_same_symbols(lib):
    """libsa_debug.so (the kernels' checks of caller data compiled in) is built beside libsa.so
    and exports every declared entry point; the release build reports no check bits."""
    if not os.path.exists(_lib.DEBUG_LIB_PATH):
        pytest.fail("libsa_debug.so is not built (run __graft_entry__.build())")
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.DEBUG_LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\sT\s(sa_\w+)", out))
    assert set(declared_functions()) <= exported
    assert lib.sa_debug_flags() == 0


def _shape(B=1, Hq=4, Hkv=1, D=128, N=256):
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim, s.seq_q, s.seq_k = B, Hq, Hkv, D, N, N
    s.q_stride[:] = (N * Hq * D, Hq * D, D)
    s.k_stride[:] = (N * Hkv * D, Hkv * D, D)
    s.v_stride[:] = (N * Hkv * D, Hkv * D, D)
    s.o_stride[:] = (N * Hq * D, Hq * D, D)
    return s


def _params(theta, Hq=4, bq=128, bk=64, gran=0):
    p = _lib.SaSparseParams()
    p.block_q, p.block_k, p.sink_tokens, p.local_tokens, p.granularity = bq, bk, 32, 256, gran
    arr = (ctypes.c_float * Hq)(*([theta] * Hq))
    p.theta = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    p.softmax_scale = 0.0
    return p, arr


FAKE = 0x7F0000000000   # never dereferenced: every call below fails validation first


def _est(lib, s, p, ws_bytes=0, stride=4, counts=FAKE, idx=FAKE, ws=FAKE, q=FAKE, k=FAKE):
    ls = _lib.SaLists()
    ls.counts, ls.idx, ls.stride, ls.margins = counts, idx, stride, None
    return lib.sa_estimate_mask(ctypes.byref(s), ctypes.byref(p), q, k, ctypes.byref(ls), ws,
                                ws_bytes, None)


def test_validation_codes(lib):
    s = _shape()
    p, keep = _params(4.0)
    need = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p))
    assert need > 256 * 1024 // 8
    assert _est(lib, s, p, q=None) == _lib.SA_ERR_NULL
    assert _est(lib, s, p, stride=3) == _lib.SA_ERR_CAPACITY          # 4 key blocks
    assert _est(lib, s, p, ws_bytes=need - 1) == _lib.SA_ERR_WORKSPACE
    assert _est(lib, s, p, ws=None, ws_bytes=need) == _lib.SA_ERR_WORKSPACE
    assert _est(lib, s, p, q=FAKE + 8, ws_bytes=need) == _lib.SA_ERR_SHAPE   # misaligned
    pn, keep2 = _params(float("nan"))
    assert _est(lib, s, pn, ws_bytes=need) == _lib.SA_ERR_PARAM
    pu, keep3 = _params(4.0, bk=16)
    assert _est(lib, s, pu, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    # 32-key blocks: block lists only (stripes stage 64-key tiles), not with the anchor state
    p32, keep32 = _params(4.0, bk=32)
    need32 = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p32))
    assert need32 > 0
    assert _est(lib, s, p32, stride=8, ws_bytes=need32 - 1) == _lib.SA_ERR_WORKSPACE
    assert _est(lib, s, p32, stride=7, ws_bytes=need32) == _lib.SA_ERR_CAPACITY   # 8 key blocks
    p32s, keep32s = _params(4.0, bk=32, gran=_lib.SA_STRIPE)
    assert _est(lib, s, p32s, ws_bytes=need32) == _lib.SA_ERR_UNSUPPORTED
    assert lib.sa_workspace_size(_lib.SA_OP_ESTIMATE_STATE, ctypes.byref(s), ctypes.byref(p32)) == 0
    # token strides of K and V are limited to 2^24 elements (32-bit tile offsets)
    big = _shape()
    big.k_stride[1] = 1 << 24
    assert _est(lib, big, p, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    pq, keep4 = _params(4.0, bq=96)
    assert _est(lib, s, pq, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    pe, keep6 = _params(4.0)
    pe.estimator = 3
    assert _est(lib, s, pe, ws_bytes=need) == _lib.SA_ERR_PARAM
    pe.estimator, pe.granularity = _lib.SA_EST_RELATIVE_MXFP4, _lib.SA_STRIPE
    assert _est(lib, s, pe, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    pe.estimator, pe.granularity = _lib.SA_EST_RELATIVE, _lib.SA_STRIPE
    assert _est(lib, s, pe, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    pe.granularity = _lib.SA_BLOCK
    ps, keep7 = _params(4.0)
    ps.step = -1
    assert _est(lib, s, ps, ws_bytes=need) == _lib.SA_ERR_PARAM
    need_rel = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(pe))
    assert need_rel >= need + 256 * 4 * (128 + 4)       # + int8 query rows and their scales
    assert _est(lib, s, pe, ws_bytes=need_rel - 1) == _lib.SA_ERR_WORKSPACE
    bad = _shape(Hq=6, Hkv=4)
    assert _est(lib, bad, p, ws_bytes=need) == _lib.SA_ERR_SHAPE
    d96 = _shape(D=96)
    assert _est(lib, d96, p, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    g3 = _shape(Hq=3, Hkv=1)
    p3, keep5 = _params(4.0, Hq=3)
    assert _est(lib, g3, p3, ws_bytes=need) == _lib.SA_ERR_UNSUPPORTED
    st = _shape()
    st.q_stride[1] = 4 * 128 + 4     # not a multiple of 8 elements
    assert _est(lib, st, p, ws_bytes=need) == _lib.SA_ERR_SHAPE
    neq = _shape()
    neq.seq_k = 200
    assert _est(lib, neq, p, ws_bytes=need) == _lib.SA_ERR_SHAPE
    # prefill validation
    ls = _lib.SaLists()
    ls.counts, ls.idx, ls.stride, ls.margins = FAKE, FAKE, 3, None
    assert lib.sa_sparse_prefill(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE,
                                 ctypes.byref(ls), FAKE, None, None) == _lib.SA_ERR_CAPACITY
    ls.stride = 4
    assert lib.sa_sparse_prefill(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, None,
                                 ctypes.byref(ls), FAKE, None, None) == _lib.SA_ERR_NULL
    # decode validation
    ds = _shape(B=2, N=1000)
    ds.seq_q = 1
    dp = _lib.SaDecodeParams()
    dp.block_k, dp.top_k_blocks, dp.sink_tokens, dp.local_tokens, dp.n_splits = 64, 8, 32, 256, 0
    dneed = lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(ds), ctypes.byref(dp))
    assert dneed > 0
    args = [ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, None, None]
    assert lib.sa_sparse_decode(*args, FAKE, dneed - 1, None) == _lib.SA_ERR_WORKSPACE
    dp.top_k_blocks = 0
    assert lib.sa_sparse_decode(*args, FAKE, dneed, None) == _lib.SA_ERR_PARAM
    # K below the largest forced set (1 sink block + up to 5 window blocks at block_k 64,
    # local 256) cannot hold it; K = 6 is the smallest accepted (the workspace query validates
    # the same parameters and answers 0 for an invalid request)
    dp.top_k_blocks = 5
    assert lib.sa_sparse_decode(*args, FAKE, dneed, None) == _lib.SA_ERR_PARAM
    assert lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(ds), ctypes.byref(dp)) == 0
    dp.top_k_blocks = 6
    assert lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(ds), ctypes.byref(dp)) > 0
    dp.block_k, dp.top_k_blocks = 32, 9                      # 1 + 7 + 2 = 10 at block_k 32
    assert lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(ds), ctypes.byref(dp)) == 0
    dp.block_k, dp.top_k_blocks = 64, 8
    for bad in (float("nan"), -0.1, 1.5):
        dp.top_p = bad
        assert lib.sa_sparse_decode(*args, FAKE, dneed, None) == _lib.SA_ERR_PARAM
    dp.top_p = 0.0
    ds.seq_q = 2
    assert lib.sa_sparse_decode(*args, FAKE, dneed, None) == _lib.SA_ERR_SHAPE
    ds.seq_q = 1
    assert lib.sa_build_block_summary(ctypes.byref(ds), 0, FAKE, FAKE, FAKE, None) == _lib.SA_ERR_PARAM
    assert lib.sa_build_block_summary(ctypes.byref(ds), 64, None, FAKE, FAKE, None) == _lib.SA_ERR_NULL
    assert lib.sa_quantize_block_summary(ctypes.byref(ds), 0, FAKE, FAKE, FAKE, None) == _lib.SA_ERR_PARAM
    assert lib.sa_quantize_block_summary(ctypes.byref(ds), 64, FAKE, None, FAKE, None) == _lib.SA_ERR_NULL
    args_q4 = [ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None]
    assert lib.sa_sparse_decode_q4(*args_q4, FAKE, dneed, None) == _lib.SA_ERR_NULL
    args_q4[6] = FAKE
    assert lib.sa_sparse_decode_q4(*args_q4, FAKE, dneed - 1, None) == _lib.SA_ERR_WORKSPACE
    assert lib.sa_quantize_block_summary_fp4(ctypes.byref(ds), 0, FAKE, FAKE, FAKE, None) == _lib.SA_ERR_PARAM
    assert lib.sa_quantize_block_summary_fp4(ctypes.byref(ds), 64, FAKE, FAKE, None, None) == _lib.SA_ERR_NULL
    args_fp4 = [ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None]
    assert lib.sa_sparse_decode_fp4(*args_fp4, FAKE, dneed, None) == _lib.SA_ERR_NULL
    args_fp4[6] = FAKE
    assert lib.sa_sparse_decode_fp4(*args_fp4, FAKE, dneed - 1, None) == _lib.SA_ERR_WORKSPACE
    # the no-allocation decode: validation as sa_sparse_decode, then the static scratch limit
    nargs = [ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, None, FAKE, FAKE, None, None,
             None]
    assert lib.sa_sparse_decode_noalloc(*nargs) == _lib.SA_ERR_NULL          # no summary
    big = _shape(B=64, Hq=32, Hkv=8, N=8192 * 64)
    big.seq_q = 1
    bp = _lib.SaDecodeParams()
    bp.block_k, bp.top_k_blocks, bp.sink_tokens, bp.local_tokens = 64, 64, 32, 256
    assert lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(big), ctypes.byref(bp)) > \
        _lib.SA_NOALLOC_SCRATCH_BYTES
    assert lib.sa_sparse_decode_noalloc(ctypes.byref(big), ctypes.byref(bp), FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, None, None, None) == _lib.SA_ERR_WORKSPACE
    dp.top_k_blocks = 0
    assert lib.sa_sparse_decode_noalloc(ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE,
                                        FAKE, FAKE, FAKE, None, None, None) == _lib.SA_ERR_PARAM
    dp.top_k_blocks = 8
    assert lib.sa_workspace_size(_lib.SA_OP_PREFILL, ctypes.byref(s), ctypes.byref(p)) == 0


def test_empty_problems_rejected(lib):
    p, keep = _params(4.0)
    for field in ("batch", "seq_q", "seq_k", "n_q_heads", "n_kv_heads"):
        s = _shape()
        setattr(s, field, 0)
        assert _est(lib, s, p, ws_bytes=1 << 30) == _lib.SA_ERR_SHAPE, field
        assert lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p)) == 0
    ds = _shape(B=0, N=1000)
    ds.seq_q = 1
    dp = _lib.SaDecodeParams()
    dp.block_k, dp.top_k_blocks, dp.sink_tokens, dp.local_tokens = 64, 8, 32, 256
    assert lib.sa_sparse_decode(ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, None, FAKE, 1 << 30, None) == _lib.SA_ERR_SHAPE
    # the decode cache is limited to 8192 key blocks
    big = _shape(B=1, N=8192 * 64 + 1)
    big.seq_q = 1
    assert lib.sa_sparse_decode(ctypes.byref(big), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE, FAKE,
                                FAKE, None, None, FAKE, 1 << 30, None) == _lib.SA_ERR_UNSUPPORTED


def test_anchor_state_validation(lib):
    s = _shape()
    p, keep = _params(4.0)
    need = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p))
    need_st = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE_STATE, ctypes.byref(s), ctypes.byref(p))
    assert need_st >= need + 4 * 256 * 4                 # + one fp32 anchor per (head, row)
    ls = _lib.SaLists()
    ls.counts, ls.idx, ls.stride, ls.margins = FAKE, FAKE, 4, None
    st = _lib.SaAnchorState()
    st.o, st.lse = FAKE, FAKE

    def est(state=ctypes.byref(st), v=FAKE, ws_bytes=need_st, pp=p):
        return lib.sa_estimate_mask_anchor_state(ctypes.byref(s), ctypes.byref(pp), FAKE, FAKE, v,
                                                 ctypes.byref(ls), state, FAKE, ws_bytes, None)

    assert est(state=None) == _lib.SA_ERR_NULL
    assert est(v=None) == _lib.SA_ERR_NULL
    assert est(ws_bytes=need_st - 1) == _lib.SA_ERR_WORKSPACE
    st.lse = FAKE + 2                                     # fp32 buffer not 4-byte aligned
    assert est() == _lib.SA_ERR_SHAPE
    st.lse = None
    assert est() == _lib.SA_ERR_NULL
    st.lse = FAKE
    pr, keep2 = _params(4.0)
    pr.estimator = _lib.SA_EST_RELATIVE
    assert est(pp=pr) == _lib.SA_ERR_UNSUPPORTED
    assert lib.sa_workspace_size(_lib.SA_OP_ESTIMATE_STATE, ctypes.byref(s), ctypes.byref(pr)) == 0
    # column lists take the anchor state too (validation reaches the workspace check)
    pst, keep3 = _params(4.0, gran=_lib.SA_STRIPE)
    need_sst = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE_STATE, ctypes.byref(s), ctypes.byref(pst))
    assert need_sst > lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(pst))
    assert est(pp=pst, ws_bytes=need_sst - 1) == _lib.SA_ERR_WORKSPACE
    # resume validation
    def resume(state=ctypes.byref(st), pp=p):
        return lib.sa_sparse_prefill_resume(ctypes.byref(s), ctypes.byref(pp), FAKE, FAKE, FAKE,
                                            ctypes.byref(ls), state, FAKE, None, None)
    assert resume(state=None) == _lib.SA_ERR_NULL
    st.o = FAKE + 8
    assert resume() == _lib.SA_ERR_SHAPE
    assert resume(pp=pst) == _lib.SA_ERR_SHAPE           # column lists accepted, then the check
    st.o = FAKE
    ls.stride = 3
    assert resume() == _lib.SA_ERR_CAPACITY
    p32, keep4 = _params(4.0, bk=32)
    ls.stride = 8
    assert resume(pp=p32) == _lib.SA_ERR_UNSUPPORTED
    assert est(pp=p32) == _lib.SA_ERR_UNSUPPORTED


def _with_map(s, m):
    arr = (ctypes.c_int32 * len(m))(*m)
    s.kv_head_of_q = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    return arr


def test_head_map_validation(lib):
    """The GQA head map: values in [0, n_kv_heads) (else SA_ERR_PARAM), equal group sizes
    (else SA_ERR_UNSUPPORTED); a valid permuted map passes every shape check."""
    p, keep = _params(4.0, Hq=4)
    s = _shape(Hq=4, Hkv=2)
    need = lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p))
    m_ok = _with_map(s, [1, 0, 0, 1])
    assert lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p)) == need
    # the map passes: the call fails only on the (short) workspace
    assert _est(lib, s, p, ws_bytes=need - 1) == _lib.SA_ERR_WORKSPACE
    for bad, code in (([0, 1, 2, 1], _lib.SA_ERR_PARAM), ([0, -1, 1, 1], _lib.SA_ERR_PARAM),
                      ([0, 0, 0, 1], _lib.SA_ERR_UNSUPPORTED), ([1, 1, 1, 1], _lib.SA_ERR_UNSUPPORTED)):
        m_bad = _with_map(s, bad)
        assert _est(lib, s, p, ws_bytes=need) == code, bad
        assert lib.sa_workspace_size(_lib.SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p)) == 0
        ls = _lib.SaLists()
        ls.counts, ls.idx, ls.stride, ls.margins = FAKE, FAKE, 4, None
        assert lib.sa_sparse_prefill(ctypes.byref(s), ctypes.byref(p), FAKE, FAKE, FAKE,
                                     ctypes.byref(ls), FAKE, None, None) == code, bad
        ds = _shape(B=2, Hq=4, Hkv=2, N=1000)
        ds.seq_q = 1
        keep_d = _with_map(ds, bad)
        dp = _lib.SaDecodeParams()
        dp.block_k, dp.top_k_blocks, dp.sink_tokens, dp.local_tokens = 64, 8, 32, 256
        assert lib.sa_workspace_size(_lib.SA_OP_DECODE, ctypes.byref(ds), ctypes.byref(dp)) == 0
        assert lib.sa_sparse_decode(ctypes.byref(ds), ctypes.byref(dp), FAKE, FAKE, FAKE, FAKE,
                                    FAKE, FAKE, None, None, FAKE, 1 << 30, None) == code, bad
        assert lib.sa_build_block_summary(ctypes.byref(ds), 64, FAKE, FAKE, FAKE, None) == code
    del m_ok, m_bad, keep_d
