"""sa_sparse_decode_noalloc (scratch in the library's static per-GPU array) against
sa_sparse_decode (caller workspace) through the C ABI: two calls in a row, the second on a
smaller problem, each bit-identical to the workspace entry point on the same inputs (the same
kernels run on the same data, so selection, output and LSE match exactly)."""
import ctypes

import numpy as np
import pytest

import synth
from helpers import log, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    import torch
    import block_sparse_attention_estimate_amd as sa
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    sa.load_library()
    return torch.device("cuda:0")


def _case(dev, batch, seq, hq, hkv, top_k, top_p, seed):
    import torch
    import block_sparse_attention_estimate_amd as sa
    from block_sparse_attention_estimate_amd import _lib
    x = synth.make_decode(batch=batch, seq=seq, hq=hq, hkv=hkv, head_dim=128, top_k=top_k,
                          seed=seed)
    if batch >= 2:
        x.cache_len[1] = seq - 777
    q, kc, vc = to_dev(x.q, dev), to_dev(x.k_cache, dev), to_dev(x.v_cache, dev)
    cl = torch.from_numpy(x.cache_len).to(dev)
    kbar = sa.build_block_summary(kc, cl, block_k=64)
    kw = dict(block_k=64, top_k=top_k, sink=32, local=256, top_p=top_p)
    o_ref, lse_ref, sel_ref = sa.sparse_decode(q, kc, vc, kbar, cl, **kw)
    # the no-allocation entry point, called through the C ABI directly
    lib = _lib.load()
    o = torch.full_like(q, float("nan"))
    lse = torch.full((batch, hq), float("nan"), dtype=torch.float32, device=dev)
    sel = torch.full((batch, hkv, top_k), -7, dtype=torch.int32, device=dev)
    s = sa._decode_shape(q, kc, vc, o)
    p = _lib.SaDecodeParams()
    p.block_k, p.top_k_blocks, p.sink_tokens, p.local_tokens = 64, top_k, 32, 256
    p.n_splits, p.softmax_scale, p.top_p = 0, 0.0, top_p
    stream = torch.cuda.current_stream().cuda_stream
    st = lib.sa_sparse_decode_noalloc(ctypes.byref(s), ctypes.byref(p), q.data_ptr(), kc.data_ptr(),
                                      vc.data_ptr(), kbar.data_ptr(), cl.data_ptr(), o.data_ptr(),
                                      lse.data_ptr(), sel.data_ptr(), ctypes.c_void_p(stream))
    assert st == _lib.SA_OK, lib.sa_status_string(st)
    torch.cuda.synchronize()
    assert torch.equal(sel, sel_ref)
    assert torch.equal(o.view(torch.int16), o_ref.view(torch.int16))
    assert torch.equal(lse, lse_ref)
    log(f"  no-alloc decode B={batch} L={seq} Hq={hq} Hkv={hkv} K={top_k} top_p={top_p}: "
        f"bit-identical to the workspace entry point")


def test_noalloc_decode_matches_workspace_entry_point(dev):
    # the larger problem first, then a smaller one that reuses the same static scratch
    _case(dev, batch=16, seq=131072 // 4, hq=32, hkv=8, top_k=64, top_p=0.0, seed=3)
    _case(dev, batch=2, seq=3000, hq=8, hkv=2, top_k=12, top_p=0.0, seed=4)
    # and a top-p budget (the per-(b, g) counts also live in the scratch)
    _case(dev, batch=3, seq=5000, hq=8, hkv=2, top_k=40, top_p=0.6, seed=5)
