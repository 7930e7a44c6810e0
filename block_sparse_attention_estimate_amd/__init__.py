"""MI355X (gfx950) training-free block/stripe-sparse attention.

Thin Python binding of libsa.so (C ABI in include/sa.h).  The functions here only marshal
arguments: device memory and streams come from PyTorch, every computation runs in the
library's HIP kernels, and nothing falls back to another implementation -- a missing or
unbuilt library raises.

Entry points (same names as the C ABI):
  estimate_mask(q, k, theta, ...)       -> Lists     (sa_estimate_mask)
  sparse_prefill(q, k, v, lists, ...)   -> (o, lse)  (sa_sparse_prefill)
  estimate_mask_anchor_state(q, k, v, theta, ...) -> (Lists, AnchorState)
                                                     (sa_estimate_mask_anchor_state)
  sparse_prefill_resume(q, k, v, lists, state, ...) -> (o, lse)  (sa_sparse_prefill_resume)
  build_block_summary(k_cache, ...)     -> kbar      (sa_build_block_summary)
  sparse_decode(q, k_cache, v_cache, kbar, cache_len, ...) -> (o, lse, selected)
  workspace_size(op, ...)                            (sa_workspace_size)
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib
from ._lib import (SA_BLOCK, SA_STRIPE, SA_OP_ESTIMATE, SA_OP_PREFILL, SA_OP_DECODE,  # noqa: F401
                   SA_OP_CALIBRATE, SA_OP_ESTIMATE_STATE, SaError)

__all__ = ["Lists", "AnchorState", "alloc_anchor_state", "estimate_mask", "sparse_prefill",
           "estimate_mask_anchor_state", "sparse_prefill_resume", "build_block_summary",
           "quantize_block_summary", "quantize_block_summary_fp4", "sparse_decode",
           "sparse_decode_noalloc", "calibrate_theta", "workspace_size",
           "SaError", "load_library"]


def load_library():
    return _lib.load()


def _stream(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def _ptr(t) -> int | None:
    return None if t is None else int(t.data_ptr())


def _gran(g) -> int:
    if g in ("block", SA_BLOCK):
        return SA_BLOCK
    if g in ("stripe", SA_STRIPE):
        return SA_STRIPE
    raise ValueError(f"granularity must be 'block' or 'stripe', got {g!r}")


def _check_bf16(name, t, ndim):
    if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA bfloat16 tensor")
    if t.dim() != ndim or t.stride(-1) != 1:
        raise ValueError(f"{name} must be {ndim}-D with a contiguous last dimension")


def _head_map(s: _lib.SaShape, kv_head_of_q) -> None:
    """Attach the GQA head map (query head -> KV head) to the shape; None keeps the default
    h // (Hq // Hkv).  The ctypes array lives as long as the shape."""
    if kv_head_of_q is None:
        return
    m = [int(x) for x in (kv_head_of_q.tolist() if hasattr(kv_head_of_q, "tolist") else kv_head_of_q)]
    if len(m) != s.n_q_heads:
        raise ValueError("kv_head_of_q needs one entry per query head")
    arr = (ctypes.c_int32 * len(m))(*m)
    s.kv_head_of_q = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))
    s._keep_map = arr


def _prefill_shape(q, k, v=None, o=None, kv_head_of_q=None) -> _lib.SaShape:
    _check_bf16("q", q, 4)
    _check_bf16("k", k, 4)
    B, N, Hq, D = q.shape
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = B, Hq, k.shape[2], D
    s.seq_q, s.seq_k = N, k.shape[1]
    _head_map(s, kv_head_of_q)
    s.q_stride[:] = q.stride()[:3]
    s.k_stride[:] = k.stride()[:3]
    vv = v if v is not None else k
    s.v_stride[:] = vv.stride()[:3]
    oo = o if o is not None else q
    s.o_stride[:] = oo.stride()[:3]
    return s


_ESTIMATORS = {"pooled": _lib.SA_EST_POOLED, "relative": _lib.SA_EST_RELATIVE,
               "relative_mxfp4": _lib.SA_EST_RELATIVE_MXFP4}


def _sparse_params(block_q, block_k, sink, local, granularity, theta, softmax_scale, n_q_heads,
                   estimator="pooled", step=1):
    p = _lib.SaSparseParams()
    p.block_q, p.block_k, p.sink_tokens, p.local_tokens = block_q, block_k, sink, local
    p.granularity = _gran(granularity)
    if estimator not in _ESTIMATORS:
        raise ValueError(f"estimator must be one of {sorted(_ESTIMATORS)}")
    p.estimator = _ESTIMATORS[estimator]
    p.step = int(step)
    p.softmax_scale = float(softmax_scale or 0.0)
    arr = None
    if theta is not None:
        th = torch.as_tensor(theta, dtype=torch.float32).reshape(-1)
        if th.numel() == 1:
            th = th.expand(n_q_heads)
        if th.numel() != n_q_heads:
            raise ValueError("theta needs one value per query head")
        arr = (ctypes.c_float * n_q_heads)(*[float(x) for x in th.tolist()])
        p.theta = ctypes.cast(arr, ctypes.POINTER(ctypes.c_float))
    return p, arr


@dataclass
class Lists:
    """Per (batch, KV head, query block) kept lists: counts [B, Hkv, nQB] int32 and idx
    [B, Hkv, nQB, stride] int32 (ascending block or column ids), optional margins."""
    counts: torch.Tensor
    idx: torch.Tensor
    stride: int
    granularity: str
    margins: torch.Tensor | None = None

    def c_struct(self) -> _lib.SaLists:
        ls = _lib.SaLists()
        ls.counts = _ptr(self.counts)
        ls.idx = _ptr(self.idx)
        ls.stride = self.stride
        ls.margins = _ptr(self.margins)
        return ls

    def overflowed(self) -> bool:
        """True when some stripe row had more entries than ``stride`` (synchronises)."""
        return bool((self.counts > self.stride).any().item())


@dataclass
class AnchorState:
    """Attention over each row's anchor region (sink tokens and causal local window):
    o [B, N, Hq, d] bf16 (normalised) and lse [B, Hq, N] fp32 (natural log)."""
    o: torch.Tensor
    lse: torch.Tensor

    def c_struct(self) -> _lib.SaAnchorState:
        st = _lib.SaAnchorState()
        st.o = _ptr(self.o)
        st.lse = _ptr(self.lse)
        return st


def _check_state(st: AnchorState, q) -> None:
    B, N, Hq, D = q.shape
    _check_bf16("state.o", st.o, 4)
    if tuple(st.o.shape) != (B, N, Hq, D) or not st.o.is_contiguous():
        raise ValueError("state.o must be a contiguous [B, N, Hq, d] tensor")
    if (not isinstance(st.lse, torch.Tensor) or st.lse.dtype != torch.float32 or not st.lse.is_cuda
            or tuple(st.lse.shape) != (B, Hq, N) or not st.lse.is_contiguous()):
        raise ValueError("state.lse must be a contiguous CUDA float32 [B, Hq, N] tensor")


def alloc_anchor_state(q) -> AnchorState:
    B, N, Hq, D = q.shape
    return AnchorState(torch.empty((B, N, Hq, D), dtype=torch.bfloat16, device=q.device),
                       torch.empty((B, Hq, N), dtype=torch.float32, device=q.device))


def workspace_size(op, *, q=None, k=None, block_q=128, block_k=64, sink=32, local=256,
                   granularity="block", theta=None, estimator="pooled", shape=None,
                   decode_params=None, kv_head_of_q=None) -> int:
    lib = _lib.load()
    if op in (SA_OP_ESTIMATE, SA_OP_CALIBRATE, SA_OP_ESTIMATE_STATE):
        s = _prefill_shape(q, k, kv_head_of_q=kv_head_of_q)
        p, keep = _sparse_params(block_q, block_k, sink, local, granularity,
                                 theta if theta is not None else 0.0, 0.0, q.shape[2], estimator)
        return int(lib.sa_workspace_size(op, ctypes.byref(s), ctypes.byref(p)))
    if op == SA_OP_DECODE:
        return int(lib.sa_workspace_size(op, ctypes.byref(shape), ctypes.byref(decode_params)))
    return 0


def alloc_lists(q, k, *, block_q, block_k=64, granularity="block", stride=None,
                margins=False) -> Lists:
    B, N, Hq, D = q.shape
    Hkv = k.shape[2]
    nqb = -(-N // block_q)
    nkb = -(-N // block_k)
    gran = "stripe" if _gran(granularity) == SA_STRIPE else "block"
    if stride is None:
        stride = nkb if gran == "block" else N
    counts = torch.empty((B, Hkv, nqb), dtype=torch.int32, device=q.device)
    idx = torch.empty((B, Hkv, nqb, stride), dtype=torch.int32, device=q.device)
    m = None
    if margins:
        ncand = nkb if gran == "block" else N
        m = torch.full((B, Hkv, nqb, ncand), float("nan"), dtype=torch.float32, device=q.device)
    return Lists(counts, idx, int(stride), gran, m)


def estimate_mask(q, k, theta, *, block_q=128, block_k=64, sink=32, local=256,
                  granularity="block", softmax_scale=0.0, stride=None, margins=False,
                  estimator="pooled", step=1, workspace=None, out: Lists | None = None,
                  kv_head_of_q=None, stream=None) -> Lists:
    """Estimation pass (sa_estimate_mask).  q [B, N, Hq, d], k [B, N, Hkv, d] bf16 CUDA
    tensors; theta scalar or [Hq] in logit units; estimator "pooled" (anchor vs pooled
    query), "relative" (element-wise int8 estimate against the row's sink-local log-sum-exp)
    or "relative_mxfp4" (the same with MXFP4 operands on the block-scaled fp4 MFMA);
    step > 1 identifies query blocks in groups of `step` (AnchorAttention's step)."""
    lib = _lib.load()
    s = _prefill_shape(q, k, kv_head_of_q=kv_head_of_q)
    p, keep = _sparse_params(block_q, block_k, sink, local, granularity, theta, softmax_scale,
                             q.shape[2], estimator, step)
    lists = out if out is not None else alloc_lists(q, k, block_q=block_q, block_k=block_k,
                                                    granularity=granularity, stride=stride,
                                                    margins=margins)
    need = int(lib.sa_workspace_size(SA_OP_ESTIMATE, ctypes.byref(s), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ls = lists.c_struct()
    _lib.check(lib.sa_estimate_mask(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k),
                                    ctypes.byref(ls), _ptr(workspace), workspace.numel(),
                                    _stream(stream)), "sa_estimate_mask")
    del keep
    return lists


def sparse_prefill(q, k, v, lists: Lists, *, block_q=128, block_k=64, sink=32, local=256,
                   softmax_scale=0.0, out=None, lse=True, kv_head_of_q=None, stream=None):
    """Block/stripe-sparse attention over given lists (sa_sparse_prefill).
    Returns (o [B, N, Hq, d] bf16, lse [B, Hq, N] fp32 or None)."""
    lib = _lib.load()
    _check_bf16("v", v, 4)
    o = out if out is not None else torch.empty_like(q)
    s = _prefill_shape(q, k, v, o, kv_head_of_q=kv_head_of_q)
    p, keep = _sparse_params(block_q, block_k, sink, local, lists.granularity, None,
                             softmax_scale, q.shape[2])
    lse_t = None
    if lse:
        lse_t = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                            device=q.device)
    ls = lists.c_struct()
    _lib.check(lib.sa_sparse_prefill(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                     ctypes.byref(ls), _ptr(o), _ptr(lse_t), _stream(stream)),
               "sa_sparse_prefill")
    del keep
    return o, lse_t


def estimate_mask_anchor_state(q, k, v, theta, *, block_q=128, block_k=64, sink=32, local=256,
                               granularity="block", softmax_scale=0.0, stride=None,
                               margins=False, step=1, workspace=None,
                               out: Lists | None = None, state: AnchorState | None = None,
                               kv_head_of_q=None, stream=None):
    """Estimation pass with the anchor state (sa_estimate_mask_anchor_state; pooled
    estimator, block or column lists).  Returns (lists, state): the lists equal
    estimate_mask's, and the state holds the attention over each row's anchor region for
    sparse_prefill_resume."""
    lib = _lib.load()
    _check_bf16("v", v, 4)
    s = _prefill_shape(q, k, v, kv_head_of_q=kv_head_of_q)
    p, keep = _sparse_params(block_q, block_k, sink, local, granularity, theta, softmax_scale,
                             q.shape[2], "pooled", step)
    lists = out if out is not None else alloc_lists(q, k, block_q=block_q, block_k=block_k,
                                                    granularity=granularity, stride=stride,
                                                    margins=margins)
    st = state if state is not None else alloc_anchor_state(q)
    _check_state(st, q)
    need = int(lib.sa_workspace_size(SA_OP_ESTIMATE_STATE, ctypes.byref(s), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    ls = lists.c_struct()
    cs = st.c_struct()
    _lib.check(lib.sa_estimate_mask_anchor_state(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k),
                                                 _ptr(v), ctypes.byref(ls), ctypes.byref(cs),
                                                 _ptr(workspace), workspace.numel(), _stream(stream)),
               "sa_estimate_mask_anchor_state")
    del keep
    return lists, st


def sparse_prefill_resume(q, k, v, lists: Lists, state: AnchorState, *, block_q=128, block_k=64,
                          sink=32, local=256, softmax_scale=0.0, out=None, lse=True,
                          kv_head_of_q=None, stream=None):
    """Sparse attention (block or column lists) that starts from the anchor state and skips
    each row's anchor region (sa_sparse_prefill_resume).  Returns (o [B, N, Hq, d] bf16, lse [B, Hq, N] fp32 or
    None)."""
    lib = _lib.load()
    _check_bf16("v", v, 4)
    o = out if out is not None else torch.empty_like(q)
    s = _prefill_shape(q, k, v, o, kv_head_of_q=kv_head_of_q)
    p, keep = _sparse_params(block_q, block_k, sink, local, lists.granularity, None,
                             softmax_scale, q.shape[2])
    lse_t = None
    if lse:
        lse_t = torch.empty((q.shape[0], q.shape[2], q.shape[1]), dtype=torch.float32,
                            device=q.device)
    _check_state(state, q)
    ls = lists.c_struct()
    cs = state.c_struct()
    _lib.check(lib.sa_sparse_prefill_resume(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k),
                                            _ptr(v), ctypes.byref(ls), ctypes.byref(cs), _ptr(o),
                                            _ptr(lse_t), _stream(stream)),
               "sa_sparse_prefill_resume")
    del keep
    return o, lse_t


def calibrate_theta(q, k, v, *, tau0=0.008, err_bound=0.4, max_halvings=16, block_q=128,
                    block_k=64, sink=32, local=256, softmax_scale=0.0, estimator="pooled",
                    workspace=None, kv_head_of_q=None, stream=None):
    """Per-head theta calibration (sa_calibrate_theta; block granularity).  Returns
    (theta [Hq] float32, err [Hq] float32, halvings [Hq] int32) as numpy arrays: theta_h =
    -ln(tau0) + halvings_h * ln 2, err_h = sum |O - O~| over the head's rows and dims / rows.
    Synchronous (the library reads the errors back every round)."""
    import numpy as np
    lib = _lib.load()
    _check_bf16("v", v, 4)
    s = _prefill_shape(q, k, v, q, kv_head_of_q=kv_head_of_q)
    p, keep = _sparse_params(block_q, block_k, sink, local, "block", 0.0, softmax_scale,
                             q.shape[2], estimator)
    need = int(lib.sa_workspace_size(SA_OP_CALIBRATE, ctypes.byref(s), ctypes.byref(p)))
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=q.device)
    hq = q.shape[2]
    theta = (ctypes.c_float * hq)()
    err = (ctypes.c_float * hq)()
    halv = (ctypes.c_int32 * hq)()
    _lib.check(lib.sa_calibrate_theta(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v),
                                      float(tau0), float(err_bound), int(max_halvings), theta, err,
                                      halv, _ptr(workspace), workspace.numel(), _stream(stream)),
               "sa_calibrate_theta")
    del keep
    return (np.array(theta, dtype=np.float32), np.array(err, dtype=np.float32),
            np.array(halv, dtype=np.int32))


def _decode_shape(q, k_cache, v_cache, o=None, kv_head_of_q=None) -> _lib.SaShape:
    _check_bf16("q", q, 3)
    _check_bf16("k_cache", k_cache, 4)
    B, Hq, D = q.shape
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = B, Hq, k_cache.shape[2], D
    s.seq_q, s.seq_k = 1, k_cache.shape[1]
    _head_map(s, kv_head_of_q)
    s.q_stride[:] = (q.stride(0), 0, q.stride(1))
    s.k_stride[:] = k_cache.stride()[:3]
    vv = v_cache if v_cache is not None else k_cache
    s.v_stride[:] = vv.stride()[:3]
    oo = o if o is not None else q
    s.o_stride[:] = (oo.stride(0), 0, oo.stride(1))
    return s


def build_block_summary(k_cache, cache_len, *, block_k=64, n_q_heads=None, out=None, stream=None):
    """Mean key per block (sa_build_block_summary): [B, ceil(L/bk), Hkv, d] bf16."""
    lib = _lib.load()
    _check_bf16("k_cache", k_cache, 4)
    B, L, Hkv, D = k_cache.shape
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = B, n_q_heads or Hkv, Hkv, D
    s.seq_q, s.seq_k = 1, L
    s.k_stride[:] = k_cache.stride()[:3]
    nkb = -(-L // block_k)
    kbar = out if out is not None else torch.empty((B, nkb, Hkv, D), dtype=torch.bfloat16,
                                                   device=k_cache.device)
    _lib.check(lib.sa_build_block_summary(ctypes.byref(s), block_k, _ptr(k_cache), _ptr(cache_len),
                                          _ptr(kbar), _stream(stream)), "sa_build_block_summary")
    return kbar


def quantize_block_summary(k_summary, *, block_k=64, seq_k=None, stream=None):
    """4-bit summaries (sa_quantize_block_summary) of bf16 summaries [B, nKB, Hkv, d]:
    returns (codes uint8 [B, nKB, Hkv, d/2], scales bf16 [B, nKB, Hkv, d/32])."""
    lib = _lib.load()
    _check_bf16("k_summary", k_summary, 4)
    B, nkb, Hkv, D = k_summary.shape
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = B, Hkv, Hkv, D
    s.seq_q, s.seq_k = 1, seq_k if seq_k is not None else nkb * block_k
    codes = torch.empty((B, nkb, Hkv, D // 2), dtype=torch.uint8, device=k_summary.device)
    scales = torch.empty((B, nkb, Hkv, D // 32), dtype=torch.bfloat16, device=k_summary.device)
    _lib.check(lib.sa_quantize_block_summary(ctypes.byref(s), block_k, _ptr(k_summary), _ptr(codes),
                                             _ptr(scales), _stream(stream)),
               "sa_quantize_block_summary")
    return codes, scales


def quantize_block_summary_fp4(k_summary, *, block_k=64, seq_k=None, stream=None):
    """FP4 (MXFP4) summaries (sa_quantize_block_summary_fp4) of bf16 summaries
    [B, nKB, Hkv, d]: returns (codes uint8 [B, nKB, Hkv, d/2], exps uint8 [B, nKB, Hkv, d/32])."""
    lib = _lib.load()
    _check_bf16("k_summary", k_summary, 4)
    B, nkb, Hkv, D = k_summary.shape
    s = _lib.SaShape()
    s.batch, s.n_q_heads, s.n_kv_heads, s.head_dim = B, Hkv, Hkv, D
    s.seq_q, s.seq_k = 1, seq_k if seq_k is not None else nkb * block_k
    codes = torch.empty((B, nkb, Hkv, D // 2), dtype=torch.uint8, device=k_summary.device)
    exps = torch.empty((B, nkb, Hkv, D // 32), dtype=torch.uint8, device=k_summary.device)
    _lib.check(lib.sa_quantize_block_summary_fp4(ctypes.byref(s), block_k, _ptr(k_summary),
                                                 _ptr(codes), _ptr(exps), _stream(stream)),
               "sa_quantize_block_summary_fp4")
    return codes, exps


def sparse_decode(q, k_cache, v_cache, k_summary, cache_len, *, block_k=64, top_k=64, sink=32,
                  local=256, n_splits=0, softmax_scale=0.0, top_p=0.0, workspace=None, out=None,
                  return_selected=True, kv_head_of_q=None, stream=None):
    """Top-K block-sparse decode (sa_sparse_decode; sa_sparse_decode_q4 when k_summary is the
    (codes, scales) pair of quantize_block_summary, sa_sparse_decode_fp4 when it is the
    (codes, exps) pair of quantize_block_summary_fp4).  q [B, Hq, d]; caches [B, L, Hkv, d].
    top_p in (0, 1] reads each (b, KV head)'s budget from the block-score distribution (at
    most top_k blocks); 0 selects top_k.
    Returns (o [B, Hq, d] bf16, lse [B, Hq] fp32, selected [B, Hkv, top_k] int32 or None;
    unused entries of selected are -1)."""
    lib = _lib.load()
    _check_bf16("v_cache", v_cache, 4)
    o = out if out is not None else torch.empty_like(q)
    s = _decode_shape(q, k_cache, v_cache, o, kv_head_of_q=kv_head_of_q)
    p = _lib.SaDecodeParams()
    p.block_k, p.top_k_blocks, p.sink_tokens, p.local_tokens = block_k, top_k, sink, local
    p.n_splits, p.softmax_scale = n_splits, float(softmax_scale or 0.0)
    p.top_p = float(top_p or 0.0)
    need = int(lib.sa_workspace_size(SA_OP_DECODE, ctypes.byref(s), ctypes.byref(p)))
    if need == 0:
        raise SaError(_lib.SA_ERR_PARAM, "sa_workspace_size(decode)")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    B, Hq, _ = q.shape
    lse = torch.empty((B, Hq), dtype=torch.float32, device=q.device)
    sel = None
    if return_selected:
        sel = torch.empty((B, k_cache.shape[2], top_k), dtype=torch.int32, device=q.device)
    if isinstance(k_summary, (tuple, list)) and k_summary[1].dtype == torch.uint8:
        codes, exps = k_summary
        _lib.check(lib.sa_sparse_decode_fp4(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k_cache),
                                            _ptr(v_cache), _ptr(codes), _ptr(exps), _ptr(cache_len),
                                            _ptr(o), _ptr(lse), _ptr(sel), _ptr(workspace),
                                            workspace.numel(), _stream(stream)), "sa_sparse_decode_fp4")
    elif isinstance(k_summary, (tuple, list)):
        codes, scales = k_summary
        _lib.check(lib.sa_sparse_decode_q4(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k_cache),
                                           _ptr(v_cache), _ptr(codes), _ptr(scales), _ptr(cache_len),
                                           _ptr(o), _ptr(lse), _ptr(sel), _ptr(workspace),
                                           workspace.numel(), _stream(stream)), "sa_sparse_decode_q4")
    else:
        _lib.check(lib.sa_sparse_decode(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k_cache),
                                        _ptr(v_cache), _ptr(k_summary), _ptr(cache_len), _ptr(o),
                                        _ptr(lse), _ptr(sel), _ptr(workspace), workspace.numel(),
                                        _stream(stream)), "sa_sparse_decode")
    return o, lse, sel


def sparse_decode_noalloc(q, k_cache, v_cache, k_summary, cache_len, *, out, lse, selected=None,
                          block_k=64, top_k=64, sink=32, local=256, n_splits=0, softmax_scale=0.0,
                          top_p=0.0, kv_head_of_q=None, stream=None):
    """sa_sparse_decode_noalloc: sparse_decode with bf16 summaries whose scratch is the
    library's static per-GPU array (no workspace, nothing allocated by the call).  The caller
    passes every output: out [B, Hq, d] bf16, lse [B, Hq] fp32, optional selected [B, Hkv,
    top_k] int32.  Calls that overlap on one GPU race (they share the array)."""
    lib = _lib.load()
    _check_bf16("v_cache", v_cache, 4)
    s = _decode_shape(q, k_cache, v_cache, out, kv_head_of_q=kv_head_of_q)
    p = _lib.SaDecodeParams()
    p.block_k, p.top_k_blocks, p.sink_tokens, p.local_tokens = block_k, top_k, sink, local
    p.n_splits, p.softmax_scale = n_splits, float(softmax_scale or 0.0)
    p.top_p = float(top_p or 0.0)
    _lib.check(lib.sa_sparse_decode_noalloc(ctypes.byref(s), ctypes.byref(p), _ptr(q), _ptr(k_cache),
                                            _ptr(v_cache), _ptr(k_summary), _ptr(cache_len),
                                            _ptr(out), _ptr(lse), _ptr(selected), _stream(stream)),
               "sa_sparse_decode_noalloc")
    return out, lse, selected
