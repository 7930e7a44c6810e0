"""ctypes view of libsa.so (the C ABI declared in include/sa.h).

Argument marshalling only: every step of the sparse-attention path runs in the HIP
kernels of libsa.so.  Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa.so")
DEBUG_LIB_PATH = os.path.join(_HERE, "libsa_debug.so")

SA_OK, SA_ERR_NULL, SA_ERR_SHAPE, SA_ERR_PARAM, SA_ERR_UNSUPPORTED, SA_ERR_CAPACITY, \
    SA_ERR_WORKSPACE, SA_ERR_DEVICE, SA_ERR_CHECK = range(9)
# bits of sa_debug_flags() (debug build)
SA_DBG_COUNT, SA_DBG_RANGE, SA_DBG_ORDER, SA_DBG_CACHE_LEN = 1, 2, 4, 8
SA_BLOCK, SA_STRIPE = 0, 1
SA_EST_POOLED, SA_EST_RELATIVE, SA_EST_RELATIVE_MXFP4 = 0, 1, 2
SA_OP_ESTIMATE, SA_OP_PREFILL, SA_OP_DECODE, SA_OP_CALIBRATE, SA_OP_ESTIMATE_STATE = 0, 1, 2, 3, 4
SA_MAX_Q_HEADS = 128

EXPORTED = ("sa_workspace_size", "sa_estimate_mask", "sa_sparse_prefill",
            "sa_build_block_summary", "sa_sparse_decode", "sa_quantize_block_summary",
            "sa_sparse_decode_q4", "sa_calibrate_theta", "sa_status_string",
            "sa_estimate_mask_anchor_state", "sa_sparse_prefill_resume",
            "sa_quantize_block_summary_fp4", "sa_sparse_decode_fp4", "sa_sparse_decode_noalloc",
            "sa_debug_flags")
SA_NOALLOC_SCRATCH_BYTES = 16 << 20


class SaShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("n_q_heads", ctypes.c_int32),
                ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("seq_q", ctypes.c_int32), ("seq_k", ctypes.c_int32),
                ("kv_head_of_q", ctypes.POINTER(ctypes.c_int32)),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3)]


class SaSparseParams(ctypes.Structure):
    _fields_ = [("block_q", ctypes.c_int32), ("block_k", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("local_tokens", ctypes.c_int32),
                ("granularity", ctypes.c_int32), ("theta", ctypes.POINTER(ctypes.c_float)),
                ("softmax_scale", ctypes.c_float), ("estimator", ctypes.c_int32),
                ("step", ctypes.c_int32)]


class SaLists(ctypes.Structure):
    _fields_ = [("counts", ctypes.c_void_p), ("idx", ctypes.c_void_p),
                ("stride", ctypes.c_int32), ("margins", ctypes.c_void_p)]


class SaAnchorState(ctypes.Structure):
    _fields_ = [("o", ctypes.c_void_p), ("lse", ctypes.c_void_p)]


class SaDecodeParams(ctypes.Structure):
    _fields_ = [("block_k", ctypes.c_int32), ("top_k_blocks", ctypes.c_int32),
                ("sink_tokens", ctypes.c_int32), ("local_tokens", ctypes.c_int32),
                ("n_splits", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("top_p", ctypes.c_float)]


_lib = None


def load(path: str | None = None) -> ctypes.CDLL:
    """Load libsa.so once; raise if it is missing (there is no fallback path).
    SA_LIB_PATH may name another build of the same library (kernel variants)."""
    global _lib
    if _lib is not None:
        return _lib
    _lib = open_library(path or os.environ.get("SA_LIB_PATH") or LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """A build of the library at `path` (libsa.so or libsa_debug.so) with its prototypes set;
    not cached."""
    if not os.path.exists(path):
        raise RuntimeError(f"{os.path.basename(path)} not found at {path}: build it with "
                           f"__graft_entry__.build() (hipcc --offload-arch=gfx950)")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    lib.sa_workspace_size.restype = ctypes.c_size_t
    lib.sa_workspace_size.argtypes = [ctypes.c_int, P(SaShape), vp]
    lib.sa_estimate_mask.restype = ctypes.c_int
    lib.sa_estimate_mask.argtypes = [P(SaShape), P(SaSparseParams), vp, vp, P(SaLists), vp,
                                     ctypes.c_size_t, vp]
    lib.sa_sparse_prefill.restype = ctypes.c_int
    lib.sa_sparse_prefill.argtypes = [P(SaShape), P(SaSparseParams), vp, vp, vp, P(SaLists), vp,
                                      vp, vp]
    lib.sa_estimate_mask_anchor_state.restype = ctypes.c_int
    lib.sa_estimate_mask_anchor_state.argtypes = [P(SaShape), P(SaSparseParams), vp, vp, vp,
                                                  P(SaLists), P(SaAnchorState), vp,
                                                  ctypes.c_size_t, vp]
    lib.sa_sparse_prefill_resume.restype = ctypes.c_int
    lib.sa_sparse_prefill_resume.argtypes = [P(SaShape), P(SaSparseParams), vp, vp, vp, P(SaLists),
                                             P(SaAnchorState), vp, vp, vp]
    lib.sa_build_block_summary.restype = ctypes.c_int
    lib.sa_build_block_summary.argtypes = [P(SaShape), ctypes.c_int32, vp, vp, vp, vp]
    lib.sa_sparse_decode.restype = ctypes.c_int
    lib.sa_sparse_decode.argtypes = [P(SaShape), P(SaDecodeParams), vp, vp, vp, vp, vp, vp, vp,
                                     vp, vp, ctypes.c_size_t, vp]
    lib.sa_sparse_decode_noalloc.restype = ctypes.c_int
    lib.sa_sparse_decode_noalloc.argtypes = [P(SaShape), P(SaDecodeParams), vp, vp, vp, vp, vp, vp,
                                             vp, vp, vp]
    lib.sa_quantize_block_summary.restype = ctypes.c_int
    lib.sa_quantize_block_summary.argtypes = [P(SaShape), ctypes.c_int32, vp, vp, vp, vp]
    lib.sa_sparse_decode_q4.restype = ctypes.c_int
    lib.sa_sparse_decode_q4.argtypes = [P(SaShape), P(SaDecodeParams), vp, vp, vp, vp, vp, vp, vp,
                                        vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_quantize_block_summary_fp4.restype = ctypes.c_int
    lib.sa_quantize_block_summary_fp4.argtypes = [P(SaShape), ctypes.c_int32, vp, vp, vp, vp]
    lib.sa_sparse_decode_fp4.restype = ctypes.c_int
    lib.sa_sparse_decode_fp4.argtypes = [P(SaShape), P(SaDecodeParams), vp, vp, vp, vp, vp, vp,
                                         vp, vp, vp, vp, ctypes.c_size_t, vp]
    lib.sa_calibrate_theta.restype = ctypes.c_int
    lib.sa_calibrate_theta.argtypes = [P(SaShape), P(SaSparseParams), vp, vp, vp, ctypes.c_float,
                                       ctypes.c_float, ctypes.c_int32, P(ctypes.c_float),
                                       P(ctypes.c_float), P(ctypes.c_int32), vp, ctypes.c_size_t, vp]
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_status_string.argtypes = [ctypes.c_int]
    lib.sa_debug_flags.restype = ctypes.c_uint32
    lib.sa_debug_flags.argtypes = []
    return lib


class SaError(RuntimeError):
    def __init__(self, status: int, where: str):
        msg = load().sa_status_string(status).decode()
        super().__init__(f"{where}: status {status} ({msg})")
        self.status = status


def check(status: int, where: str) -> None:
    if status != SA_OK:
        raise SaError(status, where)
