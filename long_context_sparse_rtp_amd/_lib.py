"""ctypes declarations of librtp.so (include/rtp.h).  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "librtp.so")

RTP_OK, RTP_ERR_INVALID_ARG, RTP_ERR_UNSUPPORTED, RTP_ERR_WORKSPACE_TOO_SMALL, RTP_ERR_HIP = range(5)
RTP_F32, RTP_BF16 = 0, 1
RTP_SEL_LIST, RTP_SEL_THRESHOLD = 0, 1
RTP_CALL_SELECT, RTP_CALL_SPARSE_PREFILL, RTP_CALL_SPARSE_DECODE, RTP_CALL_LOCAL, RTP_CALL_SELECT_BLOCKS = 1, 2, 3, 4, 5
RTP_NOALLOC_SCRATCH_BYTES = 16 << 20

EXPORTED = ("rtp_workspace_size", "rtp_index_keys", "rtp_append_kv", "rtp_select_topp", "rtp_select_topk", "rtp_select_topp_blocks",
            "rtp_sparse_attn_prefill",
            "rtp_sparse_attn_decode", "rtp_sparse_attn_decode_noalloc", "rtp_local_attn", "rtp_status_str",
            "rtp_last_hip_error")


class RtpProblem(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("idx_dim", ctypes.c_int32),
        ("n_ret", ctypes.c_int32),
        ("ret_heads", ctypes.POINTER(ctypes.c_int32)),
        ("n_sink", ctypes.c_int32),
        ("window", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("cu_seqlens_q", ctypes.c_void_p),
        ("cu_seqlens_k", ctypes.c_void_p),
        ("max_seqlen_q", ctypes.c_int32),
        ("max_seqlen_k", ctypes.c_int32),
        ("total_q", ctypes.c_int64),
        ("total_k", ctypes.c_int64),
        ("k_capacity", ctypes.c_int64),
        ("ring", ctypes.c_int32),
    ]


class RtpSelection(ctypes.Structure):
    _fields_ = [
        ("q_idx", ctypes.c_void_p),
        ("tau", ctypes.c_void_p),
        ("tie_pos", ctypes.c_void_p),
        ("count", ctypes.c_void_p),
        ("idx", ctypes.c_void_p),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load librtp.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m long_context_sparse_rtp_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER(RtpProblem)
    S = ctypes.POINTER(RtpSelection)
    vp, sz, i32 = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32
    lib.rtp_workspace_size.argtypes = [P, i32, i32]
    lib.rtp_workspace_size.restype = sz
    lib.rtp_index_keys.argtypes = [P, vp, vp, vp, vp]
    lib.rtp_index_keys.restype = i32
    lib.rtp_append_kv.argtypes = [P, vp, ctypes.c_int64, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.rtp_append_kv.restype = i32
    lib.rtp_select_topp.argtypes = [P, vp, vp, vp, vp, i32, S, vp, sz, vp]
    lib.rtp_select_topp.restype = i32
    lib.rtp_select_topk.argtypes = [P, vp, vp, vp, vp, i32, S, vp, sz, vp]
    lib.rtp_select_topk.restype = i32
    lib.rtp_select_topp_blocks.argtypes = [P, vp, vp, vp, vp, S, vp, sz, vp]
    lib.rtp_select_topp_blocks.restype = i32
    lib.rtp_sparse_attn_prefill.argtypes = [P, vp, vp, vp, vp, S, vp, vp, vp, sz, vp]
    lib.rtp_sparse_attn_prefill.restype = i32
    lib.rtp_sparse_attn_decode.argtypes = [P, vp, vp, vp, S, vp, vp, vp, sz, vp]
    lib.rtp_sparse_attn_decode.restype = i32
    lib.rtp_sparse_attn_decode_noalloc.argtypes = [P, vp, vp, vp, S, vp, vp, vp]
    lib.rtp_sparse_attn_decode_noalloc.restype = i32
    lib.rtp_local_attn.argtypes = [P, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.rtp_local_attn.restype = i32
    lib.rtp_status_str.argtypes = [i32]
    lib.rtp_status_str.restype = ctypes.c_char_p
    lib.rtp_last_hip_error.argtypes = []
    lib.rtp_last_hip_error.restype = ctypes.c_char_p
    _lib = lib
    return lib
