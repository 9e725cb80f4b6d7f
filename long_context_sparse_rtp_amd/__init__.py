"""Python binding of librtp.so: the RTPurbo-style sparse-attention hot path on MI355X.

Every function mirrors one C entry point of include/rtp.h under the same name.
The binding only marshals arguments: torch tensors supply device memory and the
current HIP stream, outputs that are not given are allocated with torch, and
all arithmetic runs in the HIP kernels.  There is no fallback: if the library
is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import dataclasses
from typing import Optional, Sequence

import torch

from . import _lib
from ._lib import (RTP_BF16, RTP_CALL_LOCAL, RTP_CALL_SELECT, RTP_CALL_SELECT_BLOCKS, RTP_CALL_SPARSE_DECODE,
                   RTP_CALL_SPARSE_PREFILL, RTP_F32, RTP_SEL_LIST, RTP_SEL_THRESHOLD)

__all__ = ["Problem", "Selection", "rtp_workspace_size", "rtp_index_keys", "rtp_append_kv", "rtp_select_topp", "rtp_select_topk", "rtp_select_topp_blocks",
           "rtp_sparse_attn_prefill", "rtp_sparse_attn_decode", "rtp_sparse_attn_decode_noalloc", "rtp_local_attn",
           "RtpError",
           "RTP_SEL_LIST", "RTP_SEL_THRESHOLD", "RTP_CALL_SELECT", "RTP_CALL_SPARSE_PREFILL",
           "RTP_CALL_SPARSE_DECODE", "RTP_CALL_LOCAL", "RTP_CALL_SELECT_BLOCKS", "library"]


class RtpError(RuntimeError):
    def __init__(self, status: int, call: str):
        lib = _lib.load()
        msg = lib.rtp_status_str(status).decode()
        if status == _lib.RTP_ERR_HIP:
            msg += ": " + lib.rtp_last_hip_error().decode()
        super().__init__(f"{call} failed ({status}): {msg}")
        self.status = status


def library() -> ctypes.CDLL:
    return _lib.load()


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensors passed to librtp must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, call: str) -> None:
    if status != _lib.RTP_OK:
        raise RtpError(status, call)


class Problem:
    """Host-side problem description (rtp_problem) plus the objects it points to."""

    def __init__(self, *, batch: int, n_q_heads: int, n_kv_heads: int, ret_heads: Sequence[int],
                 n_sink: int, window: int, dtype: torch.dtype, cu_seqlens_q: torch.Tensor,
                 cu_seqlens_k: torch.Tensor, max_seqlen_q: int, max_seqlen_k: int, total_q: int,
                 total_k: int, k_capacity: int = 0, ring: bool = False):
        self.ret_heads = list(int(h) for h in ret_heads)
        self._ret = (ctypes.c_int32 * max(1, len(self.ret_heads)))(*self.ret_heads)
        self.cu_q = cu_seqlens_q
        self.cu_k = cu_seqlens_k
        self.dtype = dtype
        if dtype == torch.bfloat16:
            dt = RTP_BF16
        elif dtype == torch.float32:
            dt = RTP_F32
        else:
            raise ValueError(f"unsupported dtype {dtype}")
        self.c = _lib.RtpProblem(
            batch=batch, n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=128, idx_dim=16,
            n_ret=len(self.ret_heads), ret_heads=ctypes.cast(self._ret, ctypes.POINTER(ctypes.c_int32)),
            n_sink=n_sink, window=window, dtype=dt,
            cu_seqlens_q=cu_seqlens_q.data_ptr() if cu_seqlens_q is not None else 0,
            cu_seqlens_k=cu_seqlens_k.data_ptr() if cu_seqlens_k is not None else 0,
            max_seqlen_q=max_seqlen_q, max_seqlen_k=max_seqlen_k, total_q=total_q, total_k=total_k,
            k_capacity=k_capacity, ring=1 if ring else 0)

    @property
    def n_ret(self) -> int:
        return len(self.ret_heads)

    @property
    def total_q(self) -> int:
        return int(self.c.total_q)

    @property
    def total_k(self) -> int:
        return int(self.c.total_k)

    @property
    def ref(self):
        return ctypes.byref(self.c)

    @classmethod
    def from_inputs(cls, inp, device=None) -> "Problem":
        """Problem of a ``synth.Inputs`` workload."""
        cfg = inp.cfg
        return cls(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                   ret_heads=cfg.ret_heads, n_sink=cfg.n_sink, window=cfg.window, dtype=inp.q.dtype,
                   cu_seqlens_q=inp.cu_q, cu_seqlens_k=inp.cu_k, max_seqlen_q=max(inp.seqlens_q),
                   max_seqlen_k=max(inp.seqlens_k), total_q=inp.total_q, total_k=inp.total_k)


@dataclasses.dataclass
class Selection:
    q_idx: torch.Tensor
    count: torch.Tensor
    tau: Optional[torch.Tensor] = None
    tie_pos: Optional[torch.Tensor] = None
    idx: Optional[torch.Tensor] = None

    def c(self) -> _lib.RtpSelection:
        return _lib.RtpSelection(
            q_idx=self.q_idx.data_ptr(),
            tau=self.tau.data_ptr() if self.tau is not None else None,
            tie_pos=self.tie_pos.data_ptr() if self.tie_pos is not None else None,
            count=self.count.data_ptr(),
            idx=self.idx.data_ptr() if self.idx is not None else None)

    @classmethod
    def empty(cls, prob: Problem, mode: int, device) -> "Selection":
        R, Tq, Tk = prob.n_ret, prob.total_q, prob.total_k
        kw = dict(device=device)
        s = cls(q_idx=torch.empty((R, Tq, 16), dtype=prob.dtype, **kw),
                count=torch.empty((R, Tq), dtype=torch.int32, **kw),
                tau=torch.empty((R, Tq), dtype=torch.float32, **kw),
                tie_pos=torch.empty((R, Tq), dtype=torch.int32, **kw))
        if mode == RTP_SEL_LIST:
            s.idx = torch.empty((R, Tk), dtype=torch.int32, **kw)
        return s


def rtp_workspace_size(prob: Problem, call: int, mode: int = RTP_SEL_LIST) -> int:
    return int(_lib.load().rtp_workspace_size(prob.ref, call, mode))


def _workspace(prob: Problem, call: int, mode: int, ws: Optional[torch.Tensor], device):
    n = rtp_workspace_size(prob, call, mode)
    if n == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(n, dtype=torch.uint8, device=device)
    return ws, ws.numel() * ws.element_size()


def rtp_index_keys(prob: Problem, k_pre: torch.Tensor, w_k: torch.Tensor,
                   k_idx: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    if k_idx is None:
        k_idx = torch.empty((prob.n_ret, prob.total_k, 16), dtype=k_pre.dtype, device=k_pre.device)
    st = _lib.load().rtp_index_keys(prob.ref, _ptr(k_pre), _ptr(w_k), _ptr(k_idx), _stream(stream))
    _check(st, "rtp_index_keys")
    return k_idx


def rtp_append_kv(prob: Problem, cu_seqlens_new: torch.Tensor, total_new: int, k_new: torch.Tensor,
                  v_new: torch.Tensor, k: torch.Tensor, v: torch.Tensor, k_pre_new: Optional[torch.Tensor] = None,
                  w_k: Optional[torch.Tensor] = None, k_idx: Optional[torch.Tensor] = None, stream=None) -> None:
    """Write new tokens (the last positions of every sequence) into the caches k, v (and k_idx)."""
    st = _lib.load().rtp_append_kv(prob.ref, _ptr(cu_seqlens_new), int(total_new), _ptr(k_new), _ptr(v_new),
                                   _ptr(k_pre_new), _ptr(w_k), _ptr(k), _ptr(v), _ptr(k_idx), _stream(stream))
    _check(st, "rtp_append_kv")


def rtp_select_topp(prob: Problem, q_pre: torch.Tensor, w_q: torch.Tensor, k_idx: torch.Tensor,
                    top_p: torch.Tensor, mode: int, sel: Optional[Selection] = None,
                    ws: Optional[torch.Tensor] = None, stream=None) -> Selection:
    if sel is None:
        sel = Selection.empty(prob, mode, q_pre.device)
    ws, nws = _workspace(prob, RTP_CALL_SELECT, mode, ws, q_pre.device)
    cs = sel.c()
    st = _lib.load().rtp_select_topp(prob.ref, _ptr(q_pre), _ptr(w_q), _ptr(k_idx), _ptr(top_p), mode,
                                     ctypes.byref(cs), _ptr(ws), nws, _stream(stream))
    _check(st, "rtp_select_topp")
    sel._ws = ws
    return sel


def rtp_select_topk(prob: Problem, q_pre: torch.Tensor, w_q: torch.Tensor, k_idx: torch.Tensor,
                    top_k: torch.Tensor, mode: int, sel: Optional[Selection] = None,
                    ws: Optional[torch.Tensor] = None, stream=None) -> Selection:
    if top_k.dtype != torch.int32:
        raise ValueError("top_k must be an int32 tensor [batch]")
    if sel is None:
        sel = Selection.empty(prob, mode, q_pre.device)
    ws, nws = _workspace(prob, RTP_CALL_SELECT, mode, ws, q_pre.device)
    cs = sel.c()
    st = _lib.load().rtp_select_topk(prob.ref, _ptr(q_pre), _ptr(w_q), _ptr(k_idx), _ptr(top_k), mode,
                                     ctypes.byref(cs), _ptr(ws), nws, _stream(stream))
    _check(st, "rtp_select_topk")
    sel._ws = ws
    return sel


def rtp_select_topp_blocks(prob: Problem, q_pre: torch.Tensor, w_q: torch.Tensor, k_idx: torch.Tensor,
                           top_p: torch.Tensor, sel: Optional[Selection] = None,
                           ws: Optional[torch.Tensor] = None, stream=None) -> Selection:
    """The pages' block-granular top-p (decode, LIST output)."""
    if sel is None:
        sel = Selection.empty(prob, RTP_SEL_LIST, q_pre.device)
    ws, nws = _workspace(prob, RTP_CALL_SELECT_BLOCKS, RTP_SEL_LIST, ws, q_pre.device)
    cs = sel.c()
    st = _lib.load().rtp_select_topp_blocks(prob.ref, _ptr(q_pre), _ptr(w_q), _ptr(k_idx), _ptr(top_p),
                                            ctypes.byref(cs), _ptr(ws), nws, _stream(stream))
    _check(st, "rtp_select_topp_blocks")
    sel._ws = ws
    return sel


def rtp_sparse_attn_prefill(prob: Problem, q, k, v, k_idx, sel: Selection, out: torch.Tensor,
                            lse: Optional[torch.Tensor] = None, ws=None, stream=None) -> torch.Tensor:
    cs = sel.c()
    st = _lib.load().rtp_sparse_attn_prefill(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(k_idx), ctypes.byref(cs),
                                             _ptr(out), _ptr(lse), None, 0, _stream(stream))
    _check(st, "rtp_sparse_attn_prefill")
    return out


def rtp_sparse_attn_decode(prob: Problem, q, k, v, sel: Selection, out: torch.Tensor,
                           lse: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                           stream=None) -> torch.Tensor:
    ws, nws = _workspace(prob, RTP_CALL_SPARSE_DECODE, RTP_SEL_LIST, ws, q.device)
    cs = sel.c()
    st = _lib.load().rtp_sparse_attn_decode(prob.ref, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs), _ptr(out),
                                            _ptr(lse), _ptr(ws), nws, _stream(stream))
    _check(st, "rtp_sparse_attn_decode")
    return out


def rtp_sparse_attn_decode_noalloc(prob: Problem, q, k, v, sel: Selection, out: torch.Tensor,
                                   lse: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """rtp_sparse_attn_decode on the library's static scratch: no workspace argument and
    nothing allocated here or in the library (the caller owns q, k, v, sel, out, lse)."""
    cs = sel.c()
    st = _lib.load().rtp_sparse_attn_decode_noalloc(prob.ref, _ptr(q), _ptr(k), _ptr(v), ctypes.byref(cs),
                                                    _ptr(out), _ptr(lse), _stream(stream))
    _check(st, "rtp_sparse_attn_decode_noalloc")
    return out


def rtp_local_attn(prob: Problem, q, k, v, out: torch.Tensor, lse: Optional[torch.Tensor] = None,
                   ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    ws, nws = _workspace(prob, RTP_CALL_LOCAL, RTP_SEL_LIST, ws, q.device)
    st = _lib.load().rtp_local_attn(prob.ref, _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), _ptr(ws), nws,
                                    _stream(stream))
    _check(st, "rtp_local_attn")
    return out
