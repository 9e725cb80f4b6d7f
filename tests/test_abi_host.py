"""Host-side checks of the C ABI (no GPU): the library loads, exports every call of
include/rtp.h, and rejects invalid arguments before launching anything."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _lib():
    from long_context_sparse_rtp_amd import _lib as L
    return L, L.load()


def _declared_calls():
    src = open(os.path.join(ROOT, "include", "rtp.h")).read()
    return sorted(set(re.findall(r"RTP_API\s+[\w\s\*]*?\b(rtp_\w+)\s*\(", src)))


def test_header_and_binding_agree():
    L, _ = _lib()
    assert _declared_calls() == sorted(L.EXPORTED)


def test_library_exports_every_declared_call():
    L, lib = _lib()
    for name in _declared_calls():
        assert hasattr(lib, name), name


def _problem(L, **kw):
    ret = (ctypes.c_int32 * 4)(0, 8, 16, 24)
    cu = (ctypes.c_int32 * 2)(0, 1024)   # host memory stands in for a device pointer: never dereferenced
    base = dict(batch=1, n_q_heads=32, n_kv_heads=4, head_dim=128, idx_dim=16, n_ret=4,
                ret_heads=ctypes.cast(ret, ctypes.POINTER(ctypes.c_int32)), n_sink=4, window=256,
                dtype=L.RTP_BF16, cu_seqlens_q=ctypes.addressof(cu), cu_seqlens_k=ctypes.addressof(cu),
                max_seqlen_q=1024, max_seqlen_k=1024, total_q=1024, total_k=1024)
    base.update(kw)
    p = L.RtpProblem(**base)
    p._keep = (ret, cu)
    return p


@pytest.mark.parametrize("field,value,expect", [
    ("head_dim", 64, 2), ("idx_dim", 32, 2), ("n_kv_heads", 5, 1), ("batch", 0, 1), ("window", 0, 1),
    ("n_sink", -1, 1), ("n_sink", 65, 2), ("n_ret", 33, 1), ("dtype", 7, 1), ("max_seqlen_q", 2048, 1),
    ("total_k", 4096, 1), ("n_q_heads", 129, 1),
])
def test_invalid_problem_rejected(field, value, expect):
    L, lib = _lib()
    p = _problem(L, **{field: value})
    st = lib.rtp_local_attn(ctypes.byref(p), 16, 16, 16, 16, None, None, 0, None)
    assert st == expect
    assert lib.rtp_workspace_size(ctypes.byref(p), L.RTP_CALL_SELECT, L.RTP_SEL_LIST) == 0


def test_ret_heads_must_be_ascending():
    L, lib = _lib()
    ret = (ctypes.c_int32 * 4)(0, 16, 8, 24)
    p = _problem(L, ret_heads=ctypes.cast(ret, ctypes.POINTER(ctypes.c_int32)))
    assert lib.rtp_index_keys(ctypes.byref(p), 16, 16, 16, None) == L.RTP_ERR_INVALID_ARG


def test_misaligned_and_null_pointers_rejected():
    L, lib = _lib()
    p = _problem(L)
    assert lib.rtp_index_keys(ctypes.byref(p), 8, 16, 16, None) == L.RTP_ERR_INVALID_ARG
    assert lib.rtp_index_keys(ctypes.byref(p), None, 16, 16, None) == L.RTP_ERR_INVALID_ARG
    sel = L.RtpSelection(q_idx=16, tau=16, tie_pos=16, count=16, idx=16)
    assert lib.rtp_sparse_attn_prefill(ctypes.byref(p), 16, 16, 16, 16, ctypes.byref(sel), 24, None, None, 0,
                                       None) == L.RTP_ERR_INVALID_ARG


def test_list_mode_needs_one_query_per_sequence():
    L, lib = _lib()
    p = _problem(L)
    sel = L.RtpSelection(q_idx=16, tau=16, tie_pos=16, count=16, idx=16)
    st = lib.rtp_select_topp(ctypes.byref(p), 16, 16, 16, 16, L.RTP_SEL_LIST, ctypes.byref(sel), 16, 1 << 30, None)
    assert st == L.RTP_ERR_UNSUPPORTED
    st = lib.rtp_sparse_attn_decode(ctypes.byref(p), 16, 16, 16, ctypes.byref(sel), 16, None, 16, 1 << 30, None)
    assert st == L.RTP_ERR_UNSUPPORTED


def test_workspace_too_small_rejected():
    L, lib = _lib()
    p = _problem(L, max_seqlen_q=1, total_q=1, max_seqlen_k=32768, total_k=32768)
    need = lib.rtp_workspace_size(ctypes.byref(p), L.RTP_CALL_SELECT, L.RTP_SEL_LIST)
    assert need >= 4 * 4 * 32768
    sel = L.RtpSelection(q_idx=16, tau=16, tie_pos=16, count=16, idx=16)
    st = lib.rtp_select_topp(ctypes.byref(p), 16, 16, 16, 16, L.RTP_SEL_LIST, ctypes.byref(sel), 16, need - 1, None)
    assert st == L.RTP_ERR_WORKSPACE_TOO_SMALL
    assert lib.rtp_workspace_size(ctypes.byref(p), L.RTP_CALL_SPARSE_DECODE, 0) > 0
    assert lib.rtp_workspace_size(ctypes.byref(p), L.RTP_CALL_SPARSE_PREFILL, 0) == 0


def test_status_strings():
    L, lib = _lib()
    assert lib.rtp_status_str(0) == b"ok"
    assert lib.rtp_status_str(3) == b"workspace too small"
    assert lib.rtp_last_hip_error() == b""


def _decode_problem(L, **kw):
    base = dict(max_seqlen_q=1, total_q=1, max_seqlen_k=1000, total_k=1024)
    base.update(kw)
    return _problem(L, **base)


def test_capacity_layout_validation():
    L, lib = _lib()
    size = lambda p: lib.rtp_workspace_size(ctypes.byref(p), L.RTP_CALL_SELECT, L.RTP_SEL_LIST)
    # capacity 1024 rows per sequence holding up to 1000 keys: valid
    assert size(_decode_problem(L, k_capacity=1024)) > 0
    # rows must be batch * capacity, the longest sequence must fit, capacity >= 0
    assert size(_decode_problem(L, k_capacity=1024, total_k=1000)) == 0
    assert size(_decode_problem(L, k_capacity=512, total_k=512)) == 0
    assert size(_decode_problem(L, k_capacity=-1)) == 0


def test_ring_layout_validation():
    L, lib = _lib()
    none = ctypes.cast((ctypes.c_int32 * 1)(0), ctypes.POINTER(ctypes.c_int32))
    # ring of 4 sinks + 256 window rows, local heads only, one query per sequence
    ok = dict(n_ret=0, ret_heads=none, ring=1, k_capacity=260, total_k=260, max_seqlen_k=100000)
    assert lib.rtp_workspace_size(ctypes.byref(_decode_problem(L, **ok)), L.RTP_CALL_LOCAL, 0) > 0
    bad_cap = dict(ok, k_capacity=256, total_k=256)
    assert lib.rtp_workspace_size(ctypes.byref(_decode_problem(L, **bad_cap)), L.RTP_CALL_LOCAL, 0) == 0
    p = _decode_problem(L, **dict(ok, ring=2))
    assert lib.rtp_local_attn(ctypes.byref(p), 16, 16, 16, 16, None, None, 0, None) == L.RTP_ERR_INVALID_ARG
    # retrieval heads need the whole cache, and a ring serves one query per sequence
    p = _decode_problem(L, ring=1, k_capacity=260, total_k=260)
    assert lib.rtp_local_attn(ctypes.byref(p), 16, 16, 16, 16, None, None, 0, None) == L.RTP_ERR_UNSUPPORTED
    p = _problem(L, n_ret=0, ret_heads=none, ring=1, k_capacity=260, total_k=260, max_seqlen_q=2, total_q=2)
    assert lib.rtp_local_attn(ctypes.byref(p), 16, 16, 16, 16, None, None, 0, None) == L.RTP_ERR_UNSUPPORTED


def test_append_kv_validation():
    L, lib = _lib()
    p = _decode_problem(L, k_capacity=1024)
    call = lambda p, total_new, *ptrs: lib.rtp_append_kv(ctypes.byref(p), 16, total_new, *ptrs, None)
    assert call(p, 1, 16, 16, 16, 16, 16, 16, None) == L.RTP_ERR_INVALID_ARG      # k_idx missing with n_ret > 0
    assert call(p, 1, 16, 8, 16, 16, 16, 16, 16) == L.RTP_ERR_INVALID_ARG         # misaligned v_new
    assert call(p, 2048, 16, 16, 16, 16, 16, 16, 16) == L.RTP_ERR_INVALID_ARG     # more new tokens than rows
    assert call(p, -1, 16, 16, 16, 16, 16, 16, 16) == L.RTP_ERR_INVALID_ARG
    assert call(p, 0, None, None, None, None, None, None, None) == L.RTP_OK        # nothing to append
