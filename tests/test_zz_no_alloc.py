"""The decode attention entry point that allocates nothing (rtp_sparse_attn_decode_noalloc)
against the one that takes a workspace (rtp_sparse_attn_decode): same selection, same
kernels, so the outputs must be bit-identical.  Two calls in a row on one device, the
second with a smaller problem, so the shared static scratch is reused with a stale tail."""
import pytest
import torch

from synth import DECODE_32K, make_inputs, scaled
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _both(cfg):
    import long_context_sparse_rtp_amd as rtp
    inp = make_inputs(cfg, DEV)
    prob = rtp.Problem.from_inputs(inp)
    k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k)
    sel = rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_LIST)
    need = rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SPARSE_DECODE)
    assert 0 < need <= rtp._lib.RTP_NOALLOC_SCRATCH_BYTES
    out_a = torch.full_like(inp.q, float("nan"))
    lse_a = torch.full((cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=DEV)
    out_b = out_a.clone()
    lse_b = lse_a.clone()
    rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out_a, lse_a)
    rtp.rtp_sparse_attn_decode_noalloc(prob, inp.q, inp.k, inp.v, sel, out_b, lse_b)
    torch.cuda.synchronize()
    ret = list(cfg.ret_heads)
    assert torch.equal(out_a[:, ret], out_b[:, ret])
    assert torch.equal(lse_a[ret], lse_b[ret])
    return inp, k_idx, out_b, lse_b


@pytest.mark.parametrize("big,small", [
    # one retrieval head per KV group: the split-list kernel
    (dict(batch=8, seqlen=32768), dict(batch=2, seqlens=(3000, 700))),
    # three retrieval heads in one KV group: the union kernel
    (dict(batch=4, seqlens=(9000, 1, 4000, 12000), n_q_heads=8, n_kv_heads=2, ret_heads=(0, 1, 2, 5),
          window=96, needles_per_seq=8),
     dict(batch=2, seqlens=(64, 2000), n_q_heads=8, n_kv_heads=2, ret_heads=(0, 1, 2, 5), window=96,
          needles_per_seq=4)),
])
def test_noalloc_matches_workspace_call_twice(big, small):
    for i, kw in enumerate((big, small)):
        cfg = scaled(DECODE_32K, name=f"noalloc_{i}", **kw)
        _say(f"[case] {cfg.name} {kw}")
        inp, k_idx, out, lse = _both(cfg)
        if i == 1:
            # the smaller call against the oracle as well
            pr = from_inputs(inp)
            pr.k_idx = k_idx.cpu()
            import long_context_sparse_rtp_amd as rtp
            prob = rtp.Problem.from_inputs(inp)
            sel = rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_LIST)
            out2 = torch.full_like(inp.q, float("nan"))
            lse2 = torch.full_like(lse, float("nan"))
            rtp.rtp_sparse_attn_decode_noalloc(prob, inp.q, inp.k, inp.v, sel, out2, lse2)
            rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out2, lse2)
            torch.cuda.synchronize()
            g = P.to_host(dict(q_idx=sel.q_idx, idx=sel.idx, count=sel.count, out=out2, lse=lse2))
            n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(cfg.batch)], list(range(cfg.n_q_heads)),
                                           P.TOL[cfg.dtype], decode=True)
            _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
            assert not fails, fails[:3]


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    import long_context_sparse_rtp_amd as rtp
    # 64 sequences of 262144 keys with 32 retrieval heads: far more split partials than 16 MiB
    B, L = 64, 262144
    cu_q = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    cu_k = torch.arange(B + 1, dtype=torch.int32, device=DEV) * L
    prob = rtp.Problem(batch=B, n_q_heads=32, n_kv_heads=4, ret_heads=list(range(32)), n_sink=4, window=1024,
                       dtype=torch.bfloat16, cu_seqlens_q=cu_q, cu_seqlens_k=cu_k, max_seqlen_q=1, max_seqlen_k=L,
                       total_q=B, total_k=B * L)
    assert rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SPARSE_DECODE) > rtp._lib.RTP_NOALLOC_SCRATCH_BYTES
    q = torch.empty((B, 32, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.empty((16, 4, 128), dtype=torch.bfloat16, device=DEV)   # never read: rejected before launch
    sel = rtp.Selection(q_idx=torch.empty((32, B, 16), dtype=torch.bfloat16, device=DEV),
                        count=torch.empty((32, B), dtype=torch.int32, device=DEV),
                        idx=torch.empty((32, 16), dtype=torch.int32, device=DEV))
    with pytest.raises(rtp.RtpError) as ei:
        rtp.rtp_sparse_attn_decode_noalloc(prob, q, kv, kv, sel, torch.empty_like(q))
    assert ei.value.status == 3
    assert "static scratch" in rtp.library().rtp_last_hip_error().decode()
