"""GPU parity of the tile-skipping retrieval attention (the kernel instance that
marks the key tiles holding a selected pair before staging any K/V) in the
layouts the masked-dense loop already covers: a ragged batch whose sequences
take different instances in one launch, and a chunked prefill whose queries sit
at the end of a longer key range.  Selections are clustered in a few 64-key
blocks (synth.gen.plant_blocks), the case the skipping is for; the oracle
recomputes every checked row from the definition (section 3.4 of the page
"Full Attention Strikes Back ...", Eq. 5 and the attention after it)."""
import pytest
import torch

from synth import PREFILL_128K, make_inputs, sample_rows, scaled
from synth.gen import plant_blocks
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def test_skip_ragged_batch_mixed_instances():
    # sequence 0: clustered and long (its rows past 4 k keys go to the skipping
    # instance); sequence 1: shorter than 4 k (masked-dense); sequence 2: unclustered
    # scores (every tile needed, masked-dense by the tile sample)
    cfg = scaled(PREFILL_128K, name="skip_ragged", batch=3, seqlens=(9000, 300, 6000), window=256,
                 needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    plant_blocks(inp, blocks=(3, 20, 21, 77, 120))
    top_k = [192, 192, 192]
    g = P.to_host(P.run_prefill(inp, top_k=top_k))
    pr = from_inputs(inp)
    pr.top_k = top_k
    rows = [(0, i) for i in sample_rows(scaled(cfg, seqlen=9000), 40, [767, 768, 8999])]
    rows += [(1, i) for i in (0, 191, 192, 299)]
    rows += [(2, i) for i in sample_rows(scaled(cfg, seqlen=6000), 24, [768, 5999])]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


@pytest.mark.parametrize("kind", ["topk", "topp"])
def test_skip_chunked_prefill(kind):
    # the last 2000 queries of a 9000-key sequence (query i at position 7000 + i)
    import long_context_sparse_rtp_amd as rtp
    cfg = scaled(PREFILL_128K, name=f"skip_chunk_{kind}", seqlen=9000, window=256, needles="none", top_p=0.5)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    plant_blocks(inp, blocks=(3, 20, 21, 77, 120))
    nq, L = 2000, cfg.seqlen
    q, q_pre = inp.q[L - nq:].contiguous(), inp.q_pre[L - nq:].contiguous()
    cu_q = torch.tensor([0, nq], dtype=torch.int32, device=DEV)
    prob = rtp.Problem(batch=1, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, ret_heads=cfg.ret_heads,
                       n_sink=cfg.n_sink, window=cfg.window, dtype=inp.q.dtype, cu_seqlens_q=cu_q,
                       cu_seqlens_k=inp.cu_k, max_seqlen_q=nq, max_seqlen_k=L, total_q=nq, total_k=inp.total_k)
    k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k)
    if kind == "topk":
        top_k = [192]
        sel = rtp.rtp_select_topk(prob, q_pre, inp.w_q, k_idx, torch.tensor(top_k, dtype=torch.int32, device=DEV),
                                  rtp.RTP_SEL_THRESHOLD)
    else:
        top_k = None
        sel = rtp.rtp_select_topp(prob, q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_THRESHOLD)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((cfg.n_q_heads, nq), float("nan"), dtype=torch.float32, device=DEV)
    rtp.rtp_sparse_attn_prefill(prob, q, inp.k, inp.v, k_idx, sel, out, lse)
    rtp.rtp_local_attn(prob, q, inp.k, inp.v, out, lse)
    P.sync()
    pr = from_inputs(inp)
    pr.q, pr.q_pre = q.cpu(), q_pre.cpu()
    pr.cu_q = [0, nq]
    if top_k is not None:
        pr.top_k = top_k
    g = P.to_host(dict(q_idx=sel.q_idx, tau=sel.tau, tie=sel.tie_pos, count=sel.count, out=out, lse=lse))
    rows = [(0, i) for i in sorted(set(sample_rows(scaled(cfg, seqlen=nq), 40, [0, 255, 256, 679, 680, 1999])))]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}, mean count "
         f"{float(g['count'][:, :nq].mean()):.1f}")
    assert not fails, fails[:5]
