"""A decode step captured in a HIP graph replays to the same bits as the eager step.

The step is what a serving loop would capture once and replay: LIST selection and
sparse decode attention on one stream, the local heads on a second stream joined by
events.  The library allocates nothing and records no memset, so the captured graph
holds kernel nodes only.  Every replay is checked (LIST, counts, thresholds, outputs,
lse), with eager work on the same buffers and a synchronisation between replays; the
eager step itself is checked against the oracle.
"""
import pytest
import torch

from synth import DECODE_32K, make_inputs, scaled
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def test_decode_step_graph_replays_match_eager():
    import long_context_sparse_rtp_amd as rtp
    cfg = scaled(DECODE_32K, name="graph_decode", batch=3, seqlen=5000)
    _say(f"[case] graph decode B={cfg.batch} L={cfg.seqlen}")
    inp = make_inputs(cfg, DEV)
    prob = rtp.Problem.from_inputs(inp)
    main, side = torch.cuda.Stream(), torch.cuda.Stream()   # default priority, both
    main.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(main):
        k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k, stream=main)
        sel = rtp.Selection.empty(prob, rtp.RTP_SEL_LIST, DEV)
        ws_sel = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SELECT, rtp.RTP_SEL_LIST),
                             dtype=torch.uint8, device=DEV)
        ws_dec = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SPARSE_DECODE), dtype=torch.uint8,
                             device=DEV)
        ws_loc = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_LOCAL), dtype=torch.uint8, device=DEV)
        out = torch.empty_like(inp.q)
        lse = torch.empty((cfg.n_q_heads, inp.total_q), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()

    def step(m):
        fork = torch.cuda.Event()
        fork.record(m)
        side.wait_event(fork)
        rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, ws_loc, stream=side)
        rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_LIST, sel, ws_sel, stream=m)
        rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out, lse, ws_dec, stream=m)
        join = torch.cuda.Event()
        join.record(side)
        m.wait_event(join)

    def lists():
        cu = inp.cu_k.tolist()
        cnt = sel.count.cpu()
        idx = sel.idx.cpu()
        return [idx[r, cu[b]:cu[b] + int(cnt[r, b])].clone() for r in range(prob.n_ret) for b in range(cfg.batch)]

    step(main)
    torch.cuda.synchronize()
    ref = dict(count=sel.count.clone(), tau=sel.tau.clone(), tie=sel.tie_pos.clone(), out=out.clone(),
               lse=lse.clone(), lists=lists())

    # the eager step against the oracle (every head of every sequence)
    pr = from_inputs(inp)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(dict(q_idx=sel.q_idx, idx=sel.idx, count=sel.count, tau=sel.tau, tie=sel.tie_pos, out=out,
                       lse=lse))
    n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(cfg.batch)], list(range(cfg.n_q_heads)),
                                   P.TOL[cfg.dtype], decode=True)
    _say(f"[result] eager step vs oracle: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]

    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=main):
        step(main)
    torch.cuda.synchronize()
    for rep in range(4):
        # eager work on the step's own buffers between replays (overwrite every output)
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        sel.idx.fill_(-1)
        sel.count.fill_(-1)
        sel.tau.fill_(float("nan"))
        sel.tie_pos.fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(sel.count, ref["count"]), f"replay {rep}: counts differ"
        assert torch.equal(sel.tau, ref["tau"]) and torch.equal(sel.tie_pos, ref["tie"]), f"replay {rep}: thresholds"
        for a, b in zip(lists(), ref["lists"]):
            assert torch.equal(a, b), f"replay {rep}: a LIST differs"
        assert torch.equal(out, ref["out"]), f"replay {rep}: outputs differ"
        assert torch.equal(lse, ref["lse"]), f"replay {rep}: lse differs"
    _say("[result] 4 graph replays bit-identical to the eager step")
