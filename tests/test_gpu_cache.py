"""GPU tests of the cache layouts and the append path: the per-sequence capacity
layout (keys grow in place), rtp_append_kv (new K/V rows plus their index keys), and
the ring that keeps only sinks + window for local heads.  Every output is checked
against the oracle on the equivalent packed problem; appended rows and index keys
are checked bit for bit."""
import numpy as np
import pytest
import torch

from synth import DECODE_32K, TINY_PREFILL, make_inputs, scaled
from oracle.problem import from_inputs
from oracle import rtp_oracle as O

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _rtp():
    import long_context_sparse_rtp_amd as rtp
    return rtp


def _to_capacity(x, cu, cap):
    """[T, ...] packed rows -> [B * cap, ...] with sequence b at rows b * cap (zeros elsewhere)."""
    B = len(cu) - 1
    out = torch.zeros((B * cap,) + tuple(x.shape[1:]), dtype=x.dtype, device=x.device)
    for b in range(B):
        out[b * cap: b * cap + cu[b + 1] - cu[b]] = x[cu[b]:cu[b + 1]]
    return out


def _problem(inp, cap, lengths=None, ring=False, ret_heads=None, n_q_heads=None):
    rtp = _rtp()
    cfg = inp.cfg
    lens = list(inp.seqlens_k) if lengths is None else list(lengths)
    cu_k = torch.tensor(np.concatenate([[0], np.cumsum(lens)]), dtype=torch.int32, device=DEV)
    return rtp.Problem(batch=cfg.batch, n_q_heads=n_q_heads or cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads,
                       ret_heads=cfg.ret_heads if ret_heads is None else ret_heads, n_sink=cfg.n_sink,
                       window=cfg.window, dtype=inp.q.dtype, cu_seqlens_q=inp.cu_q, cu_seqlens_k=cu_k,
                       max_seqlen_q=max(inp.seqlens_q), max_seqlen_k=max(lens), total_q=inp.total_q,
                       total_k=cfg.batch * cap, k_capacity=cap, ring=ring)


def _decode_on(prob, inp, k, v, k_idx):
    """select (LIST) -> sparse decode + local decode on caches in prob's layout."""
    rtp = _rtp()
    sel = rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_LIST)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((inp.cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=DEV)
    rtp.rtp_sparse_attn_decode(prob, inp.q, k, v, sel, out, lse)
    rtp.rtp_local_attn(prob, inp.q, k, v, out, lse)
    P.sync()
    return sel, out, lse


def _check_decode_capacity(inp, cap, sel, out, lse, pr):
    """Compare a capacity-layout decode with the oracle: the LIST slices are moved to
    the packed offsets the checker expects."""
    cfg = inp.cfg
    cu = inp.cu_k.cpu().tolist()
    idx = sel.idx.cpu().numpy()
    idx_packed = np.zeros((cfg.n_ret, inp.total_k), dtype=idx.dtype)
    for b in range(cfg.batch):
        idx_packed[:, cu[b]:cu[b + 1]] = idx[:, b * cap: b * cap + cu[b + 1] - cu[b]]
    g = P.to_host(dict(q_idx=sel.q_idx, count=sel.count, out=out, lse=lse))
    g["idx"] = idx_packed
    n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(cfg.batch)], list(range(cfg.n_q_heads)),
                                   P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


DEC = scaled(DECODE_32K, name="cache_decode", batch=3, seqlens=(5000, 300, 7000), needles="query",
             needles_per_seq=16)


# two retrieval heads per KV group: the decode attention takes the union path
DEC_UNION = scaled(DECODE_32K, name="cache_decode_union", batch=3, seqlens=(5000, 300, 7000), n_q_heads=8,
                   n_kv_heads=2, ret_heads=(0, 2, 4, 5), window=200, needles="query", needles_per_seq=16)


@pytest.mark.parametrize("cfg", [DEC, DEC_UNION], ids=["one_retrieval_head_per_group", "union"])
def test_capacity_layout_decode_matches_oracle_and_packed(cfg):
    rtp = _rtp()
    _say(f"[case] capacity layout decode {cfg.name}")
    inp = make_inputs(cfg, DEV)
    cu = inp.cu_k.cpu().tolist()
    cap = 8192
    prob = _problem(inp, cap)
    k, v, kp = (_to_capacity(x, cu, cap) for x in (inp.k, inp.v, inp.k_pre))
    k_idx = rtp.rtp_index_keys(prob, kp, inp.w_k)
    sel, out, lse = _decode_on(prob, inp, k, v, k_idx)
    _check_decode_capacity(inp, cap, sel, out, lse, from_inputs(inp))
    # the same kernels on the packed layout give the same bits
    g = P.run_decode(inp, rtp.rtp_index_keys(rtp.Problem.from_inputs(inp), inp.k_pre, inp.w_k))
    assert torch.equal(g["out"], out) and torch.equal(g["count"], sel.count)


def test_capacity_layout_prefill_chunk():
    # a chunked prefill: the last 200 queries of each sequence against a cache of
    # capacity 1024 that already holds the whole sequence
    rtp = _rtp()
    _say("[case] capacity layout prefill chunk")
    cfg = scaled(TINY_PREFILL, name="cache_prefill", batch=2, seqlens=(700, 300), dtype="bf16", n_q_heads=8,
                 n_kv_heads=2, ret_heads=(0, 5), window=64)
    inp = make_inputs(cfg, DEV)
    cu = inp.cu_k.cpu().tolist()
    cap = 1024
    nq = 200
    qrows = torch.cat([torch.arange(cu[b + 1] - nq, cu[b + 1]) for b in range(cfg.batch)]).to(DEV)
    cu_q = torch.tensor([0, nq, 2 * nq], dtype=torch.int32, device=DEV)
    prob = rtp.Problem(batch=2, n_q_heads=8, n_kv_heads=2, ret_heads=(0, 5), n_sink=cfg.n_sink, window=64,
                       dtype=inp.q.dtype, cu_seqlens_q=cu_q, cu_seqlens_k=inp.cu_k, max_seqlen_q=nq,
                       max_seqlen_k=700, total_q=2 * nq, total_k=2 * cap, k_capacity=cap)
    k, v, kp = (_to_capacity(x, cu, cap) for x in (inp.k, inp.v, inp.k_pre))
    q, q_pre = inp.q[qrows].contiguous(), inp.q_pre[qrows].contiguous()
    k_idx = rtp.rtp_index_keys(prob, kp, inp.w_k)
    sel = rtp.rtp_select_topp(prob, q_pre, inp.w_q, k_idx, inp.top_p, rtp.RTP_SEL_THRESHOLD)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((8, 2 * nq), float("nan"), dtype=torch.float32, device=DEV)
    rtp.rtp_sparse_attn_prefill(prob, q, k, v, k_idx, sel, out, lse)
    rtp.rtp_local_attn(prob, q, k, v, out, lse)
    P.sync()
    # oracle: the packed problem with only the chunk's query rows
    pr = from_inputs(inp)
    pr.q, pr.q_pre = q.cpu(), q_pre.cpu()
    pr.cu_q = [0, nq, 2 * nq]
    g = P.to_host(dict(q_idx=sel.q_idx, tau=sel.tau, tie=sel.tie_pos, count=sel.count, out=out, lse=lse))
    rows = [(b, i) for b in range(2) for i in range(nq)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(8)), P.TOL[cfg.dtype])
    _say(f"[result] chunk: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


def test_append_step_bit_exact_then_decode():
    rtp = _rtp()
    _say("[case] append one token per sequence, then decode")
    inp = make_inputs(DEC, DEV)
    cu = inp.cu_k.cpu().tolist()
    B, cap = DEC.batch, 8192
    lens = [cu[b + 1] - cu[b] for b in range(B)]
    last = torch.tensor([cu[b + 1] - 1 for b in range(B)], device=DEV)
    # cache before the step: every sequence without its last token
    k, v, kp = (_to_capacity(x, cu, cap) for x in (inp.k, inp.v, inp.k_pre))
    for b in range(B):
        for t in (k, v, kp):
            t[b * cap + lens[b] - 1].zero_()
    before = _problem(inp, cap, lengths=[n - 1 for n in lens])
    k_idx = rtp.rtp_index_keys(before, kp, inp.w_k)
    # the step: append the last tokens (positions L - 1 of the grown sequences)
    after = _problem(inp, cap)
    cu_new = torch.arange(B + 1, dtype=torch.int32, device=DEV)
    k_new, v_new, kp_new = (x[last].contiguous() for x in (inp.k, inp.v, inp.k_pre))
    rtp.rtp_append_kv(after, cu_new, B, k_new, v_new, k, v, k_pre_new=kp_new, w_k=inp.w_k, k_idx=k_idx)
    P.sync()
    for b in range(B):
        row = b * cap + lens[b] - 1
        assert torch.equal(k[row], inp.k[cu[b + 1] - 1]) and torch.equal(v[row], inp.v[cu[b + 1] - 1])
    # appended index keys: bit-identical to a one-pass projection and to the oracle
    kp[torch.tensor([b * cap + lens[b] - 1 for b in range(B)], device=DEV)] = kp_new
    full = rtp.rtp_index_keys(after, kp, inp.w_k)
    P.sync()
    pr = from_inputs(inp)
    for b in range(B):
        row = b * cap + lens[b] - 1
        assert torch.equal(k_idx[:, row], full[:, row])
        for r, h in enumerate(DEC.ret_heads):
            exact = O.project(pr.k_pre[cu[b + 1] - 1, pr.kv_of(h)].to(torch.float64).numpy(), pr.w("w_k", r),
                              pr.dtype)
            assert np.array_equal(k_idx[r, row].float().cpu().numpy().astype(np.float64), exact)
    sel, out, lse = _decode_on(after, inp, k, v, k_idx)
    _check_decode_capacity(inp, cap, sel, out, lse, pr)


def test_serving_loop_three_steps():
    # prefill-sized caches, then three decode steps: append, select, attend; each
    # step is checked against the oracle on the sequences as they stand
    rtp = _rtp()
    steps = 3
    cfg = scaled(DECODE_32K, name="cache_loop", batch=2, seqlens=(3000 + steps, 900 + steps), needles="query",
                 needles_per_seq=8)
    inp = make_inputs(cfg, DEV)
    cu = inp.cu_k.cpu().tolist()
    B, cap = 2, 4096
    full_len = [cu[b + 1] - cu[b] for b in range(B)]
    k = torch.zeros((B * cap, cfg.n_kv_heads, 128), dtype=inp.k.dtype, device=DEV)
    v, kp = torch.zeros_like(k), torch.zeros_like(k)
    # fill the first L - steps tokens with one append call each sequence (a prompt)
    start = [n - steps for n in full_len]
    prompt_rows = torch.cat([torch.arange(cu[b], cu[b] + start[b]) for b in range(B)]).to(DEV)
    cu_new = torch.tensor([0, start[0], start[0] + start[1]], dtype=torch.int32, device=DEV)
    prob0 = _problem(inp, cap, lengths=start)
    k_idx = torch.zeros((cfg.n_ret, B * cap, 16), dtype=inp.k.dtype, device=DEV)
    rtp.rtp_append_kv(prob0, cu_new, int(sum(start)), inp.k[prompt_rows].contiguous(), inp.v[prompt_rows].contiguous(),
                      k, v, k_pre_new=inp.k_pre[prompt_rows].contiguous(), w_k=inp.w_k, k_idx=k_idx)
    for s in range(steps):
        _say(f"[case] serving loop step {s}")
        lens = [start[b] + s + 1 for b in range(B)]
        prob = _problem(inp, cap, lengths=lens)
        rows = torch.tensor([cu[b] + lens[b] - 1 for b in range(B)], device=DEV)
        rtp.rtp_append_kv(prob, torch.arange(B + 1, dtype=torch.int32, device=DEV), B, inp.k[rows].contiguous(),
                          inp.v[rows].contiguous(), k, v, k_pre_new=inp.k_pre[rows].contiguous(), w_k=inp.w_k,
                          k_idx=k_idx)
        # this step's queries: the generator's queries stand in for the new token's
        sel, out, lse = _decode_on(prob, inp, k, v, k_idx)
        pr = from_inputs(inp)
        pr.cu_k = [0, lens[0], lens[0] + lens[1]]
        keep = torch.cat([torch.arange(cu[b], cu[b] + lens[b]) for b in range(B)])
        pr.k, pr.v, pr.k_pre = inp.k[keep].cpu(), inp.v[keep].cpu(), inp.k_pre[keep].cpu()
        packed_inp = type("Packed", (), {})()
        packed_inp.cfg, packed_inp.total_k = cfg, int(sum(lens))
        packed_inp.cu_k = torch.tensor(pr.cu_k)
        _check_decode_capacity(packed_inp, cap, sel, out, lse, pr)


def test_ring_local_heads_fill_and_advance():
    # local heads only, their KV groups stored as rings of 4 sinks + 256 window rows
    rtp = _rtp()
    cfg = scaled(DECODE_32K, name="ring", batch=3, seqlens=(1000 + 2, 100 + 2, 5 + 2), n_q_heads=8, n_kv_heads=2,
                 ret_heads=(), window=256, needles="none")
    inp = make_inputs(cfg, DEV)
    cu = inp.cu_k.cpu().tolist()
    B, cap = 3, cfg.n_sink + cfg.window
    full_len = [cu[b + 1] - cu[b] for b in range(B)]
    k = torch.full((B * cap, 2, 128), float("nan"), dtype=inp.k.dtype, device=DEV)
    v = torch.full_like(k, float("nan"))
    for s in range(3):
        lens = [n - 2 + s for n in full_len]
        prob = _problem(inp, cap, lengths=lens, ring=True, ret_heads=())
        if s == 0:   # the prompt: every token at once (only sinks and the last window are kept)
            n_new = lens
        else:        # a decode step
            n_new = [1] * B
        rows = torch.cat([torch.arange(cu[b] + lens[b] - n_new[b], cu[b] + lens[b]) for b in range(B)]).to(DEV)
        cu_new = torch.tensor(np.concatenate([[0], np.cumsum(n_new)]), dtype=torch.int32, device=DEV)
        rtp.rtp_append_kv(prob, cu_new, int(sum(n_new)), inp.k[rows].contiguous(), inp.v[rows].contiguous(), k, v)
        _say(f"[case] ring step {s}: lengths {lens}")
        out = torch.full_like(inp.q, float("nan"))
        lse = torch.full((8, B), float("nan"), dtype=torch.float32, device=DEV)
        rtp.rtp_local_attn(prob, inp.q, k, v, out, lse)
        P.sync()
        pr = from_inputs(inp)
        pr.cu_k = list(np.concatenate([[0], np.cumsum(lens)]))
        keep = torch.cat([torch.arange(cu[b], cu[b] + lens[b]) for b in range(B)])
        pr.k, pr.v = inp.k[keep].cpu(), inp.v[keep].cpu()
        g = P.to_host(dict(out=out, lse=lse))
        n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(B)], list(range(8)), P.TOL[cfg.dtype],
                                       decode=True)
        _say(f"[result] ring step {s}: {n} pairs, {len(fails)} failures, {stats}")
        assert not fails, fails[:5]
