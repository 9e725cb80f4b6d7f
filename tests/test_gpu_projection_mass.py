"""GPU parity with distinct indexer projections per retrieval head, and on rows whose
softmax mass sits in one key far above a long tail.

* Distinct projections: every retrieval slot r has its own W^Q_r and W^K_r, and
  W^Q_r != W^K_r (section 3.4 "Low-Dimensional Projection Mechanism and Stage-1
  Training" of the page "Full Attention Strikes Back ...": the projections are
  per head and per side).  A path that projected with the wrong matrix, with
  slot 0's matrix for every slot, or the post-RoPE query, fails these.
* Peaky rows: one key about 18 score units above a tail of tens of thousands of
  keys, with the top-p crossing inside the tail (Eq. 5).  The tail's mass is a
  few 1e-5 of the total, so a fixed-point mass that loses a unit per key, or
  drops keys more than 31 octaves below a loose reference, moves the crossing by
  more than the 1e-5 set tolerance.
"""
import math

import numpy as np
import pytest
import torch

from synth import DECODE_32K, PREFILL_128K, TINY_PREFILL, make_inputs, sample_rows, scaled
from synth.configs import forced_edge_rows
from oracle import rtp_oracle as O
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _check_prefill(inp, rows, heads=None):
    cfg = inp.cfg
    g = P.to_host(P.run_prefill(inp))
    pr = from_inputs(inp)
    assert P.check_index_keys(pr, g["k_idx"]) == 0
    heads = list(range(cfg.n_q_heads)) if heads is None else heads
    n, fails, stats = P.check_rows(pr, g, rows, heads, P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g, pr


def _check_decode(inp, gpu_index_keys=False):
    import long_context_sparse_rtp_amd as rtp
    cfg = inp.cfg
    pr = from_inputs(inp)
    ref_kidx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    if gpu_index_keys:
        k_idx = rtp.rtp_index_keys(rtp.Problem.from_inputs(inp), inp.k_pre, inp.w_k)
        P.sync()
        assert torch.equal(k_idx, ref_kidx)
    else:
        k_idx = ref_kidx
    pr.k_idx = ref_kidx.cpu()
    g = P.to_host(P.run_decode(inp, k_idx))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g, pr


# ---------------------------------------------------------------- distinct projections
def test_distinct_projections_inputs():
    cfg = scaled(TINY_PREFILL, name="proj_check", seqlen=64, proj="distinct")
    inp = make_inputs(cfg, DEV)
    assert not torch.equal(inp.w_q, inp.w_k)
    assert not torch.equal(inp.w_q[0], inp.w_q[1]) and not torch.equal(inp.w_k[0], inp.w_k[1])


def test_prefill_distinct_projections_f32_all_rows():
    cfg = scaled(TINY_PREFILL, name="prefill_distinct_f32", seqlen=1100, proj="distinct")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    _check_prefill(inp, [(0, i) for i in range(cfg.seqlen)])


def test_prefill_distinct_projections_bf16_sampled():
    cfg = scaled(PREFILL_128K, name="prefill_distinct_bf16", seqlen=5000, window=512, proj="distinct")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    rows = [(0, i) for i in sample_rows(cfg, 96, forced_edge_rows(cfg))]
    _check_prefill(inp, rows)


def test_prefill_distinct_projections_ragged_batch():
    cfg = scaled(PREFILL_128K, name="prefill_distinct_ragged", batch=3, seqlens=(300, 1, 2500), n_q_heads=8,
                 n_kv_heads=2, ret_heads=(1, 4, 6), window=128, needles="none", proj="distinct")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    rows = [(0, i) for i in (0, 5, 127, 128, 299)] + [(1, 0)] + [(2, i) for i in (0, 900, 1777, 2499)]
    _check_prefill(inp, rows)


def test_decode_distinct_projections_gpu_index_keys():
    cfg = scaled(DECODE_32K, name="decode_distinct", batch=3, seqlens=(5000, 777, 12000), proj="distinct")
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV), gpu_index_keys=True)


def test_decode_distinct_projections_union_groups():
    # two retrieval heads in one KV group, each with its own projections
    cfg = scaled(DECODE_32K, name="decode_distinct_union", batch=2, seqlens=(3000, 6000), n_q_heads=8,
                 n_kv_heads=2, ret_heads=(0, 1, 5), window=128, needles="query", needles_per_seq=8,
                 proj="distinct")
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV), gpu_index_keys=True)


# ---------------------------------------------------------------- peaky rows
def _plant_peak(inp, rows_q, key_rows, groups, s_peak=18.0, gap_octaves=6.0, seed=5):
    """Give the query rows ``rows_q`` (every slot) one shared pre-RoPE direction u, and in
    every listed KV group put a key c u at key_rows[0] (score about s_peak for those queries)
    and a decoy at key_rows[1] whose projection is orthogonal to W u, with a norm that puts
    the Cauchy-Schwarz bound |q_idx| max|k_idx| / 4 about gap_octaves above the peak."""
    g = torch.Generator().manual_seed(seed)
    W = inp.w_q[0].double().cpu()                     # shared projection (W^Q = W^K)
    u = torch.randn(128, generator=g, dtype=torch.float64)
    u = u / u.norm() * math.sqrt(128.0)
    Wu = W @ u
    s1 = float(Wu @ Wu) / 4.0
    c = s_peak / s1
    v = torch.randn(128, generator=g, dtype=torch.float64)
    v = v - W.T @ ((W @ v) @ Wu / (Wu @ Wu) * Wu)    # W v orthogonal to W u (W W^T = I)
    top = s_peak + gap_octaves / math.log2(math.e)
    lam = top * 4.0 / (float(Wu.norm()) * float((W @ v).norm()))
    dt = inp.q_pre.dtype
    for r in range(inp.q_pre.shape[1]):
        inp.q_pre[rows_q, r] = u.to(dt).to(DEV)
    for gk in groups:
        inp.k_pre[key_rows[0], gk] = (c * u).to(dt).to(DEV)
        inp.k_pre[key_rows[1], gk] = (lam * v).to(dt).to(DEV)


def _narrow_truncation_error(s, top):
    """Relative mass error of 31-bit truncated masses 2^(31 - (top - s) log2 e) (a discriminating
    case needs this far above 1e-5)."""
    x = np.exp2(31.0 + (s - top) * math.log2(math.e))
    return float((x - np.floor(x)).sum() / x.sum())


def test_prefill_peaky_rows_wide_mass():
    L = 32768
    cfg = scaled(PREFILL_128K, name="prefill_peaky", seqlen=L, window=256, needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    rows = sorted(set(sample_rows(scaled(cfg, seqlen=L // 2), 10)))
    rows = [L // 2 + i for i in rows] + [L - 1]
    groups = sorted({cfg.kv_of(h) for h in cfg.ret_heads})
    _plant_peak(inp, torch.tensor(rows), (77, 78), groups)
    # p from the oracle's scores: the crossing sits inside the tail for every verified row
    pr = from_inputs(inp)
    tails, errs = [], []
    for i in rows:
        for r in range(cfg.n_ret):
            q_idx = O.project(pr.q_pre_row(i, r), pr.w("w_q", r), cfg.dtype)
            kx = pr.index_keys(0, r)
            s = O.indexer_scores(q_idx, kx[: i + 1])
            top = math.sqrt(float(q_idx @ q_idx) * float((kx * kx).sum(1).max())) / 4.0 * 1.0009765625
            e = np.exp(s - s.max())
            tails.append(1.0 - e.max() / e.sum())
            errs.append(_narrow_truncation_error(s, top))
    p = 1.0 - 0.5 * min(tails)
    _say(f"[case] tail mass {min(tails):.3e}..{max(tails):.3e}, p = {p:.8f}, "
         f"31-bit truncation error {min(errs):.2e}..{max(errs):.2e}")
    assert p - 1e-5 > 1.0 - min(tails)          # tail keys are surely in the set
    assert min(errs) > 5e-5                      # a 31-bit truncated mass would miss the tolerance
    inp.top_p.fill_(p)
    _check_prefill(inp, [(0, i) for i in rows], heads=list(cfg.ret_heads) + [1, 9])


def test_decode_peaky_rows():
    cfg = scaled(DECODE_32K, name="decode_peaky", batch=2, seqlen=32768, needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    cu = inp.cu_k.cpu().tolist()
    groups = sorted({cfg.kv_of(h) for h in cfg.ret_heads})
    for b in range(cfg.batch):
        _plant_peak(inp, torch.tensor([b]), (cu[b] + 1000 + 5 * b, cu[b] + 20000), groups)
    pr = from_inputs(inp)
    tails = []
    for b in range(cfg.batch):
        for r in range(cfg.n_ret):
            q_idx = O.project(pr.q_pre_row(b, r), pr.w("w_q", r), cfg.dtype)
            s = O.indexer_scores(q_idx, pr.index_keys(b, r))
            e = np.exp(s - s.max())
            tails.append(1.0 - e.max() / e.sum())
    p = 1.0 - 0.5 * min(tails)
    _say(f"[case] tail mass {min(tails):.3e}..{max(tails):.3e}, p = {p:.8f}")
    assert p - 1e-5 > 1.0 - min(tails)
    inp.top_p.fill_(p)
    _check_decode(inp)
