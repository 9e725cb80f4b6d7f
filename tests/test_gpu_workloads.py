"""GPU parity at the full workload sizes: 128K prefill (512 sampled rows, all heads),
1M prefill (256 sampled rows), ragged decode (every row).  The 32K decode and the tiny
prefill are checked in full in test_gpu_parity.py."""
import pytest

from synth import PREFILL_128K, PREFILL_1M, RAGGED_DECODE, make_inputs, sample_rows
from synth.configs import forced_edge_rows
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _sampled_prefill(cfg, n_rows):
    _say(f"[case] prefill {cfg.name} L={cfg.seqlen}: generating")
    inp = make_inputs(cfg, DEV)
    _say(f"[case] prefill {cfg.name}: running the HIP path")
    g = P.run_prefill(inp)
    # plus the rows where the selection's window bins change width (64K, 128K, 256K, 512K keys)
    widths = [r for b in (65536, 131072, 262144, 524288) for r in (b - 2, b - 1, b) if r < cfg.seqlen]
    rows = sample_rows(cfg, n_rows, forced_edge_rows(cfg) + widths)
    import torch
    ridx = torch.tensor(rows, device=DEV)
    # bring back only what the oracle compares
    gh = P.to_host({"q_idx": g["q_idx"], "tau": g["tau"], "count": g["count"], "tie": g["tie"],
                    "lse": g["lse"]})
    out_rows = g["out"][ridx].detach().cpu().to(torch.float64).numpy()
    import numpy as np
    full = np.zeros((cfg.seqlen, cfg.n_q_heads, 128))
    full[rows] = out_rows
    gh["out"] = full
    pr = from_inputs(inp)
    krows = np.array(sorted(set(rows) | set(range(0, cfg.seqlen, 997))))
    assert P.check_index_keys(pr, P.to_host({"k": g["k_idx"]})["k"], rows=krows) == 0
    _say(f"[case] prefill {cfg.name}: oracle on {len(rows)} rows x {cfg.n_q_heads} heads")
    n, fails, stats = P.check_rows(pr, gh, [(0, i) for i in rows], list(range(cfg.n_q_heads)),
                                   P.TOL[cfg.dtype], workers=P.n_workers())
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


def test_prefill_128k_sampled():
    _sampled_prefill(PREFILL_128K, 512)


def test_prefill_1m_sampled():
    _sampled_prefill(PREFILL_1M, 256)


def test_ragged_decode_b64_all_rows():
    cfg = RAGGED_DECODE
    _say(f"[case] decode {cfg.name}: generating")
    inp = make_inputs(cfg, DEV)
    pr = from_inputs(inp)
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    _say(f"[case] decode {cfg.name}: running the HIP path, lengths {min(inp.seqlens_k)}..{max(inp.seqlens_k)}")
    g = P.to_host(P.run_decode(inp, k_idx))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True,
                                   workers=P.n_workers())
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
