"""GPU parity of the pages' block-granular top-p (rtp_select_topp_blocks) against the
oracle's ``block_top_p``, and of decode attention fed with its LIST.

The list must be a union of whole 64-token blocks; the block set may differ from the
oracle's only where a block maximum sits within the float32 scoring error of a bin
edge, and the kept mass must reach p while the blocks surely above the cut do not."""
import numpy as np
import pytest
import torch

from synth import DECODE_32K, make_inputs, scaled
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _blocks_case(inp, k_idx=None):
    cfg = inp.cfg
    pr = from_inputs(inp)
    pr.blocks = True
    if k_idx is None:
        k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(P.run_decode_blocks(inp, k_idx))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g, pr


def test_blocks_decode_small_ragged_tail():
    cfg = scaled(DECODE_32K, name="blocks_4k_b2", batch=2, seqlens=(4096 + 37, 9000))
    _say(f"[case] {cfg.name}")
    _blocks_case(make_inputs(cfg, DEV))


def test_blocks_decode_32k_b8():
    _say(f"[case] blocks {DECODE_32K.name}")
    g, pr = _blocks_case(make_inputs(DECODE_32K, DEV))
    frac = float(np.mean(g["count"])) / DECODE_32K.seqlen
    _say(f"[result] block top-p keeps {frac:.3f} of the keys")


def test_blocks_decode_short_sequences_and_p_one():
    cfg = scaled(DECODE_32K, name="blocks_short", batch=7, seqlens=(1, 3, 63, 64, 65, 1030, 70000),
                 needles="query", needles_per_seq=8)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    inp.top_p[5] = 1.0
    inp.top_p[6] = 0.3
    g, pr = _blocks_case(inp)
    k5 = int(inp.cu_k[5])
    for r in range(cfg.n_ret):
        assert int(g["count"][r, 5]) == 1030
        assert np.array_equal(g["idx"][r, k5:k5 + 1030], np.arange(1030))


def test_blocks_decode_equal_block_maxima_keep_everything():
    # all index keys equal: every block maximum is the same, so every block is kept
    cfg = scaled(DECODE_32K, name="blocks_equal", batch=2, seqlens=(5000, 300), needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    pr = from_inputs(inp)
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    k_idx[:] = k_idx[:, :1]
    g, pr = _blocks_case(inp, k_idx)
    for r in range(cfg.n_ret):
        for b, L in enumerate((5000, 300)):
            assert int(g["count"][r, b]) == L


def test_blocks_deterministic():
    cfg = scaled(DECODE_32K, name="blocks_det", batch=2, seqlen=9000)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    import long_context_sparse_rtp_amd as rtp
    k_idx = rtp.rtp_index_keys(rtp.Problem.from_inputs(inp), inp.k_pre, inp.w_k)
    a = P.run_decode_blocks(inp, k_idx)
    b = P.run_decode_blocks(inp, k_idx)
    for k in ("count", "out", "tau"):
        assert torch.equal(a[k], b[k]), k
