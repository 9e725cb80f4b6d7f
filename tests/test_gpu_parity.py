"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on seeded inputs."""
import numpy as np
import pytest
import torch

from synth import DECODE_32K, PREFILL_128K, RAGGED_DECODE, TINY_PREFILL, make_inputs, sample_rows, scaled
from synth.configs import forced_edge_rows
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _prefill_case(cfg, rows=None, heads=None, workers=None):
    _say(f"[case] prefill {cfg.name} L={cfg.seqlen} dtype={cfg.dtype} p={cfg.top_p} W={cfg.window}")
    inp = make_inputs(cfg, DEV)
    g = P.to_host(P.run_prefill(inp))
    pr = from_inputs(inp)
    assert P.check_index_keys(pr, g["k_idx"]) == 0
    if rows is None:
        rows = [(0, i) for i in range(cfg.seqlen)]
    heads = list(range(cfg.n_q_heads)) if heads is None else heads
    n, fails, stats = P.check_rows(pr, g, rows, heads, P.TOL[cfg.dtype],
                                   workers=workers or 1)
    _say(f"[result] {cfg.name}: checked {n} (row, head) pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g, pr


def test_prefill_tiny_f32_all_rows():
    _prefill_case(TINY_PREFILL)


def test_prefill_small_bf16_sampled():
    cfg = scaled(PREFILL_128K, name="prefill_4k_bf16", seqlen=4096, window=512)
    rows = [(0, i) for i in sample_rows(cfg, 160, forced_edge_rows(cfg))]
    _prefill_case(cfg, rows=rows)


def _decode_case(cfg, workers=None):
    _say(f"[case] decode {cfg.name} B={cfg.batch} L={cfg.seqlen or (cfg.ragged_min, cfg.ragged_max)} "
         f"dtype={cfg.dtype} W={cfg.window}")
    inp = make_inputs(cfg, DEV)
    pr = from_inputs(inp)
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(P.run_decode(inp, k_idx))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True,
                                   workers=workers or 1)
    _say(f"[result] {cfg.name}: checked {n} (row, head) pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    # the emitted lists have exactly `count` entries and nothing else matters
    return g, pr


def test_decode_small():
    _decode_case(scaled(DECODE_32K, name="decode_4k_b2", batch=2, seqlen=4096))


def test_decode_32k_b8():
    _decode_case(DECODE_32K)


def test_index_keys_f32_and_bf16_exact():
    import long_context_sparse_rtp_amd as rtp
    for cfg in (TINY_PREFILL, scaled(PREFILL_128K, name="ik_bf16", seqlen=8192 + 37)):
        _say(f"[case] index keys {cfg.name}")
        inp = make_inputs(cfg, DEV)
        prob = rtp.Problem.from_inputs(inp)
        k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k)
        P.sync()
        pr = from_inputs(inp)
        assert P.check_index_keys(pr, P.to_host({"k": k_idx})["k"]) == 0
