"""GPU parity on edge cases: ragged batches, tiny sequences, p = 1 and p -> 0, window 1,
window >= L, exact score ties (the fallback key spaces of both selections), v == 1,
and run-to-run determinism."""
import numpy as np
import pytest
import torch

from synth import DECODE_32K, PREFILL_128K, TINY_PREFILL, make_inputs, scaled
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _check_prefill(inp, rows=None):
    cfg = inp.cfg
    g = P.to_host(P.run_prefill(inp))
    pr = from_inputs(inp)
    assert P.check_index_keys(pr, g["k_idx"]) == 0
    if rows is None:
        rows = [(b, i) for b in range(cfg.batch) for i in range(inp.seqlens_q[b])]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g


def _check_decode(inp):
    cfg = inp.cfg
    pr = from_inputs(inp)
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(P.run_decode(inp, k_idx))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    return g


SMALL = dict(n_q_heads=8, n_kv_heads=2, ret_heads=(0, 5), window=64, needles="none")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_ragged_prefill_batch(dtype):
    cfg = scaled(TINY_PREFILL, name=f"ragged_prefill_{dtype}", batch=4, seqlens=(37, 300, 1, 1000),
                 dtype=dtype, **SMALL)
    _say(f"[case] {cfg.name}")
    _check_prefill(make_inputs(cfg, DEV))


def test_prefill_dense_limit_p1_window_ge_L():
    cfg = scaled(TINY_PREFILL, name="dense_limit", seqlen=700, top_p=1.0, window=4096)
    _say(f"[case] {cfg.name}")
    g = _check_prefill(make_inputs(cfg, DEV))
    assert np.all(g["tau"] == -np.inf)


def test_pages_prefill_retrieval_dense_bf16():
    # the pages' prefill: retrieval heads keep every key (top-p 1), local heads sinks + window
    cfg = scaled(PREFILL_128K, name="pages_prefill_p1", seqlen=1300, top_p=1.0, window=256)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    rows = [(0, i) for i in (0, 1, 17, 255, 256, 700, 1023, 1024, 1299)]
    g = P.to_host(P.run_prefill(inp))
    assert np.all(g["tau"] == -np.inf)
    pr = from_inputs(inp)
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


def test_dense_causal_baseline_all_heads():
    # every head dense causal: no retrieval heads, window covering the sequence, no sinks
    import long_context_sparse_rtp_amd as rtp
    cfg = scaled(PREFILL_128K, name="dense_all_heads", seqlen=1100, ret_heads=(), window=1100, n_sink=0,
                 needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    prob = rtp.Problem.from_inputs(inp)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=DEV)
    rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse)
    torch.cuda.synchronize()
    g = P.to_host(dict(out=out, lse=lse))
    pr = from_inputs(inp)
    rows = [(0, i) for i in (0, 1, 63, 64, 65, 511, 700, 1099)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


def test_prefill_argmax_limit_and_window_one():
    cfg = scaled(TINY_PREFILL, name="argmax_w1", seqlen=513, top_p=1e-7, window=1, n_sink=0)
    _say(f"[case] {cfg.name}")
    g = _check_prefill(make_inputs(cfg, DEV))
    assert np.all(g["count"] == 1)


def test_prefill_bf16_tiny_batch_sinks():
    cfg = scaled(PREFILL_128K, name="prefill_bf16_1k", seqlen=1027, window=100, n_sink=7)
    _say(f"[case] {cfg.name}")
    _check_prefill(make_inputs(cfg, DEV))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_exact_ties(dtype):
    cfg = scaled(TINY_PREFILL, name=f"ties_{dtype}", seqlen=1500, dtype=dtype, top_p=0.5)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    # three distinct pre-RoPE keys repeated: the indexer scores take only three values
    k3 = inp.k_pre[:3].clone()
    idx = torch.arange(inp.total_k, device=DEV) % 3
    inp.k_pre.copy_(k3[idx])
    _check_prefill(inp)


def test_decode_exact_ties_all_equal():
    cfg = scaled(DECODE_32K, name="decode_ties", batch=2, seqlen=5000, needles="none")
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    inp.k_pre.copy_(inp.k_pre[:1].expand_as(inp.k_pre))
    _check_decode(inp)


def test_decode_ragged_short_sequences():
    cfg = scaled(DECODE_32K, name="decode_ragged_short", batch=5, seqlens=(1, 3, 1024, 1030, 7000),
                 needles="query", needles_per_seq=8)
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV))


def test_decode_f32():
    # float32 decode: the split-list kernel for the local heads, float32 selection
    cfg = scaled(DECODE_32K, name="decode_f32", batch=3, seqlens=(700, 5000, 9000), dtype="f32",
                 n_q_heads=8, n_kv_heads=2, ret_heads=(0, 5), window=256, needles="query", needles_per_seq=8)
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV))


def test_decode_mqa_many_local_heads_per_group():
    # one KV group holding 20 local heads: the bfloat16 local kernel takes them as
    # tiles of 8, 8 and 4 heads that share every K/V row
    cfg = scaled(DECODE_32K, name="decode_mqa", batch=2, seqlens=(3000, 1100), n_q_heads=22, n_kv_heads=1,
                 ret_heads=(3, 17), window=512, needles="query", needles_per_seq=8)
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV))


def test_decode_groups_without_local_heads():
    # KV groups 0 and 2 hold only retrieval heads; groups 1 and 3 only local heads
    cfg = scaled(DECODE_32K, name="decode_mixed_groups", batch=2, seqlens=(2000, 4500), n_q_heads=8,
                 n_kv_heads=4, ret_heads=(0, 1, 4, 5), window=300, needles="none")
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV))


def test_decode_union_three_retrieval_heads_ragged():
    # KV group 0 holds retrieval heads 0, 1, 2 (their K/V rows are read once for the
    # union of the three LISTs), group 1 one retrieval head; ragged lengths down to 1
    cfg = scaled(DECODE_32K, name="decode_union3", batch=5, seqlens=(1, 63, 64, 65, 3000), n_q_heads=8,
                 n_kv_heads=2, ret_heads=(0, 1, 2, 5), window=96, needles="query", needles_per_seq=4)
    _say(f"[case] {cfg.name}")
    _check_decode(make_inputs(cfg, DEV))


def test_v_one_gives_one():
    cfg = scaled(PREFILL_128K, name="v_one", seqlen=800, window=64)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    inp.v.fill_(1.0)
    g = P.run_prefill(inp)
    # P enters the PV product rounded to bf16 while the row sum uses float32 weights,
    # so the bf16 path reproduces 1 to within the bf16 weight rounding
    assert float((g["out"].float() - 1.0).abs().max()) <= 4e-3


def test_selection_deterministic():
    cfg = scaled(PREFILL_128K, name="determinism", seqlen=3000, window=128)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    a = P.run_prefill(inp)
    b = P.run_prefill(inp)
    for k in ("tau", "tie", "count", "out"):
        assert torch.equal(a[k], b[k]), k
    dcfg = scaled(DECODE_32K, name="determinism_dec", batch=2, seqlen=9000)
    dinp = make_inputs(dcfg, DEV)
    import long_context_sparse_rtp_amd as rtp
    k_idx = rtp.rtp_index_keys(rtp.Problem.from_inputs(dinp), dinp.k_pre, dinp.w_k)
    a = P.run_decode(dinp, k_idx)
    b = P.run_decode(dinp, k_idx)
    for k in ("count", "out", "tau", "tie"):
        assert torch.equal(a[k], b[k]), k
    cu = dinp.cu_k.cpu().tolist()
    for r in range(dcfg.n_ret):
        for bb in range(dcfg.batch):
            c = int(a["count"][r, bb])
            assert torch.equal(a["idx"][r, cu[bb]:cu[bb] + c], b["idx"][r, cu[bb]:cu[bb] + c])
