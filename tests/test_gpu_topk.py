"""GPU parity of the fixed top-k selection (rtp_select_topk) against the oracle's
top-k, in both output forms, and of the attention calls fed with its sets.

Top-k is the static-budget variant the page compares dynamic top-p with
(k = 4096 there).  Sets must equal the oracle's except for keys whose float64
score lies within the float32 scoring error of the k-th score; count is exact."""
import numpy as np
import pytest
import torch

from synth import DECODE_32K, PREFILL_128K, TINY_PREFILL, make_inputs, sample_rows, scaled
from synth.gen import plant_blocks
from synth.configs import forced_edge_rows
from oracle.problem import from_inputs

from . import parity as P

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _say(msg):
    print(msg, flush=True)


def _prefill(cfg, top_k, rows=None, heads=None):
    _say(f"[case] top-k prefill {cfg.name} L={cfg.seqlens or cfg.seqlen} dtype={cfg.dtype} k={top_k}")
    inp = make_inputs(cfg, DEV)
    g = P.to_host(P.run_prefill(inp, top_k=top_k))
    pr = from_inputs(inp)
    pr.top_k = list(top_k)
    if rows is None:
        rows = [(b, i) for b in range(cfg.batch) for i in range(inp.seqlens_q[b])]
    heads = list(range(cfg.n_q_heads)) if heads is None else heads
    n, fails, stats = P.check_rows(pr, g, rows, heads, P.TOL[cfg.dtype])
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    # count is exactly min(k, pos + 1) on every row, checked or not
    for r in range(cfg.n_ret):
        for b in range(cfg.batch):
            q0, lq = int(inp.cu_q[b]), inp.seqlens_q[b]
            pos = np.arange(lq)
            assert np.array_equal(g["count"][r, q0:q0 + lq], np.minimum(max(top_k[b], 1), pos + 1))
    return g


def _decode(cfg, top_k):
    _say(f"[case] top-k decode {cfg.name} B={cfg.batch} k={top_k}")
    inp = make_inputs(cfg, DEV)
    pr = from_inputs(inp)
    pr.top_k = list(top_k)
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(P.run_decode(inp, k_idx, top_k=top_k))
    rows = [(b, 0) for b in range(cfg.batch)]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]
    for r in range(cfg.n_ret):
        for b in range(cfg.batch):
            assert int(g["count"][r, b]) == min(max(top_k[b], 1), inp.seqlens_k[b])
    return g


def test_topk_prefill_tiny_f32_all_rows():
    # rows 0..255 keep every key, later rows exactly 256
    _prefill(TINY_PREFILL, [256])


def test_topk_prefill_bf16_k4096_sampled():
    cfg = scaled(PREFILL_128K, name="topk_prefill_9k_bf16", seqlen=9000, window=512)
    rows = [(0, i) for i in sample_rows(cfg, 96, forced_edge_rows(cfg) + [4094, 4095, 4096, 4097])]
    _prefill(cfg, [4096], rows=rows)


def test_topk_prefill_ragged_batch_extremes():
    # k = 1 (the argmax), k < 1 (read as 1), a mid budget, and k beyond the length
    cfg = scaled(TINY_PREFILL, name="topk_ragged", batch=4, seqlens=(37, 300, 1, 1000), dtype="bf16",
                 n_q_heads=8, n_kv_heads=2, ret_heads=(0, 5), window=64, needles="none")
    _prefill(cfg, [1, 0, 5, 123])
    _prefill(cfg, [2000, 64, 1, 999])


def test_topk_prefill_exact_ties():
    # many identical index keys: the k-th score is shared by hundreds of keys, so the
    # tie key spaces (score bits, then positions) decide the set
    cfg = scaled(TINY_PREFILL, name="topk_ties", seqlen=1500, n_q_heads=2, n_kv_heads=1, ret_heads=(0,),
                 window=32, needles="none")
    inp = make_inputs(cfg, DEV)
    kp = inp.k_pre.view(-1, 128)
    kp[:] = kp[torch.arange(kp.shape[0], device=kp.device) % 7]   # seven distinct keys
    _say("[case] top-k prefill exact ties")
    g = P.to_host(P.run_prefill(inp, top_k=[300]))
    pr = from_inputs(inp)
    pr.top_k = [300]
    rows = [(0, i) for i in (0, 6, 7, 299, 300, 301, 700, 1024, 1499)]
    n, fails, stats = P.check_rows(pr, g, rows, [0, 1], P.TOL[cfg.dtype])
    _say(f"[result] topk ties: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


def test_topk_decode_k4096():
    _decode(scaled(DECODE_32K, name="topk_decode_16k_b2", batch=2, seqlen=16384), [4096, 4096])


def test_topk_decode_ragged_extremes():
    cfg = scaled(DECODE_32K, name="topk_ragged_decode", batch=6, seqlens=(4096, 5000, 300, 70000, 1, 9000),
                 needles="query", needles_per_seq=16)
    _decode(cfg, [4096, 1, 300, 4096, 4096, 0])


def test_topk_decode_union_of_group_heads():
    # two retrieval heads per KV group: the attention reads each group's rows once
    # for the union of the two top-k LISTs
    cfg = scaled(DECODE_32K, name="topk_union_decode", batch=3, seqlens=(5000, 300, 9000), n_q_heads=8,
                 n_kv_heads=2, ret_heads=(0, 1, 4, 7), window=128, needles="query", needles_per_seq=8)
    _decode(cfg, [1024, 4096, 700])


def test_topk_decode_exact_ties_all_equal():
    # every index key equal: the first k positions win
    cfg = scaled(DECODE_32K, name="topk_decode_ties", batch=2, seqlen=9000, needles="none")
    inp = make_inputs(cfg, DEV)
    pr = from_inputs(inp)
    pr.top_k = [4096, 5000]
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    k_idx[:] = k_idx[:, :1]
    pr.k_idx = k_idx.cpu()
    _say("[case] top-k decode all-equal keys")
    g = P.to_host(P.run_decode(inp, k_idx, top_k=pr.top_k))
    for r in range(cfg.n_ret):
        for b in range(cfg.batch):
            k0 = int(inp.cu_k[b])
            cnt = int(g["count"][r, b])
            assert cnt == pr.top_k[b]
            assert np.array_equal(g["idx"][r, k0:k0 + cnt], np.arange(cnt))
    n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(cfg.batch)], list(range(cfg.n_q_heads)),
                                   P.TOL[cfg.dtype], decode=True)
    assert not fails, fails[:5]


@pytest.mark.parametrize("kind", ["topk", "topp", "topk_ties"])
def test_clustered_selection_skips_tiles(kind):
    # selections that sit in a few 64-key blocks: the sparse attention path finds the
    # tiles that hold a selected pair from the index keys and skips every other tile.
    # "topk_ties" plants collinear keys (no jitter), so the index scores tie exactly in
    # bfloat16 and the threshold's tie position decides membership.
    cfg = scaled(PREFILL_128K, name=f"clustered_{kind}", seqlen=9000, window=256, needles="none",
                 top_p=0.5)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    plant_blocks(inp, blocks=(3, 20, 21, 77, 120), jitter=0.0 if kind == "topk_ties" else 0.25)
    top_k = None if kind == "topp" else [192]
    g = P.to_host(P.run_prefill(inp, top_k=top_k))
    pr = from_inputs(inp)
    if top_k is not None:
        pr.top_k = top_k
    rows = [(0, i) for i in sample_rows(cfg, 48, [0, 191, 192, 767, 768, 1343, 1344, 1345, 4999, 8999])]
    n, fails, stats = P.check_rows(pr, g, rows, list(range(cfg.n_q_heads)), P.TOL[cfg.dtype])
    ties = int((g["tie"] != 0x7FFFFFFF).sum())
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}, mean count "
         f"{float(g['count'].mean()):.1f}, rows with a tie position {ties}")
    assert not fails, fails[:5]
    if kind == "topk_ties":
        assert ties > 0


def test_clustered_topk_128k_sampled():
    # the 128K prefill with every row's highest index scores in the first 32 64-key blocks
    # and k = 2048: the k-th key sits in the thin lower tail of the planted scores, where
    # the sampled first sweep places the windowed sweep with wider bins
    cfg = PREFILL_128K
    _say("[case] clustered top-k 2048 at 128K")
    inp = make_inputs(cfg, DEV)
    plant_blocks(inp, blocks=list(range(32)))
    top_k = [2048]
    g = P.to_host(P.run_prefill(inp, top_k=top_k))
    pr = from_inputs(inp)
    pr.top_k = top_k
    rows = [(0, i) for i in sample_rows(cfg, 24, [2047, 2048, 2049, 4095, 4096, 65535, 131071])]
    n, fails, stats = P.check_rows(pr, g, rows, list(cfg.ret_heads), P.TOL[cfg.dtype], workers=P.n_workers())
    _say(f"[result] clustered top-k 128K: {n} pairs, {len(fails)} failures, {stats}")
    assert not fails, fails[:5]


@pytest.mark.parametrize("kind", ["topk", "topp"])
def test_clustered_decode_wide_score_range(kind):
    # planted keys (the first 32 64-key blocks of sequence 0) score tens of octaves of
    # softmax mass above the rest and spread over tens more, so a count target's k-th
    # key sits far below the row maximum: the units' 32-octave histograms clamp it into
    # their last bin and the crossing is resolved from the stored scores
    cfg = scaled(DECODE_32K, name=f"clustered_decode_{kind}", batch=2, seqlen=16384, needles="none", top_p=0.9)
    _say(f"[case] {cfg.name}")
    inp = make_inputs(cfg, DEV)
    plant_blocks(inp, blocks=list(range(32)))
    pr = from_inputs(inp)
    top_k = [2048, 2048] if kind == "topk" else None
    if top_k is not None:
        pr.top_k = top_k
    k_idx = P.oracle_index_keys(pr, inp.q.dtype, DEV)
    pr.k_idx = k_idx.cpu()
    g = P.to_host(P.run_decode(inp, k_idx, top_k=top_k))
    n, fails, stats = P.check_rows(pr, g, [(b, 0) for b in range(cfg.batch)], list(range(cfg.n_q_heads)),
                                   P.TOL[cfg.dtype], decode=True)
    _say(f"[result] {cfg.name}: {n} pairs, {len(fails)} failures, {stats}, counts "
         f"{[int(c) for c in np.asarray(g['count']).reshape(-1)]}")
    assert not fails, fails[:5]
    if top_k is not None:
        for r in range(cfg.n_ret):
            for b in range(cfg.batch):
                assert int(g["count"][r, b]) == 2048
