"""Benchmark of the sparse-attention hot path on one MI355X.

A step of the prefill workload (128K tokens, 32 query / 4 KV heads, bf16) is
one full pass of the path: index-key projection, THRESHOLD top-p selection and
sparse attention of the 4 retrieval heads on the main stream, sink+window
attention of the 28 local heads on a second stream beside them.  A step of the decode workload (batch 8 x 32K, index cache already
built) is LIST selection then sparse decode attention on the main stream, with local
decode attention on a second stream (overlapping them); both streams join at the
end of the step.
Inputs are seeded synthetic tensors resident in HBM before timing starts.

Prints one JSON line: ``value`` is prefill tokens/s; the decode step time, the
per-kernel times, the roofline of the dominant kernel and the CPU oracle
baseline ride along in the same line, and so do the same steps with the fixed top-k
selection (k = 4096, the pages' static-budget ablation) under ``topk_4096`` and the
decode step with the pages' block-granular top-p under ``topp_blocks64``.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "sparse-attn prefill tokens/s @128K and decode step µs @32K, 1 MI355X, % roofline"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
# v_exp_f32 issues at half the fp32 rate: 256 CUs x 4 SIMDs x 16 lanes x 2.4 GHz / 2
EXP_PEAK_TEXPS = 256 * 4 * 16 * 2.4e9 / 2 / 1e12
# kernel behind each timed call, its source, and the committed HBM counter summary
KERNELS = {
    "select_topp": ("rtp::select_prefill_kernel", "long_context_sparse_rtp_amd/csrc/select_prefill.hip",
                    "profiles/select_prefill_128k_traffic.txt"),
    "sparse_attn_prefill": ("rtp::attn_prefill_kernel<MODE 0>", "long_context_sparse_rtp_amd/csrc/attn_prefill.hip",
                            "profiles/attn_prefill_ret_128k_traffic.txt"),
    "local_attn": ("rtp::attn_prefill_kernel<MODE 1>", "long_context_sparse_rtp_amd/csrc/attn_prefill.hip",
                   "profiles/attn_prefill_local_128k_traffic.txt"),
}


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-references", action="store_true", help="skip the dense and pages'-prefill references")
    ap.add_argument("--no-variants", action="store_true", help="skip the fixed top-k (k = 4096) steps")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "decode", "both"], default="both")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only copy a 1 GiB buffer 4 times (a known-size kernel for HBM counter calibration)")
    return ap.parse_args()


class Timer:
    """HIP events on the stream the kernels run on."""

    def __init__(self, torch, stream):
        self.torch, self.stream = torch, stream
        self.acc = {}

    def run(self, name, fn):
        e0 = self.torch.cuda.Event(enable_timing=True)
        e1 = self.torch.cuda.Event(enable_timing=True)
        e0.record(self.stream)
        fn()
        e1.record(self.stream)
        self.acc.setdefault(name, []).append((e0, e1))

    def means_ms(self):
        return {k: sum(a.elapsed_time(b) for a, b in v) / len(v) for k, v in self.acc.items()}


def _traffic(name):
    """HBM bytes per launch from the committed counter summary, or None when the
    kernel's source changed since the counters were taken (or none were)."""
    import hashlib
    _, src, summ = KERNELS[name]
    try:
        kv = {}
        for ln in open(os.path.join(ROOT, summ)):
            if ":" in ln and not ln.startswith("#"):
                a, b = ln.split(":", 1)
                kv[a.strip()] = b.strip()
        sha = hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()
        if kv.get("kernel_source_sha256") != sha:
            return None
        return float(kv["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def _select_call(rtp, prob, inp, k_idx, mode, sel, ws, stream, top_k):
    if top_k is None:
        return lambda: rtp.rtp_select_topp(prob, inp.q_pre, inp.w, k_idx, inp.top_p, mode, sel, ws, stream=stream)
    return lambda: rtp.rtp_select_topk(prob, inp.q_pre, inp.w, k_idx, top_k, mode, sel, ws, stream=stream)


def bench_prefill(args, torch, rtp, synth, inp=None, top_k=None):
    """The prefill step; with ``top_k`` (int32 [batch]) the selection is the fixed top-k."""
    cfg = synth.PREFILL_128K
    dev = "cuda"
    if inp is None:
        inp = synth.make_inputs(cfg, dev)
    prob = rtp.Problem.from_inputs(inp)
    stream = torch.cuda.current_stream()
    k_idx = torch.empty((cfg.n_ret, inp.total_k, 16), dtype=inp.q.dtype, device=dev)
    sel = rtp.Selection.empty(prob, rtp.RTP_SEL_THRESHOLD, dev)
    ws_sel = torch.empty(max(16, rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SELECT, rtp.RTP_SEL_THRESHOLD)),
                         dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp.q)
    lse = torch.empty((cfg.n_q_heads, inp.total_q), dtype=torch.float32, device=dev)

    def step(t: Timer = None):
        calls = [
            ("index_keys", lambda: rtp.rtp_index_keys(prob, inp.k_pre, inp.w, k_idx, stream=stream)),
            ("select_topp" if top_k is None else "select_topk",
             _select_call(rtp, prob, inp, k_idx, rtp.RTP_SEL_THRESHOLD, sel, ws_sel, stream, top_k)),
            ("sparse_attn_prefill", lambda: rtp.rtp_sparse_attn_prefill(prob, inp.q, inp.k, inp.v, k_idx, sel,
                                                                        out, lse, stream=stream)),
            ("local_attn", lambda: rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, stream=stream)),
        ]
        if t is not None:   # per-kernel breakdown: everything in order on one stream
            for name, fn in calls:
                t.run(name, fn)
            return
        # the step: local heads (which read neither the index keys nor the selection, and
        # write other heads' rows of out and lse) on a second stream beside the rest
        fork = torch.cuda.Event()
        fork.record(stream)
        side.wait_event(fork)
        rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, stream=side)
        for _, fn in calls[:3]:
            fn()
        join = torch.cuda.Event()
        join.record(side)
        stream.wait_event(join)

    side = torch.cuda.Stream()   # default priority, like the main stream
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    # per-kernel times: a second pass with an event pair around every call on the launch stream
    t = Timer(torch, stream)
    for _ in range(args.steps):
        step(t)
    torch.cuda.synchronize()
    per = t.means_ms()

    # algorithmic work (sets measured from this run's selection)
    L, d, r = cfg.seqlen, 128, 16
    sum_S = float(sel.count.to(torch.float64).sum().item())
    causal_pairs = L * (L + 1) / 2
    n_local = cfg.n_q_heads - cfg.n_ret
    W, ns = cfg.window, cfg.n_sink
    i = torch.arange(L, dtype=torch.float64)
    local_keys = torch.minimum(i + 1, torch.full_like(i, W)) + torch.clamp(torch.minimum(i - W + 1, torch.full_like(i, ns)), min=0)
    sum_local = float(local_keys.sum().item()) * n_local
    flops = {
        "sparse_attn_prefill": 4 * d * sum_S,
        "local_attn": 4 * d * sum_local,
        "select_topp": 2 * r * causal_pairs * cfg.n_ret,
    }
    total_flops = sum(flops.values())
    exps_select = causal_pairs * cfg.n_ret    # one softmax-mass exponential per causal (row, key) pair
    bytes_ik = inp.total_k * cfg.n_ret * (d * 2 + r * 2)
    return dict(ms=ms, per_kernel_ms=per, flops=flops, total_flops=total_flops, sum_S=sum_S, exps_select=exps_select,
                mean_frac_selected=sum_S / (cfg.n_ret * causal_pairs), bytes_index_keys=bytes_ik,
                tokens=L, cfg=cfg, inp=inp, sel=sel)


def bench_prefill_references(args, torch, rtp, synth, pre):
    """Two references on the same 128K inputs:
    - dense: causal attention of all 32 heads (our attention kernel with no
      retrieval heads and a window covering the whole sequence), the baseline
      the pages' prefill speedups are quoted against;
    - pages_prefill: the pages' own prefill, where retrieval heads stay dense
      (top-p = 1, so the selection keeps every key) and local heads attend to
      sinks + window; the index cache is still built for the decode steps."""
    cfg, inp = pre["cfg"], pre["inp"]
    dev = "cuda"
    stream = torch.cuda.current_stream()
    L = cfg.seqlen
    dense = rtp.Problem(batch=cfg.batch, n_q_heads=cfg.n_q_heads, n_kv_heads=cfg.n_kv_heads, ret_heads=[],
                        n_sink=0, window=L, dtype=inp.q.dtype, cu_seqlens_q=inp.cu_q, cu_seqlens_k=inp.cu_k,
                        max_seqlen_q=L, max_seqlen_k=L, total_q=inp.total_q, total_k=inp.total_k)
    prob = rtp.Problem.from_inputs(inp)
    out = torch.empty_like(inp.q)
    lse = torch.empty((cfg.n_q_heads, inp.total_q), dtype=torch.float32, device=dev)
    k_idx = torch.empty((cfg.n_ret, inp.total_k, 16), dtype=inp.q.dtype, device=dev)
    sel = rtp.Selection.empty(prob, rtp.RTP_SEL_THRESHOLD, dev)
    ws_sel = torch.empty(max(16, rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SELECT, rtp.RTP_SEL_THRESHOLD)),
                         dtype=torch.uint8, device=dev)
    p_one = torch.ones_like(inp.top_p)

    def dense_step():
        rtp.rtp_local_attn(dense, inp.q, inp.k, inp.v, out, lse, stream=stream)

    def pages_step():
        rtp.rtp_index_keys(prob, inp.k_pre, inp.w, k_idx, stream=stream)
        rtp.rtp_select_topp(prob, inp.q_pre, inp.w, k_idx, p_one, rtp.RTP_SEL_THRESHOLD, sel, ws_sel, stream=stream)
        rtp.rtp_sparse_attn_prefill(prob, inp.q, inp.k, inp.v, k_idx, sel, out, lse, stream=stream)
        rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, stream=stream)

    def timed(fn, n):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(n):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    n = max(1, min(args.steps, 3))
    dense_ms = timed(dense_step, n)
    pages_ms = timed(pages_step, n)
    dense_flop = 4 * 128 * cfg.n_q_heads * L * (L + 1) / 2
    return dict(dense_ms=dense_ms, pages_ms=pages_ms, dense_tflops=dense_flop / (dense_ms * 1e-3) / 1e12)


def bench_decode(args, torch, rtp, synth, inp=None, top_k=None, blocks=False):
    """The decode step; with ``top_k`` (int32 [batch]) the selection is the fixed top-k,
    with ``blocks`` the pages' block-granular top-p."""
    cfg = synth.DECODE_32K
    dev = "cuda"
    if inp is None:
        inp = synth.make_inputs(cfg, dev)
    prob = rtp.Problem.from_inputs(inp)
    stream = torch.cuda.current_stream()
    k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w, stream=stream)   # cache built before timing
    sel = rtp.Selection.empty(prob, rtp.RTP_SEL_LIST, dev)
    ws_sel = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SELECT_BLOCKS if blocks else rtp.RTP_CALL_SELECT,
                                                 rtp.RTP_SEL_LIST), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SPARSE_DECODE), dtype=torch.uint8, device=dev)
    ws_loc = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_LOCAL), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp.q)
    lse = torch.empty((cfg.n_q_heads, inp.total_q), dtype=torch.float32, device=dev)

    side = torch.cuda.Stream()   # default priority, like the main stream

    def step(t: Timer = None):
        calls = [
            ("select_topp_blocks" if blocks else "select_topp" if top_k is None else "select_topk",
             (lambda: rtp.rtp_select_topp_blocks(prob, inp.q_pre, inp.w, k_idx, inp.top_p, sel, ws_sel,
                                                 stream=stream)) if blocks else
             _select_call(rtp, prob, inp, k_idx, rtp.RTP_SEL_LIST, sel, ws_sel, stream, top_k)),
            ("sparse_attn_decode", lambda: rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out, lse,
                                                                      ws_dec, stream=stream)),
            ("local_attn", lambda: rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, ws_loc, stream=stream)),
        ]
        if t is not None:   # per-kernel breakdown: everything in order on one stream
            for name, fn in calls:
                t.run(name, fn)
            return
        # the step: local heads on a second stream, overlapping selection + sparse attention
        fork = torch.cuda.Event()
        fork.record(stream)
        side.wait_event(fork)
        rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, ws_loc, stream=side)
        calls[0][1]()
        calls[1][1]()
        join = torch.cuda.Event()
        join.record(side)
        stream.wait_event(join)

    steps = args.decode_steps
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    t = Timer(torch, stream)
    for _ in range(steps):
        step(t)
    torch.cuda.synchronize()
    per = t.means_ms()

    counts = sel.count.to(torch.float64).cpu()
    B, L, W, ns = cfg.batch, cfg.seqlen, cfg.window, cfg.n_sink
    kv_row = 2 * 128 * 2            # K + V bytes per token per KV head
    sparse_bytes = float(counts.sum().item()) * kv_row
    local_keys = min(W, L) + min(ns, max(0, L - W))
    local_bytes = B * cfg.n_kv_heads * local_keys * kv_row   # each KV group's window once
    idx_bytes = cfg.n_ret * B * L * 16 * 2
    qo_bytes = B * cfg.n_q_heads * 128 * 2 * 2
    return dict(ms=ms, per_kernel_ms=per, bytes=dict(sparse_attn_decode=sparse_bytes, local_attn=local_bytes,
                                                     select_topp=idx_bytes, q_out=qo_bytes),
                total_bytes=sparse_bytes + local_bytes + idx_bytes + qo_bytes,
                mean_frac_selected=float(counts.mean().item()) / L, inp=inp)


def cpu_baseline(args, pre):
    """The oracle, untuned, on a bounded sample of the prefill workload's query rows."""
    import numpy as np
    import multiprocessing as mp
    from oracle.problem import from_inputs
    cfg, inp = pre["cfg"], pre["inp"]
    pr = from_inputs(inp)
    L = cfg.seqlen
    heads = list(range(cfg.n_q_heads))
    # warm the per-KV-head float64 caches before forking so workers share them
    for h in heads:
        pr._kv("k", 0, pr.kv_of(h))
        pr._kv("v", 0, pr.kv_of(h))
    for r in range(cfg.n_ret):
        pr.index_keys(0, r)
    rng = np.random.default_rng(0)
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count() or 1
    cores = max(1, min(cores, 16))
    global _PR
    _PR = pr
    t0 = time.time()
    done_rows, cost_rows = 0, 0.0
    with mp.get_context("fork").Pool(cores) as pool:
        while time.time() - t0 < args.cpu_seconds:
            rows = rng.integers(0, L, size=cores).tolist()
            res = pool.map(_cpu_row_all_heads, rows)
            done_rows += len(rows)
    wall = time.time() - t0
    # rows drawn uniformly over [0, L) so their mean cost is the mean over the prefill
    tok_s = done_rows / wall
    return dict(value=tok_s, unit="tokens/s", cores=cores, kind="oracle",
                sample=f"{done_rows} query rows drawn uniformly from the 128K prefill, all 32 heads each, "
                       f"float64 numpy, {cores} worker processes, {wall:.1f} s")


_PR = None


def _cpu_row_all_heads(i):
    pr = _PR
    for h in range(pr.n_q_heads):
        pr.row(0, int(i), h)
    return i


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    if args.calibrate_copy:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes_per_launch": 1 << 30, "launches": 4}))
        return
    import long_context_sparse_rtp_amd as rtp
    import synth
    rtp.library()  # fail loudly if the HIP library is missing
    print(f"[bench] device {torch.cuda.get_device_name(0)}", file=sys.stderr, flush=True)

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    pre = dec = None
    if args.only in ("prefill", "both"):
        print("[bench] prefill 128K ...", file=sys.stderr, flush=True)
        pre = bench_prefill(args, torch, rtp, synth)
        tok_s = pre["tokens"] / (pre["ms"] * 1e-3)
        per = pre["per_kernel_ms"]
        dom = max(("sparse_attn_prefill", "local_attn", "select_topp"), key=lambda k: per[k])
        fl = {k: pre["flops"][k] / (per[k] * 1e-3) / 1e12 for k in pre["flops"]}
        line.update(value=tok_s, unit="tokens/s", ms_per_step=pre["ms"])
        line["config"] = {"workload": "prefill_128k: L=131072 causal, 32 q / 4 kv heads, d=128, bf16, "
                                      "4 retrieval heads (top-p 0.9, 16-dim indexer), 28 local heads "
                                      "(window 2048 + 4 sinks)",
                          "global_batch": 1, "seq_len": pre["tokens"], "parallelism": "none (1 GPU)"}
        roofs = {}
        for k in ("select_topp", "sparse_attn_prefill", "local_attn"):
            rt = per[k] * 1e-3
            if k == "select_topp":   # bound by the exponential unit
                ach = pre["exps_select"] / rt / 1e12
                roofs[k] = {"kernel": KERNELS[k][0], "bound": "alu", "achieved": ach, "peak": EXP_PEAK_TEXPS,
                            "unit": "Texp/s", "frac": ach / EXP_PEAK_TEXPS, "traffic": _traffic(k)}
            else:
                ach = pre["flops"][k] / rt / 1e12
                roofs[k] = {"kernel": KERNELS[k][0], "bound": "mfma", "achieved": ach,
                            "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                            "traffic": _traffic(k)}
        line["roofline"] = roofs[dom]
        line["prefill"] = {"ms_per_step": pre["ms"], "per_kernel_ms": per,
                           "per_kernel_roofline": roofs,
                           "per_kernel_tflops": fl,
                           "algorithmic_tflop": pre["total_flops"] / 1e12,
                           "step_frac_of_mfma_roofline": (pre["total_flops"] / MFMA_BF16_PEAK_TFLOPS / 1e12 * 1e3)
                           / pre["ms"],
                           "mean_selected_fraction": pre["mean_frac_selected"]}
        if not args.no_references:
            print("[bench] prefill references (dense, pages' prefill) ...", file=sys.stderr, flush=True)
            ref = bench_prefill_references(args, torch, rtp, synth, pre)
            line["prefill"]["references"] = {
                "dense_causal_ms": ref["dense_ms"], "dense_causal_tflops": ref["dense_tflops"],
                "pages_prefill_ms": ref["pages_ms"],
                "speedup_vs_dense": ref["dense_ms"] / pre["ms"],
                "pages_prefill_speedup_vs_dense": ref["dense_ms"] / ref["pages_ms"],
                "note": "dense = all 32 heads causal on our attention kernel; pages_prefill = retrieval heads "
                        "dense (top-p 1) + local heads, as the pages run prefill"}
    if args.only in ("decode", "both"):
        print("[bench] decode 32K x 8 ...", file=sys.stderr, flush=True)
        dec = bench_decode(args, torch, rtp, synth)
        per = dec["per_kernel_ms"]
        line["decode"] = {"workload": "decode_32k_b8: batch 8, KV 32768, 32 q / 4 kv heads, bf16, "
                                      "4 retrieval heads (top-p 0.95), local window 1024 + 4 sinks",
                          "step_us": dec["ms"] * 1e3, "per_kernel_us": {k: v * 1e3 for k, v in per.items()},
                          "algorithmic_bytes": dec["total_bytes"],
                          "achieved_GBps": dec["total_bytes"] / (dec["ms"] * 1e-3) / 1e9,
                          "step_frac_of_hbm_roofline": dec["total_bytes"] / (HBM_PEAK_GBS * 1e9) / (dec["ms"] * 1e-3),
                          "mean_selected_fraction": dec["mean_frac_selected"]}
        if pre is None:
            line.update(value=dec["ms"] * 1e3, unit="us", higher_is_better=False, ms_per_step=dec["ms"])
    if not args.no_variants:
        # the pages' static-budget ablation: the same steps with the fixed top-k selection
        var = {"note": "fixed top-k, k = 4096 (the pages' top-k ablation) in place of top-p; same inputs"}
        if pre is not None:
            print("[bench] prefill 128K, top-k 4096 ...", file=sys.stderr, flush=True)
            kt = torch.full((pre["cfg"].batch,), 4096, dtype=torch.int32, device="cuda")
            pk = bench_prefill(args, torch, rtp, synth, inp=pre["inp"], top_k=kt)
            var["prefill_128k"] = {"ms_per_step": pk["ms"], "tokens_per_s": pk["tokens"] / (pk["ms"] * 1e-3),
                                   "per_kernel_ms": pk["per_kernel_ms"],
                                   "mean_selected_fraction": pk["mean_frac_selected"]}
        if dec is not None:
            print("[bench] decode 32K x 8, top-k 4096 ...", file=sys.stderr, flush=True)
            kt = torch.full((synth.DECODE_32K.batch,), 4096, dtype=torch.int32, device="cuda")
            dk = bench_decode(args, torch, rtp, synth, inp=dec["inp"], top_k=kt)
            var["decode_32k_b8"] = {"step_us": dk["ms"] * 1e3,
                                    "per_kernel_us": {k: v * 1e3 for k, v in dk["per_kernel_ms"].items()},
                                    "algorithmic_bytes": dk["total_bytes"],
                                    "step_frac_of_hbm_roofline": dk["total_bytes"] / (HBM_PEAK_GBS * 1e9)
                                    / (dk["ms"] * 1e-3),
                                    "mean_selected_fraction": dk["mean_frac_selected"]}
        line["topk_4096"] = var
        if dec is not None:
            print("[bench] decode 32K x 8, block top-p ...", file=sys.stderr, flush=True)
            db = bench_decode(args, torch, rtp, synth, inp=dec["inp"], blocks=True)
            line["topp_blocks64"] = {
                "note": "the pages' block-granular top-p (64-token blocks, 256-bin histogram of block masses "
                        "over block maxima) in place of the token-exact selection; same inputs and p",
                "decode_32k_b8": {"step_us": db["ms"] * 1e3,
                                  "per_kernel_us": {k: v * 1e3 for k, v in db["per_kernel_ms"].items()},
                                  "algorithmic_bytes": db["total_bytes"],
                                  "step_frac_of_hbm_roofline": db["total_bytes"] / (HBM_PEAK_GBS * 1e9)
                                  / (db["ms"] * 1e-3),
                                  "mean_selected_fraction": db["mean_frac_selected"],
                                  "token_exact_mean_selected_fraction": dec["mean_frac_selected"]}}
    if pre is not None and not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle) ...", file=sys.stderr, flush=True)
        line["cpu_baseline"] = cpu_baseline(args, pre)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
