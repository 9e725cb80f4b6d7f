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
    "sparse_attn_prefill": ("rtp::attn_prefill_kernel<MODE 0> + <MODE 2>", "long_context_sparse_rtp_amd/csrc/attn_prefill.hip",
                            "profiles/attn_prefill_ret_128k_traffic.txt"),
    "local_attn": ("rtp::attn_prefill_kernel<MODE 1>", "long_context_sparse_rtp_amd/csrc/attn_prefill.hip",
                   "profiles/attn_prefill_local_128k_traffic.txt"),
    "index_keys": ("rtp::index_keys_kernel", "long_context_sparse_rtp_amd/csrc/index_keys.hip",
                   "profiles/index_keys_128k_traffic.txt"),
    # decode calls (32K x 8): the traffic of a call sums its kernels
    "select_decode": ("rtp::sel_dec_*", "long_context_sparse_rtp_amd/csrc/select_decode.hip",
                      "profiles/select_decode_32k_traffic.txt"),
    "sparse_attn_decode": ("rtp::attn_decode_kernel<MODE 0> + combine",
                           "long_context_sparse_rtp_amd/csrc/attn_decode.hip",
                           "profiles/attn_decode_ret_32k_traffic.txt"),
    "local_attn_decode": ("rtp::group_decode<false> + combine", "long_context_sparse_rtp_amd/csrc/attn_decode.hip",
                          "profiles/attn_decode_local_32k_traffic.txt"),
}

# the kernels each timed call launches, as substrings of their names in a rocprofv3 trace
# (a call's counters and durations sum over its kernels)
CALL_KERNELS = {
    "select_topp": ["select_prefill_kernel<unsigned short, false>"],
    "sparse_attn_prefill": ["attn_prefill_kernel<unsigned short, 0>", "attn_prefill_kernel<unsigned short, 2>"],
    "local_attn": ["attn_prefill_kernel<unsigned short, 1>"],
    "index_keys": ["index_keys_kernel<unsigned short>"],
    "select_decode": ["sel_dec_score<unsigned short>", "sel_dec_finish"],
    "sparse_attn_decode": ["attn_decode_kernel<unsigned short, 0>", "attn_decode_combine<unsigned short, 0>"],
    "local_attn_decode": ["group_decode<false>", "group_decode_combine<false>"],
}
# the workload pass each call's counters come from
CALL_PASS = {"select_topp": "pre", "sparse_attn_prefill": "pre", "local_attn": "pre", "index_keys": "pre",
             "select_decode": "dec", "sparse_attn_decode": "dec", "local_attn_decode": "dec"}
# the rocprofv3 passes behind the summaries under profiles/ (run from the repo root after
# cd /tmp && export TMPDIR=/tmp; one counter set per pass), written under PROF_OUT
PROF_OUT = "prof_out"
_PRE_ARGS = "--only prefill --steps 1 --warmup 0 --no-cpu-baseline --no-references --no-variants --no-long"
_DEC_ARGS = ("--only decode --steps 1 --warmup 0 --decode-steps 2 --no-cpu-baseline --no-references --no-variants "
             "--no-ragged --no-cold --no-graph")
_MFMA_COUNTERS = ("SQ_WAVES SQ_BUSY_CYCLES SQ_WAVE_CYCLES SQ_VALU_MFMA_BUSY_CYCLES SQ_INSTS_VALU SQ_INSTS_MFMA "
                  "SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT GRBM_GUI_ACTIVE")
PMC_PASSES = {
    "cal_fetch": ("FETCH_SIZE", "--calibrate-copy"),
    "cal_write": ("WRITE_SIZE", "--calibrate-copy"),
    "pre_fetch": ("FETCH_SIZE", _PRE_ARGS),
    "pre_write": ("WRITE_SIZE", _PRE_ARGS),
    "dec_fetch": ("FETCH_SIZE", _DEC_ARGS),
    "dec_write": ("WRITE_SIZE", _DEC_ARGS),
    "pre_mfma": (_MFMA_COUNTERS, _PRE_ARGS),
}
# what the algorithmic bytes of each call are (for the summaries' headers)
ALGO_NOTE = {
    "select_topp": "q_pre 134.2 MB + k_idx 16.8 MB read once; q_idx, tau, tie_pos, count written",
    "sparse_attn_prefill": "q rows of 4 heads 134 MB + K,V of 4 KV groups 268 MB + k_idx/q_idx 34 MB read once; "
                           "out 134 MB written (each 256-row query block re-reads the causal K/V prefix, from L2 "
                           "or the Infinity Cache, which FETCH_SIZE also counts)",
    "local_attn": "q rows of 28 heads 940 MB + the K,V window prefix of 4 KV groups 268 MB read; out 940 MB written",
    "index_keys": "k_pre of 4 KV groups 134.2 MB read once; k_idx 16.8 MB written",
    "select_decode": "k_idx of 4 retrieval heads x 8 x 32K 33.5 MB read; scores 4.2 MB written and read back; "
                     "unit histograms and the lists written",
    "sparse_attn_decode": "K,V rows of each group's selected union (about 386 MB at top-p 0.95) read once",
    "local_attn_decode": "K,V rows of the 1028-key window + sinks of 8 sequences x 4 groups, 16.8 MB",
}
TRACE_ARGS = ("--steps 3 --warmup 1 --decode-steps 20 --no-cpu-baseline --no-references --no-variants --no-long "
              "--no-ragged --no-cold --no-graph")


def pmc_command(name):
    counters, bargs = PMC_PASSES[name]
    return (f"rocprofv3 --pmc {counters} -d {PROF_OUT}/{name} -o p --output-format csv -- "
            f"python3 bench.py {bargs}")


def trace_command():
    return (f"rocprofv3 --kernel-trace --stats -d {PROF_OUT}/ktrace -o kt --output-format csv -- "
            f"python3 bench.py {TRACE_ARGS}")


def _args():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-references", action="store_true", help="skip the dense and pages'-prefill references")
    ap.add_argument("--no-variants", action="store_true", help="skip the fixed top-k (k = 4096) steps")
    ap.add_argument("--no-long", action="store_true", help="skip the 1M prefill and the 32K..1M prefill curve")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged batch-64 decode")
    ap.add_argument("--no-cold", action="store_true", help="skip the cold-cache decode steps")
    ap.add_argument("--no-graph", dest="graph", action="store_false",
                    help="skip the decode step replayed from a HIP graph")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("DIR", "KERNEL"),
                    help="summarise a rocprofv3 --pmc output directory for one kernel (no GPU work)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--only", choices=["prefill", "decode", "both"], default="both")
    ap.add_argument("--pmc-commands", action="store_true",
                    help="print the rocprofv3 counter passes behind the summaries under profiles/, one per line")
    ap.add_argument("--traffic-summary", metavar="CALL",
                    help="print the HBM traffic summary of a timed call from the counter passes under prof_out/")
    ap.add_argument("--mfma-summary", metavar="CALL",
                    help="print the matrix-core summary of a prefill call from the pre_mfma counter pass")
    ap.add_argument("--trace-summary", action="store_true",
                    help="print the kernel table of the rocprofv3 kernel trace under prof_out/ktrace")
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


def local_key_total(L, window, n_sink):
    """Keys a local head attends over a causal prefill of L rows, summed over the rows.

    Row i keeps its last `window` positions (i - window, i] clipped at 0, and the first
    `n_sink` positions (the attention sinks) that lie before that window.
    """
    total = 0
    for i in range(min(L, window)):             # the window reaches back to position 0
        total += i + 1
    for i in range(window, L):                  # full window, plus the sinks before it
        total += window + min(i - window + 1, n_sink)
    return total


def decode_union_rows(torch, lens, cu, counts, idx, window, n_sink, groups):
    """K/V rows one decode step must read: per (sequence, KV group), the union of the
    group's retrieval LISTs, and of its window and sinks when the group holds local heads.

    `groups` lists, per KV group, (has_local_heads, retrieval slots of the group);
    `counts[r, b]` members of slot r in sequence b sit at idx[r, cu[b]:cu[b] + counts[r, b]].
    """
    rows = 0
    for has_local, slots in groups:
        for b, L in enumerate(lens):
            mark = torch.zeros(L, dtype=torch.bool, device=idx.device)
            if has_local:
                mark[max(0, L - window):] = True
                mark[:min(n_sink, L)] = True
            for r in slots:
                c = int(counts[r, b])
                mark[idx[r, cu[b]:cu[b] + c].long()] = True
            rows += int(mark.sum().item())
    return rows


def _select_call(rtp, prob, inp, k_idx, mode, sel, ws, stream, top_k):
    if top_k is None:
        return lambda: rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, mode, sel, ws, stream=stream)
    return lambda: rtp.rtp_select_topk(prob, inp.q_pre, inp.w_q, k_idx, top_k, mode, sel, ws, stream=stream)


def _timed_steps(torch, stream, step, steps, warmup):
    """Mean ms of ``steps`` consecutive steps (events on the launch stream) after ``warmup``."""
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / max(1, steps)


def bench_prefill(args, torch, rtp, synth, cfg=None, inp=None, top_k=None, steps=None, warmup=None):
    """The prefill step of ``cfg`` (default the 128K workload); with ``top_k`` (int32 [batch])
    the selection is the fixed top-k."""
    cfg = cfg or synth.PREFILL_128K
    steps = args.steps if steps is None else steps
    warmup = args.warmup if warmup is None else warmup
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
    side = torch.cuda.Stream()   # default priority, like the main stream

    def step(t: Timer = None):
        calls = [
            ("index_keys", lambda: rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k, k_idx, stream=stream)),
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

    ms = _timed_steps(torch, stream, step, steps, warmup)
    # per-kernel times: a second pass with an event pair around every call on the launch stream
    t = Timer(torch, stream)
    for _ in range(steps):
        step(t)
    torch.cuda.synchronize()
    per = t.means_ms()

    # algorithmic work (sets measured from this run's selection)
    L, d, r = cfg.seqlen, 128, 16
    sum_S = float(sel.count.to(torch.float64).sum().item())
    causal_pairs = L * (L + 1) / 2
    n_local = cfg.n_q_heads - cfg.n_ret
    sum_local = float(local_key_total(L, cfg.window, cfg.n_sink)) * n_local
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


def prefill_rooflines(pre, counters=True):
    """Per-kernel roofline objects of a prefill run, and the dominant kernel's name.
    ``counters``: the run is the workload the committed counter summaries were taken on
    (prefill_128k); on any other workload their traffic does not apply and is null."""
    tr = _traffic if counters else (lambda k: None)
    per = pre["per_kernel_ms"]
    roofs = {}
    for k in ("select_topp", "sparse_attn_prefill", "local_attn", "index_keys"):
        if k not in per:
            continue
        rt = per[k] * 1e-3
        if k == "select_topp":   # bound by the exponential unit
            ach = pre["exps_select"] / rt / 1e12
            roofs[k] = {"kernel": KERNELS[k][0], "bound": "alu", "achieved": ach, "peak": EXP_PEAK_TEXPS,
                        "unit": "Texp/s", "frac": ach / EXP_PEAK_TEXPS, "traffic": tr(k)}
        elif k == "index_keys":  # bound by HBM
            ach = pre["bytes_index_keys"] / rt / 1e9
            roofs[k] = {"kernel": KERNELS[k][0], "bound": "hbm", "achieved": ach, "peak": HBM_PEAK_GBS,
                        "unit": "GB/s", "frac": ach / HBM_PEAK_GBS, "traffic": tr(k)}
        else:
            ach = pre["flops"][k] / rt / 1e12
            roofs[k] = {"kernel": KERNELS[k][0], "bound": "mfma", "achieved": ach,
                        "peak": MFMA_BF16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": ach / MFMA_BF16_PEAK_TFLOPS,
                        "traffic": tr(k)}
    dom = max(("sparse_attn_prefill", "local_attn", "select_topp"), key=lambda k: per[k])
    return roofs, dom


def prefill_summary(pre, counters=True):
    roofs, dom = prefill_rooflines(pre, counters)
    per = pre["per_kernel_ms"]
    return {"ms_per_step": pre["ms"], "tokens_per_s": pre["tokens"] / (pre["ms"] * 1e-3),
            "per_kernel_ms": per, "per_kernel_roofline": roofs, "dominant_kernel": dom,
            "per_kernel_tflops": {k: pre["flops"][k] / (per[k] * 1e-3) / 1e12 for k in pre["flops"]},
            "algorithmic_tflop": pre["total_flops"] / 1e12,
            "step_frac_of_mfma_roofline": (pre["total_flops"] / MFMA_BF16_PEAK_TFLOPS / 1e12 * 1e3) / pre["ms"],
            "mean_selected_fraction": pre["mean_frac_selected"]}


def bench_prefill_references(args, torch, rtp, synth, cfg, inp, n=1, topp=False):
    """References on one prefill input:
    - dense: causal attention of all 32 heads (our attention kernel with no retrieval
      heads and a window covering the whole sequence), the baseline the pages' prefill
      speedups are quoted against;
    - pages_prefill: the pages' own prefill, where retrieval heads stay dense (top-p = 1,
      so the selection keeps every key) and local heads attend to sinks + window; the
      index cache is still built for the decode steps;
    - topp (optional): the top-p prefill step of this repository, all kernels in order."""
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

    def sparse_step(pvec):
        def f():
            rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k, k_idx, stream=stream)
            rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, pvec, rtp.RTP_SEL_THRESHOLD, sel, ws_sel,
                                stream=stream)
            rtp.rtp_sparse_attn_prefill(prob, inp.q, inp.k, inp.v, k_idx, sel, out, lse, stream=stream)
            rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, stream=stream)
        return f

    warm = 0 if L > (1 << 18) else 1    # the longest inputs: their first call is the measured one
    res = dict(dense_ms=_timed_steps(torch, stream, dense_step, n, warm),
               pages_ms=_timed_steps(torch, stream, sparse_step(p_one), n, warm))
    if topp:
        res["topp_ms"] = _timed_steps(torch, stream, sparse_step(inp.top_p), n, warm)
    dense_flop = 4 * 128 * cfg.n_q_heads * L * (L + 1) / 2
    res["dense_tflops"] = dense_flop / (res["dense_ms"] * 1e-3) / 1e12
    return res


def bench_decode(args, torch, rtp, synth, cfg=None, inp=None, top_k=None, blocks=False, cold=0, graph=False):
    """The decode step of ``cfg`` (default the 32K x 8 workload); with ``top_k`` (int32 [batch])
    the selection is the fixed top-k, with ``blocks`` the pages' block-granular top-p.
    ``cold`` > 0 also times that many single steps, each after a 512 MiB write that
    evicts the caches (L2 and the 256 MB Infinity Cache); ``graph`` also times the step
    captured in a HIP graph and replayed."""
    cfg = cfg or synth.DECODE_32K
    dev = "cuda"
    if inp is None:
        inp = synth.make_inputs(cfg, dev)
    prob = rtp.Problem.from_inputs(inp)
    stream = torch.cuda.current_stream()
    k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k, stream=stream)   # cache built before timing
    sel = rtp.Selection.empty(prob, rtp.RTP_SEL_LIST, dev)
    ws_sel = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SELECT_BLOCKS if blocks else rtp.RTP_CALL_SELECT,
                                                 rtp.RTP_SEL_LIST), dtype=torch.uint8, device=dev)
    ws_dec = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_SPARSE_DECODE), dtype=torch.uint8, device=dev)
    ws_loc = torch.empty(rtp.rtp_workspace_size(prob, rtp.RTP_CALL_LOCAL), dtype=torch.uint8, device=dev)
    out = torch.empty_like(inp.q)
    lse = torch.empty((cfg.n_q_heads, inp.total_q), dtype=torch.float32, device=dev)

    side = torch.cuda.Stream()   # default priority, like the main stream

    def step(t: Timer = None, main=None):
        m = stream if main is None else main
        calls = [
            ("select_topp_blocks" if blocks else "select_topp" if top_k is None else "select_topk",
             (lambda: rtp.rtp_select_topp_blocks(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, sel, ws_sel,
                                                 stream=m)) if blocks else
             _select_call(rtp, prob, inp, k_idx, rtp.RTP_SEL_LIST, sel, ws_sel, m, top_k)),
            ("sparse_attn_decode", lambda: rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out, lse,
                                                                      ws_dec, stream=m)),
            ("local_attn", lambda: rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, ws_loc, stream=m)),
        ]
        if t is not None:   # per-kernel breakdown: everything in order on one stream
            for name, fn in calls:
                t.run(name, fn)
            return
        # the step: local heads on a second stream, overlapping selection + sparse attention
        fork = torch.cuda.Event()
        fork.record(m)
        side.wait_event(fork)
        rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse, ws_loc, stream=side)
        calls[0][1]()
        calls[1][1]()
        join = torch.cuda.Event()
        join.record(side)
        m.wait_event(join)

    steps = args.decode_steps
    ms = _timed_steps(torch, stream, step, steps, args.warmup)
    # single steps, warm: median and min
    singles = []
    for _ in range(steps):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        step()
        e1.record(stream)
        singles.append((e0, e1))
    torch.cuda.synchronize()
    warm_us = sorted(a.elapsed_time(b) * 1e3 for a, b in singles)
    cold_us = None
    if cold:
        scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        pairs = []
        for it in range(cold):
            scrub.fill_(it & 0xFF)     # on the launch stream, before the step's first event
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        cold_us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
        del scrub
    # the same step captured once in a HIP graph and replayed (as a serving loop would):
    # kernel nodes only (the library records no memset); back-to-back replays and single ones
    graph_ms = graph_us = None
    if graph and args.graph:
        cap = torch.cuda.Stream()   # default priority; capture needs a stream other than the null one
        cap.wait_stream(stream)
        torch.cuda.synchronize()
        cg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(cg, stream=cap):
            step(main=cap)
        torch.cuda.synchronize()
        graph_ms = _timed_steps(torch, stream, cg.replay, steps, args.warmup)
        pairs = []
        for _ in range(steps):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            cg.replay()
            e1.record(stream)
            pairs.append((e0, e1))
        torch.cuda.synchronize()
        graph_us = sorted(a.elapsed_time(b) * 1e3 for a, b in pairs)
        del cg
    t = Timer(torch, stream)
    for _ in range(steps):
        step(t)
    torch.cuda.synchronize()
    per = t.means_ms()

    # algorithmic bytes: per (sequence, KV group) the rows of U = S of its retrieval heads
    # union window union sinks (K + V), the index keys of its retrieval heads, q and out
    kv_row = 2 * 128 * 2            # K + V bytes per token per KV head
    lens = inp.seqlens_k
    B = cfg.batch
    counts = sel.count.to(torch.int64).cpu()
    groups_with_local = {cfg.kv_of(h) for h in cfg.local_heads}
    groups = [(g in groups_with_local, [r for r, h in enumerate(cfg.ret_heads) if cfg.kv_of(h) == g])
              for g in range(cfg.n_kv_heads)]
    union_rows = decode_union_rows(torch, lens, inp.cu_k.tolist(), counts, sel.idx, cfg.window, cfg.n_sink,
                                   groups)
    kv_bytes = union_rows * kv_row
    idx_bytes = cfg.n_ret * sum(lens) * 16 * 2
    qo_bytes = B * cfg.n_q_heads * 128 * 2 * 2
    total = kv_bytes + idx_bytes + qo_bytes
    sum_sel = float(counts.sum().item())
    return dict(ms=ms, per_kernel_ms=per, warm_us=warm_us, cold_us=cold_us, graph_ms=graph_ms, graph_us=graph_us,
                bytes=dict(kv_union=kv_bytes, index_keys=idx_bytes, q_out=qo_bytes),
                total_bytes=total, union_rows=union_rows,
                mean_frac_selected=sum_sel / (cfg.n_ret * sum(lens)), inp=inp, cfg=cfg)


def decode_summary(dec, counters=True):
    d = {"step_us": dec["ms"] * 1e3, "per_kernel_us": {k: v * 1e3 for k, v in dec["per_kernel_ms"].items()},
         "single_step_us": {"median": _median(dec["warm_us"]), "min": dec["warm_us"][0]},
         "algorithmic_bytes": dec["total_bytes"], "bytes": dec["bytes"],
         "achieved_GBps": dec["total_bytes"] / (dec["ms"] * 1e-3) / 1e9,
         "step_frac_of_hbm_roofline": dec["total_bytes"] / (HBM_PEAK_GBS * 1e9) / (dec["ms"] * 1e-3),
         "mean_selected_fraction": dec["mean_frac_selected"]}
    if dec.get("graph_ms"):
        d["graph"] = {"note": "the same step captured once in a HIP graph and replayed (kernel nodes only)",
                      "step_us": dec["graph_ms"] * 1e3, "single_step_median_us": _median(dec["graph_us"]),
                      "step_frac_of_hbm_roofline": dec["total_bytes"] / (HBM_PEAK_GBS * 1e9) / (dec["graph_ms"] * 1e-3)}
    if dec["cold_us"]:
        c = dec["cold_us"]
        d["cold"] = {"note": "single steps, each after a 512 MiB write that evicts L2 and the Infinity Cache",
                     "median_us": _median(c), "min_us": c[0], "n": len(c),
                     "step_frac_of_hbm_roofline_median": dec["total_bytes"] / (HBM_PEAK_GBS * 1e9) / (_median(c) * 1e-6)}
    per = dec["per_kernel_ms"]
    sk = [k for k in per if k.startswith("select")][0]
    d["per_kernel_roofline"] = {
        sk: _hbm_roof("select_decode" if sk in ("select_topp", "select_topk") else sk, dec["bytes"]["index_keys"],
                      per[sk], counters),
        "sparse_attn_decode": _hbm_roof("sparse_attn_decode", None, per["sparse_attn_decode"], counters),
        "local_attn": _hbm_roof("local_attn_decode", None, per["local_attn"], counters)}
    return d


def _median(xs):
    xs = sorted(xs)
    n = len(xs)
    return 0.5 * (xs[(n - 1) // 2] + xs[n // 2]) if n else None


def _hbm_roof(name, algo_bytes, ms, counters=True):
    """HBM roofline object of a decode call: algorithmic bytes (when they split per call)
    over the call time, and the counter traffic of its kernels when committed for this
    workload (decode_32k_b8; ``counters`` False for any other)."""
    o = {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "time_us": ms * 1e3,
         "traffic": _traffic(name) if (counters and name in KERNELS) else None}
    if algo_bytes is not None:
        o["achieved"] = algo_bytes / (ms * 1e-3) / 1e9
        o["frac"] = o["achieved"] / HBM_PEAK_GBS
    if o["traffic"] is not None:
        o["traffic_GBps"] = o["traffic"] / (ms * 1e-3) / 1e9
    return o


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
    return dict(value=tok_s, unit="tokens/s", cores=cores, kind="oracle", cpu=_cpu_model(),
                sample=f"{done_rows} query rows drawn uniformly from the 128K prefill, all 32 heads each, "
                       f"float64 numpy, {cores} worker processes, {wall:.1f} s")


_PR = None


def _cpu_row_all_heads(i):
    pr = _PR
    for h in range(pr.n_q_heads):
        pr.row(0, int(i), h)
    return i


def _cpu_model():
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def pmc_summary(d, kernel_substr):
    """Sum of a rocprofv3 --pmc counter CSV over the dispatches of one kernel: prints the
    counter's mean per dispatch (the counter-summary files under profiles/ quote it)."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    vals = {}
    for f in files:
        for row in csv.DictReader(open(f)):
            if kernel_substr not in row.get("Kernel_Name", ""):
                continue
            key = (row.get("Dispatch_Id"), row["Counter_Name"])
            vals[key] = vals.get(key, 0.0) + float(row["Counter_Value"])
    per = {}
    for (disp, name), v in vals.items():
        per.setdefault(name, []).append(v)
    out = {name: {"mean_per_dispatch": sum(v) / len(v), "dispatches": len(v)} for name, v in per.items()}
    print(json.dumps({"kernel": kernel_substr, "files": len(files), "counters": out}))


def _pmc_rows(d):
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        rows.extend(csv.DictReader(open(f)))
    return rows


def _pmc_means(d, substrs):
    """{counter: (sum over the call's kernels of the mean per dispatch, dispatches of each kernel)}"""
    out = {}
    for sub in substrs:
        per = {}
        for row in _pmc_rows(d):
            if sub not in row.get("Kernel_Name", ""):
                continue
            key = (row["Dispatch_Id"], row["Counter_Name"])
            per[key] = per.get(key, 0.0) + float(row["Counter_Value"])
        by = {}
        for (disp, name), v in per.items():
            by.setdefault(name, []).append(v)
        for name, vs in by.items():
            tot, ns = out.get(name, (0.0, []))
            out[name] = (tot + sum(vs) / len(vs), ns + [len(vs)])
    return out


def _src_sha(call):
    import hashlib
    src = KERNELS[call][1]
    return src, hashlib.sha256(open(os.path.join(ROOT, src), "rb").read()).hexdigest()


def traffic_summary(call):
    """HBM bytes per launch of one timed call: FETCH_SIZE and WRITE_SIZE (KiB per dispatch,
    summed over the call's kernels), each scaled by what the same counter reads per
    dispatch for a device copy of 1 GiB."""
    base = os.path.join(ROOT, PROF_OUT)
    ps = CALL_PASS[call]
    cal_f = _pmc_means(os.path.join(base, "cal_fetch"), ["copyBuffer"])["FETCH_SIZE"][0]
    cal_w = _pmc_means(os.path.join(base, "cal_write"), ["copyBuffer"])["WRITE_SIZE"][0]
    fs = (1 << 30) / (cal_f * 1024.0)
    wsc = (1 << 30) / (cal_w * 1024.0)
    f, nf = _pmc_means(os.path.join(base, f"{ps}_fetch"), CALL_KERNELS[call])["FETCH_SIZE"]
    w, nw = _pmc_means(os.path.join(base, f"{ps}_write"), CALL_KERNELS[call])["WRITE_SIZE"]
    fb, wb = f * 1024.0 * fs, w * 1024.0 * wsc
    src, sha = _src_sha(call)
    lines = [f"# HBM traffic of the {call} call ({' + '.join(CALL_KERNELS[call])}), "
             f"{'prefill_128k' if ps == 'pre' else 'decode_32k_b8'} workload",
             "# commands (cd /tmp && export TMPDIR=/tmp; then from the repo root):"]
    for pn in ("cal_fetch", "cal_write", f"{ps}_fetch", f"{ps}_write"):
        lines.append("#   " + pmc_command(pn))
    lines += [f"#   python3 bench.py --traffic-summary {call}",
              f"# calibration: a 1 GiB device copy reads FETCH_SIZE {cal_f:.0f} KiB and WRITE_SIZE {cal_w:.0f} KiB "
              "per dispatch",
              f"# algorithmic: {ALGO_NOTE[call]}",
              f"fetch_size_kib_per_dispatch: {f:.1f}", f"write_size_kib_per_dispatch: {w:.1f}",
              f"fetch_scale: {fs:.4f}", f"write_scale: {wsc:.4f}",
              f"fetch_bytes_per_launch: {fb:.0f}", f"write_bytes_per_launch: {wb:.0f}",
              f"traffic_bytes_per_launch: {fb + wb:.0f}",
              f"dispatches_counted: {' + '.join(str(n) for n in nf)}",
              f"kernel_source: {src}", f"kernel_source_sha256: {sha}"]
    print("\n".join(lines))


def mfma_summary(call):
    """Matrix-core and instruction counters of a prefill call from the pre_mfma pass.
    GRBM_GUI_ACTIVE is summed over the 8 XCDs; busy fractions are per SIMD (1024)."""
    m = _pmc_means(os.path.join(ROOT, PROF_OUT, "pre_mfma"), CALL_KERNELS[call])
    g = m["GRBM_GUI_ACTIVE"][0]
    cyc = g / 8.0
    simd_cycles = cyc * 1024.0
    src, sha = _src_sha(call)
    lines = [f"# matrix-core counters of the {call} call ({' + '.join(CALL_KERNELS[call])}), prefill_128k",
             "# commands (cd /tmp && export TMPDIR=/tmp; then from the repo root):",
             "#   " + pmc_command("pre_mfma"), f"#   python3 bench.py --mfma-summary {call}",
             "# GRBM_GUI_ACTIVE sums the 8 XCDs' busy cycles; per-SIMD fractions divide by 1024 SIMDs x cycles"]
    for k in sorted(m):
        lines.append(f"{k.lower()}_per_launch: {m[k][0]:.0f}")
    lines.append(f"kernel_cycles_2p4GHz: {cyc:.0f}")
    lines.append(f"kernel_ms_from_cycles: {cyc / 2.4e6:.3f}")
    lines.append(f"mfma_busy_frac: {m['SQ_VALU_MFMA_BUSY_CYCLES'][0] / simd_cycles:.4f}")
    if "SQ_INSTS_MFMA" in m and "SQ_INSTS_VALU" in m:
        lines.append(f"valu_insts_per_mfma_inst: {m['SQ_INSTS_VALU'][0] / max(m['SQ_INSTS_MFMA'][0], 1.0):.3f}")
    if call == "select_topp" and "SQ_INSTS_VALU" in m:
        # one wave instruction covers a 16-key x 16-row tile of (row, key) pairs (4 per lane)
        L, R = 131072, 4
        tiles = R * L * (L + 1) / 2 / 256
        lines.append(f"causal_pair_tiles_per_launch: {tiles:.0f}")
        lines.append(f"valu_insts_per_pair_tile_all_sweeps: {m['SQ_INSTS_VALU'][0] / tiles:.2f}")
        lines.append(f"lds_insts_per_pair_tile_all_sweeps: {m['SQ_INSTS_LDS'][0] / tiles:.2f}")
    lines.append(f"kernel_source: {src}")
    lines.append(f"kernel_source_sha256: {sha}")
    print("\n".join(lines))


def trace_summary():
    """Per-kernel table of the rtp:: kernels in the kernel trace: launches, mean, min and
    max duration (us), and the resources of the code object."""
    import csv
    import glob
    rows = []
    for f in glob.glob(os.path.join(ROOT, PROF_OUT, "ktrace", "**", "*kernel_trace.csv"), recursive=True):
        rows.extend(csv.DictReader(open(f)))
    agg = {}
    order = []
    for r in sorted(rows, key=lambda r: int(r["Start_Timestamp"])):
        name = r["Kernel_Name"]
        if "rtp::" not in name:
            continue
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        key = (short, f'{r["Grid_Size_X"]}x{r["Grid_Size_Y"]}', r["Workgroup_Size_X"])
        if key not in agg:
            agg[key] = {"d": [], "vgpr": r["VGPR_Count"], "agpr": r["Accum_VGPR_Count"], "lds": r["LDS_Block_Size"],
                        "scr": r["Scratch_Size"]}
            order.append(key)
        agg[key]["d"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"# every rtp:: kernel of the traced run, in order of first launch (durations in us)")
    print("# commands (cd /tmp && export TMPDIR=/tmp; then from the repo root):")
    print("#   " + trace_command())
    print("#   python3 bench.py --trace-summary")
    print(f"{'kernel':62s} {'grid':>12s} {'wg':>4s} {'calls':>5s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s} "
          f"{'vgpr':>4s} {'agpr':>4s} {'lds':>6s} {'scr':>4s}")
    for key in order:
        a = agg[key]
        d = a["d"]
        print(f"{key[0][:62]:62s} {key[1]:>12s} {key[2]:>4s} {len(d):5d} {sum(d) / len(d):10.1f} {min(d):10.1f} "
              f"{max(d):10.1f} {a['vgpr']:>4s} {a['agpr']:>4s} {a['lds']:>6s} {a['scr']:>4s}")
    # the bench's per-kernel pass runs every call alone on one stream after the timed steps:
    # the last --steps launches of each prefill kernel and the last --decode-steps of each
    # decode kernel (the step itself overlaps the local heads on a second stream)
    ta = TRACE_ARGS.split()
    n_pre, n_dec = int(ta[ta.index("--steps") + 1]), int(ta[ta.index("--decode-steps") + 1])
    print()
    print(f"# the per-kernel pass alone (last {n_pre} launches of each prefill kernel, last {n_dec} of each decode "
          "kernel); the bench's per-call times are these sums")
    print(f"{'kernel':62s} {'grid':>12s} {'calls':>5s} {'avg_us':>10s} {'min_us':>10s} {'max_us':>10s}")
    for key in order:
        d = agg[key]["d"]
        dec = any(t in key[0] for t in ("sel_dec", "attn_decode", "group_decode"))
        n = n_dec if dec else n_pre
        if len(d) < n:
            continue
        d = d[-n:]
        print(f"{key[0][:62]:62s} {key[1]:>12s} {len(d):5d} {sum(d) / len(d):10.1f} {min(d):10.1f} {max(d):10.1f}")


def main():
    args = _args()
    if args.gpus != 1:
        print(json.dumps({"error": "runs on one GPU only: --gpus must be 1 (the library has no multi-GPU path)"}))
        sys.exit(2)
    if args.pmc_summary:
        pmc_summary(args.pmc_summary[0], args.pmc_summary[1])
        return
    if args.pmc_commands:
        print("\n".join(pmc_command(n) for n in PMC_PASSES))
        print(trace_command())
        return
    if args.traffic_summary:
        traffic_summary(args.traffic_summary)
        return
    if args.mfma_summary:
        mfma_summary(args.mfma_summary)
        return
    if args.trace_summary:
        trace_summary()
        return
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

    def say(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    line = {"metric": METRIC, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
            "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
            "data": "synthetic"}
    pre = dec = None
    if args.only in ("prefill", "both"):
        say("prefill 128K ...")
        pre = bench_prefill(args, torch, rtp, synth)
        summ = prefill_summary(pre)
        line.update(value=summ["tokens_per_s"], unit="tokens/s", ms_per_step=pre["ms"])
        line["config"] = {"workload": "prefill_128k: L=131072 causal, 32 q / 4 kv heads, d=128, bf16, "
                                      "4 retrieval heads (top-p 0.9, 16-dim indexer), 28 local heads "
                                      "(window 2048 + 4 sinks)",
                          "global_batch": 1, "seq_len": pre["tokens"], "parallelism": "none (1 GPU)"}
        line["roofline"] = summ["per_kernel_roofline"][summ["dominant_kernel"]]
        line["prefill"] = summ
        if not args.no_references:
            say("prefill references at 128K (dense, pages' prefill) ...")
            ref = bench_prefill_references(args, torch, rtp, synth, pre["cfg"], pre["inp"], n=max(1, min(args.steps, 3)))
            line["prefill"]["references"] = {
                "dense_causal_ms": ref["dense_ms"], "dense_causal_tflops": ref["dense_tflops"],
                "pages_prefill_ms": ref["pages_ms"],
                "speedup_vs_dense": ref["dense_ms"] / pre["ms"],
                "pages_prefill_speedup_vs_dense": ref["dense_ms"] / ref["pages_ms"],
                "note": "dense = all 32 heads causal on our attention kernel; pages_prefill = retrieval heads "
                        "dense (top-p 1) + local heads, as the pages run prefill"}
    if args.only in ("decode", "both"):
        say("decode 32K x 8 (warm, then cold) ...")
        dec = bench_decode(args, torch, rtp, synth, cold=0 if args.no_cold else 20, graph=True)
        line["decode"] = dict({"workload": "decode_32k_b8: batch 8, KV 32768, 32 q / 4 kv heads, bf16, "
                                           "4 retrieval heads (top-p 0.95), local window 1024 + 4 sinks"},
                              **decode_summary(dec))
        if pre is None:
            line.update(value=dec["ms"] * 1e3, unit="us", higher_is_better=False, ms_per_step=dec["ms"])
    if not args.no_variants:
        # the pages' static-budget ablation: the same steps with the fixed top-k selection
        var = {"note": "fixed top-k, k = 4096 (the pages' top-k ablation) in place of top-p; same inputs"}
        if pre is not None:
            say("prefill 128K, top-k 4096 ...")
            kt = torch.full((pre["cfg"].batch,), 4096, dtype=torch.int32, device="cuda")
            pk = bench_prefill(args, torch, rtp, synth, inp=pre["inp"], top_k=kt)
            var["prefill_128k"] = {"ms_per_step": pk["ms"], "tokens_per_s": pk["tokens"] / (pk["ms"] * 1e-3),
                                   "per_kernel_ms": pk["per_kernel_ms"],
                                   "mean_selected_fraction": pk["mean_frac_selected"]}
            del pk
            # clustered selections: the same step with every row's highest index scores in the
            # first 32 64-key blocks (a shared prefix) and k = 2048, so that rows past 8K keys keep
            # under a quarter of their prefix in 32 tiles (the sparse attention path skips the rest)
            say("prefill 128K, clustered top-k 2048 ...")
            import dataclasses
            cinp = dataclasses.replace(pre["inp"], q_pre=pre["inp"].q_pre.clone(), k_pre=pre["inp"].k_pre.clone())
            synth.gen.plant_blocks(cinp, blocks=list(range(32)))
            kt = torch.full((pre["cfg"].batch,), 2048, dtype=torch.int32, device="cuda")
            pc = bench_prefill(args, torch, rtp, synth, inp=cinp, top_k=kt)
            var["prefill_128k_clustered_k2048"] = {
                "ms_per_step": pc["ms"], "tokens_per_s": pc["tokens"] / (pc["ms"] * 1e-3),
                "per_kernel_ms": pc["per_kernel_ms"], "mean_selected_fraction": pc["mean_frac_selected"],
                "sparse_attn_tflops_on_selected_pairs": pc["flops"]["sparse_attn_prefill"]
                / (pc["per_kernel_ms"]["sparse_attn_prefill"] * 1e-3) / 1e12}
            del pc, cinp
        if dec is not None:
            say("decode 32K x 8, top-k 4096 ...")
            kt = torch.full((synth.DECODE_32K.batch,), 4096, dtype=torch.int32, device="cuda")
            dk = bench_decode(args, torch, rtp, synth, inp=dec["inp"], top_k=kt)
            var["decode_32k_b8"] = {k: v for k, v in decode_summary(dk).items() if k != "per_kernel_roofline"}
        line["topk_4096"] = var
        if dec is not None:
            say("decode 32K x 8, block top-p ...")
            db = bench_decode(args, torch, rtp, synth, inp=dec["inp"], blocks=True)
            line["topp_blocks64"] = {
                "note": "the pages' block-granular top-p (64-token blocks, 256-bin histogram of block masses "
                        "over block maxima) in place of the token-exact selection; same inputs and p",
                "decode_32k_b8": dict({k: v for k, v in decode_summary(db).items() if k != "per_kernel_roofline"},
                                      token_exact_mean_selected_fraction=dec["mean_frac_selected"])}
    if args.only in ("decode", "both") and not args.no_ragged:
        say("ragged decode, batch 64 ...")
        rd = bench_decode(args, torch, rtp, synth, cfg=synth.RAGGED_DECODE)
        line["ragged_decode"] = dict({"workload": "ragged_decode_b64: batch 64, KV lengths log-uniform in "
                                                  "[4096, 262144] (sum %d), 32 q / 4 kv heads, bf16, per-sequence "
                                                  "top-p in [0.8, 0.99], local window 1024 + 4 sinks, half the "
                                                  "sequences peaky (256 needles)" % sum(rd["inp"].seqlens_k)},
                                     **decode_summary(rd, counters=False))
        del rd
    if args.only in ("prefill", "both") and not args.no_long:
        say("prefill 1M ...")
        c4 = bench_prefill(args, torch, rtp, synth, cfg=synth.PREFILL_1M, steps=2, warmup=1)
        line["prefill_1m"] = dict({"workload": "prefill_1m: L=1048576 causal, 32 q / 4 kv heads, bf16, "
                                               "4 retrieval heads (top-p 0.9), 28 local heads (window 4096 + 4 sinks)"},
                                  **prefill_summary(c4, counters=False))
        line["prefill_1m"]["roofline"] = line["prefill_1m"]["per_kernel_roofline"][line["prefill_1m"]["dominant_kernel"]]
        if not args.no_references:
            # the shape of the pages' Fig. 1 (prefill speedup over dense attention against context
            # length) on this GPU: our dense causal kernel against the pages' prefill (retrieval
            # heads dense) and against this repository's top-p prefill, one call each
            say("prefill curve 32K .. 1M (dense, pages' prefill, top-p) ...")
            curve = []
            for L in (32768, 65536, 131072, 524288, 1048576):
                if L == 1048576:
                    cfg, inp = c4["cfg"], c4["inp"]
                elif L == 131072 and pre is not None:
                    cfg, inp = pre["cfg"], pre["inp"]
                else:
                    base = synth.PREFILL_1M if L > 131072 else synth.PREFILL_128K
                    cfg = synth.scaled(base, name=f"prefill_{L // 1024}k", seqlen=L)
                    inp = synth.make_inputs(cfg, "cuda")
                say(f"  curve L={L}")
                ref = bench_prefill_references(args, torch, rtp, synth, cfg, inp, n=1, topp=True)
                curve.append({"L": L, "window": cfg.window, "dense_ms": ref["dense_ms"],
                              "pages_prefill_ms": ref["pages_ms"], "topp_prefill_ms": ref["topp_ms"],
                              "pages_prefill_speedup": ref["dense_ms"] / ref["pages_ms"],
                              "topp_prefill_speedup": ref["dense_ms"] / ref["topp_ms"],
                              "dense_tflops": ref["dense_tflops"]})
                del inp
                torch.cuda.empty_cache()
            line["prefill_1m"]["references"] = {
                "curve": curve,
                "pages_published_speedup_vs_flashattention2": {"32K": 2.83, "64K": 4.25, "512K": 8.62, "1M": 9.36},
                "note": "dense = all 32 heads causal on our own attention kernel (the pages compare with "
                        "FlashAttention-2 on unstated hardware: context only); pages_prefill = retrieval heads "
                        "dense + local heads (sinks + window 2048 up to 128K, 4096 above); topp = this "
                        "repository's top-p 0.9 prefill step, kernels in order"}
        del c4
        torch.cuda.empty_cache()
    if pre is not None and not args.no_cpu_baseline:
        say("cpu baseline (oracle) ...")
        line["cpu_baseline"] = cpu_baseline(args, pre)
    print(json.dumps(line))


if __name__ == "__main__":
    main()
