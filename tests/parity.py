"""Helpers for the GPU parity tests: run the HIP path through the C ABI and compare
it with the CPU oracle row by row.  Imported by tests only."""
from __future__ import annotations

import itertools
import math
import os
import time
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np
import torch

from oracle import rtp_oracle as O
from oracle.problem import Problem, from_inputs

TOL = {"f32": 1e-4, "bf16": 2e-2}


def sync():
    torch.cuda.synchronize()


def _select(rtp, prob, inp, k_idx, mode, top_k):
    if top_k is None:
        return rtp.rtp_select_topp(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p, mode)
    kt = torch.as_tensor(list(top_k), dtype=torch.int32, device=inp.q.device)
    return rtp.rtp_select_topk(prob, inp.q_pre, inp.w_q, k_idx, kt, mode)


def run_prefill(inp, top_k: Optional[Sequence[int]] = None) -> Dict[str, torch.Tensor]:
    """Prefill path: index keys -> THRESHOLD select (top-p, or top-k per sequence when
    ``top_k`` is given) -> sparse attention + local attention."""
    import long_context_sparse_rtp_amd as rtp
    prob = rtp.Problem.from_inputs(inp)
    k_idx = rtp.rtp_index_keys(prob, inp.k_pre, inp.w_k)
    sel = _select(rtp, prob, inp, k_idx, rtp.RTP_SEL_THRESHOLD, top_k)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((inp.cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=inp.q.device)
    rtp.rtp_sparse_attn_prefill(prob, inp.q, inp.k, inp.v, k_idx, sel, out, lse)
    rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse)
    sync()
    return dict(k_idx=k_idx, q_idx=sel.q_idx, tau=sel.tau, tie=sel.tie_pos, count=sel.count, out=out, lse=lse)


def run_decode(inp, k_idx: torch.Tensor, top_k: Optional[Sequence[int]] = None) -> Dict[str, torch.Tensor]:
    """Decode path with a precomputed index cache: LIST select (top-p, or top-k) ->
    sparse decode + local decode."""
    import long_context_sparse_rtp_amd as rtp
    prob = rtp.Problem.from_inputs(inp)
    sel = _select(rtp, prob, inp, k_idx, rtp.RTP_SEL_LIST, top_k)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((inp.cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=inp.q.device)
    rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out, lse)
    rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse)
    sync()
    return dict(q_idx=sel.q_idx, idx=sel.idx, count=sel.count, tau=sel.tau, tie=sel.tie_pos, out=out, lse=lse)


def oracle_index_keys(pr: Problem, dtype: torch.dtype, device) -> torch.Tensor:
    """[R, T_k, 16] index cache computed by the oracle, stored in ``dtype`` (exactly representable)."""
    R = len(pr.ret_heads)
    Tk = pr.k.shape[0]
    out = torch.empty((R, Tk, 16), dtype=dtype)
    for r in range(R):
        g = pr.kv_of(pr.ret_heads[r])
        for c0 in range(0, Tk, 1 << 18):
            c1 = min(Tk, c0 + (1 << 18))
            x = pr.k_pre[c0:c1, g].to(torch.float64).numpy()
            out[r, c0:c1] = torch.from_numpy(O.project(x, pr.w("w_k", r), pr.dtype)).to(dtype)
    return out.to(device)


def to_host(d: Dict[str, torch.Tensor]) -> Dict[str, np.ndarray]:
    h = {}
    for k, v in d.items():
        if v is None:
            continue
        t = v.detach().cpu()
        h[k] = t.to(torch.float64).numpy() if t.is_floating_point() else t.numpy()
    return h


def near_midpoint(x: np.ndarray, dtype: str) -> np.ndarray:
    """Elements whose float64 value lies within 1e-12 (relative) of a rounding midpoint of ``dtype``."""
    bits = 8 if dtype == "bf16" else 24
    _, e = np.frexp(x)
    q = np.ldexp(1.0, e - bits)
    frac = x / q - np.floor(x / q)
    return np.abs(frac - 0.5) < 1e-12 * np.abs(x / q) + 1e-300


def check_index_keys(pr: Problem, gpu_kidx: np.ndarray, rows: Optional[np.ndarray] = None) -> int:
    """Bit-exact comparison with the oracle projection; returns the number of mismatches
    (mismatches at float64 rounding midpoints, where the float64 dot itself is ambiguous,
    are not counted)."""
    bad = 0
    Tk = pr.k.shape[0]
    rows = np.arange(Tk) if rows is None else rows
    for r, h in enumerate(pr.ret_heads):
        g = pr.kv_of(h)
        x = pr.k_pre[torch.as_tensor(rows), g].to(torch.float64).numpy()
        exact = x @ pr.w("w_k", r).T
        ref = O.round_to(exact, pr.dtype)
        got = gpu_kidx[r, rows]
        diff = got != ref
        if diff.any():
            diff &= ~near_midpoint(exact, pr.dtype)
        bad += int(diff.sum())
    return bad


def _amb_eps(q_idx: np.ndarray, k_idx: np.ndarray) -> np.ndarray:
    # bound on |float32 MFMA score - float64 score| (products are exact; 16 fp32 additions)
    return 2.0 ** -19 * (np.abs(k_idx) @ np.abs(q_idx)) * O.IDX_SCALE + 1e-30


def topk_set_ok(t: O.TopP, got, eps: np.ndarray):
    """Is ``got`` the oracle's top-k set, up to keys whose float64 score lies within the
    float32 scoring error of the k-th score (where the two precisions may order them
    differently)?  Returns (ok, n_differing)."""
    n = t.scores.size
    G = np.asarray(got, dtype=np.int64)
    if G.size != t.count or (G.size and (G.min() < 0 or G.max() >= n or np.unique(G).size != G.size)):
        return False, -1
    gm = np.zeros(n, dtype=bool)
    gm[G] = True
    sm = np.zeros(n, dtype=bool)
    sm[t.selected] = True
    diff = gm ^ sm
    if not diff.any():
        return True, 0
    kth = t.order[t.count - 1]
    ok = np.all(np.abs(t.scores[diff] - t.scores[kth]) <= eps[diff] + eps[kth])
    return bool(ok), int(diff.sum())


def _set_check(pr: Problem, b: int, t: O.TopP, eps: np.ndarray):
    """The set rule of the row: near-threshold mass for top-p, score ambiguity for top-k."""
    if pr.top_k is None:
        p = float(pr.top_p[b])
        return lambda G: O.set_ok(t, p, G)
    return lambda G: topk_set_ok(t, G, eps)


def _keeps_all(pr: Problem, b: int, pos: int) -> bool:
    if pr.top_k is None:
        return float(pr.top_p[b]) >= 1.0
    return int(pr.top_k[b]) >= pos + 1


def check_retrieval_row(pr: Problem, b: int, i: int, h: int, g: Dict[str, np.ndarray], tol: float):
    """Compare one retrieval-head row (THRESHOLD output).  Returns (ok, info)."""
    r = pr.slot_of(h)
    qi = int(pr.cu_q[b]) + i
    res = pr.row(b, i, h)
    info = {}
    if not np.array_equal(g["q_idx"][r, qi], res.q_idx):
        return False, {"why": "q_idx mismatch"}
    tau = g["tau"][r, qi]
    count = int(g["count"][r, qi])
    t = res.topp
    pos = pr.pos_of(b, i)
    tie = int(g["tie"][r, qi])
    INT_MAX = 2 ** 31 - 1
    eps = _amb_eps(res.q_idx, pr.index_keys(b, r)[: pos + 1])
    set_check = _set_check(pr, b, t, eps)
    if _keeps_all(pr, b, pos):
        G_list = [np.arange(pos + 1)]
    else:
        if not (0 <= tie <= pos or tie == INT_MAX):
            return False, {"why": f"tie_pos {tie} outside [0, {pos}]"}
        s = t.scores
        n = np.arange(s.size)
        if tie != INT_MAX:
            # the crossing token is at tie_pos; tokens with exactly its score are
            # admitted by position, as the threshold rule says
            same = s == s[tie]
        else:
            same = np.zeros(s.size, dtype=bool)
        sure = np.nonzero(((s > tau + eps) & ~same) | (same & (n <= tie)))[0]
        amb = np.nonzero((np.abs(s - tau) <= eps) & ~same)[0]
        k_amb = count - sure.size
        info.update(n_amb=int(amb.size))
        if k_amb < 0 or k_amb > amb.size:
            return False, {"why": f"count {count} inconsistent (sure {sure.size}, amb {amb.size})"}
        # tokens with equal float64 scores (equal index keys) share their float32 score,
        # so under {s >= tau} they are in or out together
        vals, inv = np.unique(s[amb], return_inverse=True)
        groups = [amb[inv == j] for j in range(vals.size)]
        sizes = [gg.size for gg in groups]
        combos = [c for kk in range(len(groups) + 1) for c in itertools.combinations(range(len(groups)), kk)
                  if sum(sizes[j] for j in c) == k_amb] if len(groups) <= 12 else None
        if combos is None or len(combos) > 256:
            return False, {"why": f"too many ambiguous tokens ({amb.size})"}
        G_list = [np.sort(np.concatenate([sure] + [groups[j] for j in c])).astype(np.int64) for c in combos]
    pr_k = pr._kv("k", b, pr.kv_of(h))
    pr_v = pr._kv("v", b, pr.kv_of(h))
    qv = pr.q_row(qi, h)
    best = None
    for G in G_list:
        ok_set, ndiff = set_check(G)
        if not ok_set:
            continue
        a = O.attend(qv, pr_k, pr_v, G)
        err = float(np.max(np.abs(g["out"][qi, h] - a.out)))
        lerr = abs(float(g["lse"][h, qi]) - a.lse)
        if err <= tol and lerr <= max(tol, 1e-4):
            return True, dict(info, err=err, lerr=lerr, ndiff=ndiff)
        best = (err, lerr) if best is None or err < best[0] else best
    return False, dict(info, why="no valid set matches", best=best, count=count, oracle_count=t.count)


def check_list_row(pr: Problem, b: int, h: int, g: Dict[str, np.ndarray], tol: float):
    """Compare one retrieval-head decode row (LIST output)."""
    r = pr.slot_of(h)
    qi = int(pr.cu_q[b])
    res = pr.row(b, 0, h)
    if not np.array_equal(g["q_idx"][r, qi], res.q_idx):
        return False, {"why": "q_idx mismatch"}
    k0, k1 = pr.seq_range_k(b)
    count = int(g["count"][r, qi])
    G = g["idx"][r, k0:k0 + count].astype(np.int64)
    if count < 1 or np.any(np.diff(G) <= 0) or G.min() < 0 or G.max() >= k1 - k0:
        return False, {"why": "list not ascending / out of range", "count": count}
    eps = _amb_eps(res.q_idx, pr.index_keys(b, r))
    ok_set, ndiff = _set_check(pr, b, res.topp, eps)(G)
    if not ok_set:
        return False, {"why": "set differs beyond near-threshold tokens", "count": count,
                       "oracle_count": res.topp.count, "ndiff": ndiff}
    a = O.attend(pr.q_row(qi, h), pr._kv("k", b, pr.kv_of(h)), pr._kv("v", b, pr.kv_of(h)), G)
    err = float(np.max(np.abs(g["out"][qi, h] - a.out)))
    lerr = abs(float(g["lse"][h, qi]) - a.lse)
    ok = err <= tol and lerr <= max(tol, 1e-4)
    return ok, dict(err=err, lerr=lerr, ndiff=ndiff, count=count)


def run_decode_blocks(inp, k_idx: torch.Tensor) -> Dict[str, torch.Tensor]:
    """Decode path with the pages' block-granular top-p: block LIST select -> sparse decode + local decode."""
    import long_context_sparse_rtp_amd as rtp
    prob = rtp.Problem.from_inputs(inp)
    sel = rtp.rtp_select_topp_blocks(prob, inp.q_pre, inp.w_q, k_idx, inp.top_p)
    out = torch.full_like(inp.q, float("nan"))
    lse = torch.full((inp.cfg.n_q_heads, inp.total_q), float("nan"), dtype=torch.float32, device=inp.q.device)
    rtp.rtp_sparse_attn_decode(prob, inp.q, inp.k, inp.v, sel, out, lse)
    rtp.rtp_local_attn(prob, inp.q, inp.k, inp.v, out, lse)
    sync()
    return dict(q_idx=sel.q_idx, idx=sel.idx, count=sel.count, tau=sel.tau, tie=sel.tie_pos, out=out, lse=lse)


def block_set_ok(bt: O.BlockTopP, p: float, got_blocks: np.ndarray, eps_max: float, tol: float = 1e-5):
    """Is ``got_blocks`` a valid block top-p set?  The kernel bins float32 block maxima
    in float32, so a block whose oracle bin coordinate lies within the scoring error of
    a bin edge may land on either side; the kept mass must reach p (within tol) and the
    blocks surely above the cut must not.  Returns (ok, n_blocks_differing)."""
    nb = bt.block_max.size
    gm = np.zeros(nb, dtype=bool)
    gm[got_blocks] = True
    sm = np.zeros(nb, dtype=bool)
    sm[bt.blocks] = True
    ndiff = int((gm ^ sm).sum())
    if p >= 1.0:
        return bool(gm.all()), ndiff
    if ndiff == 0:
        return True, 0
    span = bt.hi - bt.lo
    delta = (256.0 * 4.0 * eps_max / span if span > 0 else 0.0) + 1e-3
    mass = bt.block_mass
    if mass[gm].sum() < (p - tol) * bt.Z:
        return False, ndiff
    for j in range(256):
        certain = bt.pos - delta >= j
        possible = bt.pos + delta >= j
        if np.any(certain & ~gm) or np.any(gm & ~possible):
            continue
        above = bt.pos - delta >= j + 1
        if mass[above].sum() < (p + tol) * bt.Z:
            return True, ndiff
    return False, ndiff


def check_block_list_row(pr: Problem, b: int, h: int, g: Dict[str, np.ndarray], tol: float):
    """Compare one retrieval-head decode row under the block-granular top-p."""
    r = pr.slot_of(h)
    qi = int(pr.cu_q[b])
    res = pr.row(b, 0, h)
    if not np.array_equal(g["q_idx"][r, qi], res.q_idx):
        return False, {"why": "q_idx mismatch"}
    k0, k1 = pr.seq_range_k(b)
    L = k1 - k0
    count = int(g["count"][r, qi])
    G = g["idx"][r, k0:k0 + count].astype(np.int64)
    if count < 1 or np.any(np.diff(G) <= 0) or G.min() < 0 or G.max() >= L:
        return False, {"why": "list not ascending / out of range", "count": count}
    blocks = np.unique(G // 64)
    whole = np.concatenate([np.arange(64 * bb, min(64 * bb + 64, L)) for bb in blocks])
    if not np.array_equal(whole, G):
        return False, {"why": "list is not a union of whole 64-token blocks", "count": count}
    bt = res.topp
    eps = _amb_eps(res.q_idx, pr.index_keys(b, r))
    ok_set, ndiff = block_set_ok(bt, float(pr.top_p[b]), blocks, float(eps.max()))
    if not ok_set:
        return False, {"why": "block set invalid", "count": count, "oracle_count": bt.count, "ndiff": ndiff}
    a = O.attend(pr.q_row(qi, h), pr._kv("k", b, pr.kv_of(h)), pr._kv("v", b, pr.kv_of(h)), G)
    err = float(np.max(np.abs(g["out"][qi, h] - a.out)))
    lerr = abs(float(g["lse"][h, qi]) - a.lse)
    ok = err <= tol and lerr <= max(tol, 1e-4)
    return ok, dict(err=err, lerr=lerr, ndiff=ndiff, count=count)


def check_local_row(pr: Problem, b: int, i: int, h: int, g: Dict[str, np.ndarray], tol: float):
    qi = int(pr.cu_q[b]) + i
    a = pr.row(b, i, h).attn
    err = float(np.max(np.abs(g["out"][qi, h] - a.out)))
    lerr = abs(float(g["lse"][h, qi]) - a.lse)
    return err <= tol and lerr <= max(tol, 1e-4), dict(err=err, lerr=lerr)


def warm(pr: Problem, tasks) -> None:
    """Convert every slice the tasks need to float64 numpy now (before any fork)."""
    for (b, i, h) in tasks:
        g = pr.kv_of(h)
        pr._kv("k", b, g)
        pr._kv("v", b, g)
        qi = int(pr.cu_q[b]) + i
        pr.q_row(qi, h)
        r = pr.slot_of(h)
        if r >= 0:
            pr.index_keys(b, r)
            pr.w("w_q", r)
            pr.q_pre_row(qi, r)


def check_rows(pr: Problem, g: Dict[str, np.ndarray], rows: Sequence[Tuple[int, int]], heads: Sequence[int],
               tol: float, decode: bool = False, workers: int = 1):
    """Check every (row, head); returns (n_checked, failures list, stats)."""
    tasks = [(b, i, h) for (b, i) in rows for h in heads]
    warm(pr, tasks)
    results = _map(_check_task, [(pr, g, t, tol, decode) for t in tasks], workers)
    fails = [(t, info) for t, (ok, info) in zip(tasks, results) if not ok]
    errs = [info.get("err", 0.0) for ok, info in results if ok]
    ndiff = sum(info.get("ndiff", 0) or 0 for ok, info in results if ok)
    stats = dict(max_err=max(errs) if errs else 0.0, n=len(tasks), set_diffs=ndiff)
    return len(tasks), fails, stats


_SHARED = {}


def _check_task(args):
    pr, g, (b, i, h), tol, decode = args
    if pr.slot_of(h) >= 0:
        if decode and pr.blocks:
            return check_block_list_row(pr, b, h, g, tol)
        if decode:
            return check_list_row(pr, b, h, g, tol)
        return check_retrieval_row(pr, b, i, h, g, tol)
    return check_local_row(pr, b, i, h, g, tol)


def _worker_task(idx):
    args = _SHARED["args"][idx]
    return _check_task(args)


class _Progress:
    """A line every 30 s while the oracle works, so a long check is visibly alive."""

    def __init__(self, n):
        self.n, self.t0 = n, time.time()
        self.last = self.t0

    def tick(self, done):
        now = time.time()
        if now - self.last >= 30.0:
            print(f"[progress] oracle: {done}/{self.n} (row, head) pairs in {now - self.t0:.0f} s", flush=True)
            self.last = now


def _map(fn, arglist, workers):
    prog = _Progress(len(arglist))
    out = []
    if workers <= 1 or len(arglist) < 8:
        for a in arglist:
            out.append(fn(a))
            prog.tick(len(out))
        return out
    import multiprocessing as mp
    _SHARED["args"] = arglist
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        for r in pool.imap(_worker_task, range(len(arglist)), chunksize=max(1, len(arglist) // (16 * workers))):
            out.append(r)
            prog.tick(len(out))
    _SHARED.clear()
    return out


def n_workers() -> int:
    """Oracle worker processes: a few, so that the GPU process count stays small."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(8, n))
