"""CPU oracle for RTPurbo-style sparse attention.  TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this module.  The HIP library never calls it and
shares no code with it.

Everything here is plain numpy in float64, one query row at a time, written
from the method's definitions on the page "Full Attention Strikes Back:
Transferring Full Attention into Sparse within Hundred Training Steps"
(paper-graph-ui summary of arXiv 2605.16928), section 3.4:

* "Low-Dimensional Projection Mechanism and Stage-1 Training": pre-RoPE
  projections q_idx = W^Q q_pre, k_idx = W^K k_pre (r = 16, d_h = 128) and the
  indexer score s(m, n) = q_idx . k_idx (score-computation equation).  The
  workloads add the scale 1/sqrt(16); it is applied here as s / 4.
* "Dynamic Top-p Selection Mechanism" (Eq. 5 and the equation after it):
  softmax over the indexer scores of all cached keys, descending order, the
  smallest prefix whose cumulative mass reaches p; then exact softmax
  attention with post-RoPE q, k over the selected set only.
* Sections "Evaluation Methodology" and "Ablation Studies and Robustness
  Checks": the static top-k variant (k = 4096) the page measures top-p
  against - the same scores, a fixed number of keys.
* Section "Hardware-Aware Fast Top-p Decoding Kernel": the page's own
  block-granular approximation of top-p (64-token blocks, 256-bin histogram
  of block masses over block maxima), ``block_top_p``.
* "Local Head Attention Pattern": the first n_sink tokens plus a causal
  sliding window.

Readings of points the page leaves open:

* index precision: q_idx / k_idx are the float64 dot products rounded once,
  round-to-nearest-even, straight to the stored dtype (float32 or bfloat16);
* "reaches" means cumulative mass >= p; equal scores are ordered by ascending
  position; p >= 1 selects every candidate; the set is never empty;
* top-k keeps min(k, candidates) keys, equal scores by ascending position,
  and reads k < 1 as 1;
* candidates are the causal prefix including the query's own position;
  sinks and window are not added to the retrieval set;
* the window holds the W positions ending at and including the query
  (pos - W < n <= pos); sinks n < n_sink are added without double counting.

Pins (tests under ``tests/`` marked ``not gpu``): brute-force minimal subsets,
dense causal attention from torch's SDPA when p = 1 and W >= L, closed forms
(v == 1, window 1), exact rational rounding of the projection, the GQA union
example and the Table 6 sparsity values; top-k against a pairwise rank count,
the argmax and the top-p set of the same size; block top-p against a worked
example, the token-exact top-p it reduces to with one-token blocks and fine
bins, and a brute-force scan over the cut bin.  The composition of a whole
retrieval row at p < 1 (which query is projected, which matrix on which side,
which slot, which KV group) is pinned against a row written out from the
definition with exact rational arithmetic and subset enumeration, with
distinct q / q_pre, W^Q != W^K and a different pair per slot.  Every function
here has a pin; what stays "parity unpinned" is anything that would need the
pages' trained projections or their evaluation data, which this module does
not model.
"""
from __future__ import annotations

import dataclasses
from typing import Optional, Sequence

import numpy as np

HEAD_DIM = 128
IDX_DIM = 16
IDX_SCALE = 0.25          # 1 / sqrt(16)


# ---------------------------------------------------------------- rounding
def round_bf16(x) -> np.ndarray:
    """Round float64 values once, to nearest even, onto the bfloat16 grid.

    bfloat16 keeps 8 significant bits and float32's exponent range; the
    result is returned as float64 holding bfloat16-representable values.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # subnormal range keeps quantum 2**-133
    quantum = np.ldexp(1.0, e - 8)
    y = np.rint(x / quantum) * quantum       # x / quantum is exact; rint is half-to-even
    big = np.ldexp(2.0 - 2.0 ** -7, 127)
    y = np.where(np.abs(y) > big, np.copysign(np.inf, x), y)
    return np.where(x == 0, x, y)


def round_to(x, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# ---------------------------------------------------------------- indexer
def project(x_pre, w, dtype: str) -> np.ndarray:
    """Low-dimensional projection W x_pre of pre-RoPE vectors, rounded once to ``dtype``.

    x_pre: [..., 128]; w: [16, 128].  Returns [..., 16] float64 holding
    ``dtype`` values.
    """
    x = np.asarray(x_pre, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    return round_to(x @ w.T, dtype)


def indexer_scores(q_idx, k_idx) -> np.ndarray:
    """s_n = (q_idx . k_idx_n) / sqrt(16) for every key row of k_idx [n, 16].

    The 16 products are summed in a fixed order for every row, so equal index
    keys always get equal scores and exact ties are broken by position only.
    """
    k = np.asarray(k_idx, dtype=np.float64)
    q = np.asarray(q_idx, dtype=np.float64)
    acc = np.zeros(k.shape[0])
    for j in range(q.size):
        acc += k[:, j] * q[j]
    return acc * IDX_SCALE


@dataclasses.dataclass
class TopP:
    selected: np.ndarray     # ascending candidate indices of the active set
    count: int
    order: np.ndarray        # candidates by (score desc, index asc)
    prob: np.ndarray         # softmax mass of each candidate (by index)
    cum: np.ndarray          # inclusive cumulative mass of each candidate (by index)
    scores: np.ndarray       # the scores (by index)


def top_p(scores, p: float) -> TopP:
    """Dynamic top-p (Eq. 5): smallest descending-score prefix whose softmax mass reaches p."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    if n == 0:
        raise ValueError("no candidates")
    m = s.max()
    e = np.exp(s - m)
    prob = e / e.sum()
    order = np.lexsort((np.arange(n), -s))
    cum_sorted = np.cumsum(prob[order])
    if p >= 1.0:
        k = n
    else:
        k = int(np.searchsorted(cum_sorted, p, side="left")) + 1
        k = min(max(k, 1), n)
    cum = np.empty(n)
    cum[order] = cum_sorted
    return TopP(selected=np.sort(order[:k]), count=k, order=order, prob=prob, cum=cum, scores=s)


def top_k(scores, k: int) -> TopP:
    """Fixed top-k, the static-budget variant the page compares top-p against
    (section "Evaluation Methodology", baselines; section "Ablation Studies and
    Robustness Checks", static top-k vs. dynamic top-p, k = 4096).

    The k highest scores of the candidates, equal scores taken by ascending
    position; every candidate when there are at most k; k < 1 reads as 1 so
    that the set is never empty.  ``prob`` / ``cum`` are the softmax masses of
    the same scores, for reporting the mass a fixed budget keeps.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    if n == 0:
        raise ValueError("no candidates")
    kk = min(max(int(k), 1), n)
    order = np.lexsort((np.arange(n), -s))
    e = np.exp(s - s.max())
    prob = e / e.sum()
    cum = np.empty(n)
    cum[order] = np.cumsum(prob[order])
    return TopP(selected=np.sort(order[:kk]), count=kk, order=order, prob=prob, cum=cum, scores=s)


@dataclasses.dataclass
class BlockTopP:
    selected: np.ndarray     # ascending token positions of the kept blocks
    count: int
    blocks: np.ndarray       # kept block indices (ascending)
    j_star: int              # crossing bin
    block_max: np.ndarray    # m_b per block
    block_mass: np.ndarray   # sum over the block of exp(s - max s)
    pos: np.ndarray          # fractional bin coordinate of m_b: 256 (m_b - lo) / (hi - lo)
    bins: np.ndarray         # bin of each block
    lo: float
    hi: float
    Z: float


def block_top_p(scores, p: float, block: int = 64, nbins: int = 256) -> BlockTopP:
    """Block-granular top-p of the page's decode kernel (section "Hardware-Aware
    Fast Top-p Decoding Kernel", steps 1-5 of the sort-free histogram).

    1. positions are cut into blocks of ``block`` consecutive tokens (the last
       one may be short);
    2. each block keeps its maximum score m_b and its log-sum-exp; the mass it
       carries is exp(logsumexp_b - M) = sum over the block of exp(s - M), with
       M the row maximum (a common factor that cancels in the fractions);
    3. the range [min m_b, max m_b] of the row is cut into ``nbins`` equal bins
       and every block's mass goes to the bin of its m_b (the top value falls
       in the last bin; a row whose blocks all share one m_b uses the last bin);
    4. bins are scanned from the highest down, accumulating mass, to the first
       bin where the cumulative fraction reaches p (p >= 1: every block);
    5. every block in that bin or above is kept, whole.
    Readings: the histogram sums block masses (the page calls the deposited
    value the block's log-sum-exp; adding logs would not be a mass); the
    crossing bin is kept whole, since a bin cannot be split without ordering
    its blocks.
    """
    s = np.asarray(scores, dtype=np.float64)
    n = s.size
    if n == 0:
        raise ValueError("no candidates")
    nb = -(-n // block)
    M = s.max()
    m = np.array([s[b * block:(b + 1) * block].max() for b in range(nb)])
    mass = np.array([np.exp(s[b * block:(b + 1) * block] - M).sum() for b in range(nb)])
    lo, hi = float(m.min()), float(m.max())
    if hi > lo:
        pos = (m - lo) / (hi - lo) * nbins
        bins = np.minimum(np.floor(pos), nbins - 1).astype(np.int64)
    else:
        pos = np.full(nb, float(nbins))
        bins = np.full(nb, nbins - 1, dtype=np.int64)
    Z = float(mass.sum())
    if p >= 1.0:
        j_star = 0
    else:
        # the non-empty bins, highest first (empty bins add nothing to the scan)
        occupied, inv = np.unique(bins, return_inverse=True)
        hist = np.zeros(occupied.size)
        np.add.at(hist, inv, mass)
        cum = 0.0
        j_star = int(occupied[0])
        for j in range(occupied.size - 1, -1, -1):
            cum += hist[j]
            if cum >= p * Z:
                j_star = int(occupied[j])
                break
    kept = np.nonzero(bins >= j_star)[0]
    sel = np.concatenate([np.arange(b * block, min((b + 1) * block, n)) for b in kept])
    return BlockTopP(selected=sel, count=int(sel.size), blocks=kept, j_star=j_star, block_max=m, block_mass=mass,
                     pos=pos, bins=bins, lo=lo, hi=hi, Z=Z)


def near_threshold(t: TopP, p: float, tol: float = 1e-5) -> np.ndarray:
    """Mask of candidates whose cumulative mass lies within ``tol`` of the threshold p."""
    return (t.cum >= p - tol) & (t.cum - t.prob <= p + tol)


def set_ok(t: TopP, p: float, got: Sequence[int], tol: float = 1e-5):
    """Is ``got`` the oracle set up to near-threshold tokens?  Returns (ok, n_differing)."""
    n = t.scores.size
    g = np.zeros(n, dtype=bool)
    got = np.asarray(got, dtype=np.int64)
    if got.size and (got.min() < 0 or got.max() >= n or np.unique(got).size != got.size):
        return False, -1
    g[got] = True
    s = np.zeros(n, dtype=bool)
    s[t.selected] = True
    diff = g ^ s
    if p >= 1.0:
        return (not diff.any()), int(diff.sum())
    ok = bool(np.all(near_threshold(t, p, tol)[diff]))
    return ok, int(diff.sum())


# ---------------------------------------------------------------- attention
@dataclasses.dataclass
class Attn:
    out: np.ndarray          # [128]
    lse: float               # natural-log sum of exp of the scaled logits over the set
    weights: np.ndarray      # softmax weights over ``keys``
    keys: np.ndarray         # key indices attended (ascending)


def attend(q, K, V, keys) -> Attn:
    """Exact softmax attention of one query over the key rows ``keys`` (equation after Eq. 5)."""
    keys = np.asarray(keys, dtype=np.int64)
    q = np.asarray(q, dtype=np.float64)
    Kk = np.asarray(K[keys], dtype=np.float64)
    Vk = np.asarray(V[keys], dtype=np.float64)
    a = (Kk @ q) / np.sqrt(HEAD_DIM)
    m = a.max()
    e = np.exp(a - m)
    l = e.sum()
    w = e / l
    return Attn(out=w @ Vk, lse=float(m + np.log(l)), weights=w, keys=keys)


def local_keys(pos: int, window: int, n_sink: int) -> np.ndarray:
    """Key positions of a local head: sinks n < n_sink plus pos - window < n <= pos."""
    lo = max(0, pos - window + 1)
    win = np.arange(lo, pos + 1)
    sinks = np.arange(0, min(n_sink, pos + 1))
    return np.union1d(sinks, win)


@dataclasses.dataclass
class RowResult:
    attn: Attn
    topp: Optional[TopP] = None
    q_idx: Optional[np.ndarray] = None


def retrieval_row(q, q_pre, w_q, K, V, k_idx, pos: int, p: float, dtype: str,
                  keys: Optional[np.ndarray] = None, k: Optional[int] = None, blocks: bool = False) -> RowResult:
    """A retrieval head for one query: project, score the causal prefix, top-p, attend.

    ``k_idx`` holds the (already rounded) index keys of positions 0..pos.
    ``keys`` overrides the attended set (used to re-evaluate the output on a
    different valid set); the selection is still returned.  With ``k`` given
    the set is the fixed top-k instead of top-p; with ``blocks`` it is the
    page's block-granular top-p.
    """
    q_idx = project(q_pre, w_q, dtype)
    s = indexer_scores(q_idx, k_idx[: pos + 1])
    if blocks:
        t = block_top_p(s, p)
    else:
        t = top_p(s, p) if k is None else top_k(s, k)
    sel = t.selected if keys is None else np.asarray(keys, dtype=np.int64)
    return RowResult(attn=attend(q, K, V, sel), topp=t, q_idx=q_idx)


def local_row(q, K, V, pos: int, window: int, n_sink: int) -> RowResult:
    return RowResult(attn=attend(q, K, V, local_keys(pos, window, n_sink)))


# ---------------------------------------------------------------- metrics
def compute_sparsity(attended_per_head: Sequence[float], context_len: int) -> float:
    """Mean over query heads of 1 - attended / L (Table 6, compute sparsity)."""
    a = np.asarray(attended_per_head, dtype=np.float64)
    return float(np.mean(1.0 - a / context_len))


def kv_union(sets: Sequence[Sequence[int]]) -> np.ndarray:
    """Tokens a KV head must keep: the union of its query heads' sets (GQA memory sparsity)."""
    if not sets:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate([np.asarray(s, dtype=np.int64) for s in sets]))


def memory_sparsity(sets_per_kv_head: Sequence[Sequence[Sequence[int]]], context_len: int) -> float:
    """Mean over KV heads of 1 - |union of its query heads' sets| / L."""
    u = [kv_union(g).size for g in sets_per_kv_head]
    return float(np.mean(1.0 - np.asarray(u, dtype=np.float64) / context_len))
