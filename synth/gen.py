"""Seeded synthetic inputs for the sparse-attention hot path.

This module draws random tensors and lays them out; it contains none of the
method's own arithmetic (no indexer projection, no selection, no attention).
Both the HIP path and the CPU oracle read the tensors it returns.

Recipe (all draws iid N(0, 1) in float64 unless stated, rounded once to the
workload dtype when stored):

* pre-RoPE q and k, and v, for every head;
* RoPE on q and k: consecutive dimension pairs (2i, 2i+1) rotated by angle
  pos * theta**(-2i/128), the rotary form written out in the paper-graph-ui
  summary of "Full Attention Strikes Back ..." (section 3.4, RoPE recap).
  Computed in float64 from the float64 pre-RoPE draw, then rounded;
* the indexer projection: one orthonormal 16x128 matrix (QR of a 128x16
  Gaussian with the signs fixed so diag(R) > 0), stored as float32 and used
  for every retrieval head, for q and for k; with ``proj = "distinct"`` every
  retrieval slot gets its own W^Q and W^K, each drawn the same way from a
  stream of its own;
* needles ("topic", prefill): per retrieval head a seeded unit direction t;
  floor(frac * L) key positions get k <- |k| (0.8 t + 0.6 u) with u the unit
  part of the original k orthogonal to t, and every query of that head is
  bent the same way, so the needles are relevant to all query blocks;
* needles ("query", decode): t is the direction of the decode query of the
  group's retrieval head and the planted keys get cosine 0.8 with it;
* ragged decode: lengths log-uniform in [lo, hi], per-sequence p uniform in
  the stated range, and each sequence carries needles with probability
  ``peaky_frac`` (flat otherwise).

Random numbers come from ``torch.Generator`` objects seeded from a 64-bit mix
of (seed, tensor tag, chunk index); large tensors are drawn in fixed
16384-row chunks so the result never depends on available memory.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import torch

from .configs import Config, log_uniform_lengths

CHUNK = 16384
_MASK = (1 << 64) - 1


def _mix(*xs: int) -> int:
    """splitmix64 fold of integers -> a seed in [0, 2**63)."""
    h = 0x9E3779B97F4A7C15
    for x in xs:
        h = (h + (int(x) & _MASK) + 0x9E3779B97F4A7C15) & _MASK
        z = h
        z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _MASK
        z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _MASK
        h = z ^ (z >> 31)
    return h & ((1 << 63) - 1)


def _gen(device, *tags) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(_mix(*tags))
    return g


_TAG = {"q": 1, "k": 2, "v": 3, "w": 4, "topic": 5, "npos": 6, "len": 7, "p": 8, "peaky": 9, "wq": 10, "wk": 11}


def _randn_chunk(seed: int, tag: str, chunk: int, shape, device) -> torch.Tensor:
    g = _gen(device, seed, _TAG[tag], chunk)
    return torch.randn(shape, generator=g, device=device, dtype=torch.float64)


def torch_dtype(name: str) -> torch.dtype:
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def rope_inplace(x: torch.Tensor, pos: torch.Tensor, theta: float) -> torch.Tensor:
    """Rotate consecutive pairs of the last dim of float64 ``x`` [n, H, d] by pos*theta^(-2i/d)."""
    d = x.shape[-1]
    i = torch.arange(d // 2, device=x.device, dtype=torch.float64)
    inv = theta ** (-(2.0 * i) / d)
    ang = pos.to(torch.float64)[:, None] * inv[None, :]
    c = torch.cos(ang)[:, None, :]
    s = torch.sin(ang)[:, None, :]
    xe = x[..., 0::2].clone()
    xo = x[..., 1::2].clone()
    x[..., 0::2] = xe * c - xo * s
    x[..., 1::2] = xe * s + xo * c
    return x


def orthonormal_projection(seed: int, r: int = 16, d: int = 128, tag: str = "w", index: int = 0) -> torch.Tensor:
    """A [r, d] float64 matrix with orthonormal rows (QR of a Gaussian, sign-fixed)."""
    g = _gen("cpu", seed, _TAG[tag], index)
    a = torch.randn((d, r), generator=g, dtype=torch.float64)
    qm, rm = torch.linalg.qr(a)
    sgn = torch.sign(torch.diagonal(rm))
    sgn[sgn == 0] = 1.0
    return (qm * sgn[None, :]).T.contiguous()


def _bend(x: torch.Tensor, t: torch.Tensor, cos: float) -> torch.Tensor:
    """Rows of x [n, d] -> |x| (cos t + sin u), u = unit part of x orthogonal to unit t.

    ``t`` is one unit direction [d] or one per row [n, d]."""
    if t.dim() == 1:
        t = t[None, :].expand_as(x)
    nrm = torch.linalg.vector_norm(x, dim=-1, keepdim=True)
    par = (x * t).sum(-1, keepdim=True) * t
    u = x - par
    u = u / torch.linalg.vector_norm(u, dim=-1, keepdim=True).clamp_min(1e-300)
    sin = math.sqrt(max(0.0, 1.0 - cos * cos))
    return nrm * (cos * t + sin * u)


@dataclasses.dataclass
class Inputs:
    cfg: Config
    q: torch.Tensor            # [T_q, Hq, 128] post-RoPE, dtype
    k: torch.Tensor            # [T_k, Hkv, 128] post-RoPE, dtype
    v: torch.Tensor            # [T_k, Hkv, 128] dtype
    q_pre: torch.Tensor        # [T_q, R, 128] pre-RoPE q of the retrieval heads, dtype
    k_pre: torch.Tensor        # [T_k, Hkv, 128] pre-RoPE k, dtype
    w_q: torch.Tensor          # [R, 16, 128] float32: W^Q of every retrieval slot
    w_k: torch.Tensor          # [R, 16, 128] float32: W^K of every retrieval slot (the same tensor as w_q
                               # when the projection is shared)
    cu_q: torch.Tensor         # [B+1] int32
    cu_k: torch.Tensor         # [B+1] int32
    top_p: torch.Tensor        # [B] float32
    seqlens_q: List[int]
    seqlens_k: List[int]
    ret_heads: torch.Tensor    # [R] int32 (host)
    needle_pos: dict           # (b, slot) -> sorted list of key positions (within the sequence)
    peaky: List[bool]

    @property
    def total_q(self) -> int:
        return int(sum(self.seqlens_q))

    @property
    def total_k(self) -> int:
        return int(sum(self.seqlens_k))


def _lengths(cfg: Config):
    if cfg.seqlens is not None:
        lk = [int(x) for x in cfg.seqlens]
        assert len(lk) == cfg.batch
        return (list(lk) if cfg.kind == "prefill" else [1] * cfg.batch), lk
    if cfg.kind == "prefill":
        return [cfg.seqlen] * cfg.batch, [cfg.seqlen] * cfg.batch
    if cfg.ragged:
        g = _gen("cpu", cfg.seed, _TAG["len"], 0)
        u = torch.rand(cfg.batch, generator=g, dtype=torch.float64).tolist()
        lk = log_uniform_lengths(cfg.batch, cfg.ragged_min, cfg.ragged_max, u)
    else:
        lk = [cfg.seqlen] * cfg.batch
    return [1] * cfg.batch, lk


def _top_p(cfg: Config) -> List[float]:
    if cfg.top_p_range is None:
        return [cfg.top_p] * cfg.batch
    g = _gen("cpu", cfg.seed, _TAG["p"], 0)
    lo, hi = cfg.top_p_range
    u = torch.rand(cfg.batch, generator=g, dtype=torch.float64)
    return (lo + (hi - lo) * u).tolist()


def _peaky(cfg: Config) -> List[bool]:
    if cfg.kind != "decode" or cfg.needles != "query":
        return [False] * cfg.batch
    if not cfg.ragged:
        return [True] * cfg.batch
    g = _gen("cpu", cfg.seed, _TAG["peaky"], 0)
    u = torch.rand(cfg.batch, generator=g, dtype=torch.float64)
    return (u < cfg.peaky_frac).tolist()


def make_inputs(cfg: Config, device="cpu") -> Inputs:
    """Draw every input tensor of ``cfg`` on ``device`` (seeded, chunked)."""
    dt = torch_dtype(cfg.dtype)
    d, R, Hq, Hkv = cfg.head_dim, cfg.n_ret, cfg.n_q_heads, cfg.n_kv_heads
    lq, lk = _lengths(cfg)
    Tq, Tk = sum(lq), sum(lk)
    cu_q = [0]
    cu_k = [0]
    for a, b in zip(lq, lk):
        cu_q.append(cu_q[-1] + a)
        cu_k.append(cu_k[-1] + b)
    ret = list(cfg.ret_heads)
    peaky = _peaky(cfg)

    # positions of every packed query / key row
    qpos = torch.empty(Tq, dtype=torch.int64)
    kpos = torch.empty(Tk, dtype=torch.int64)
    for b in range(cfg.batch):
        kpos[cu_k[b]:cu_k[b + 1]] = torch.arange(lk[b])
        qpos[cu_q[b]:cu_q[b + 1]] = torch.arange(lk[b] - lq[b], lk[b])

    if cfg.proj == "shared":
        w64 = orthonormal_projection(cfg.seed, cfg.idx_dim, d)
        w_q = w64.to(torch.float32)[None].repeat(R, 1, 1).contiguous()
        w_k = w_q
    elif cfg.proj == "distinct":
        w_q = torch.stack([orthonormal_projection(cfg.seed, cfg.idx_dim, d, "wq", r) for r in range(R)]
                          ).to(torch.float32).contiguous() if R else torch.zeros((0, cfg.idx_dim, d))
        w_k = torch.stack([orthonormal_projection(cfg.seed, cfg.idx_dim, d, "wk", r) for r in range(R)]
                          ).to(torch.float32).contiguous() if R else torch.zeros((0, cfg.idx_dim, d))
    else:
        raise ValueError(f"unknown projection kind {cfg.proj!r}")

    # topic directions for prefill needles
    topics = None
    if cfg.needles == "topic":
        g = _gen("cpu", cfg.seed, _TAG["topic"], 0)
        t = torch.randn((R, d), generator=g, dtype=torch.float64)
        topics = (t / torch.linalg.vector_norm(t, dim=-1, keepdim=True)).to(device)

    q = torch.empty((Tq, Hq, d), dtype=dt, device=device)
    q_pre = torch.empty((Tq, R, d), dtype=dt, device=device)
    qdir = torch.empty((Tq, R, d), dtype=torch.float64, device=device) if cfg.needles == "query" else None
    for c0 in range(0, Tq, CHUNK):
        c1 = min(Tq, c0 + CHUNK)
        x = _randn_chunk(cfg.seed, "q", c0 // CHUNK, (c1 - c0, Hq, d), device)
        if topics is not None:
            for r, h in enumerate(ret):
                x[:, h, :] = _bend(x[:, h, :], topics[r], cfg.needle_cos)
        if qdir is not None:
            for r, h in enumerate(ret):
                qdir[c0:c1, r] = x[:, h, :] / torch.linalg.vector_norm(x[:, h, :], dim=-1, keepdim=True)
        q_pre[c0:c1] = x[:, ret, :].to(dt)
        rope_inplace(x, qpos[c0:c1].to(device), cfg.rope_theta)
        q[c0:c1] = x.to(dt)
        del x

    # needle positions
    needle_pos = {}
    if cfg.needles == "topic":
        for b in range(cfg.batch):
            n = int(math.floor(cfg.needle_frac * lk[b]))
            for r in range(R):
                g = _gen("cpu", cfg.seed, _TAG["npos"], b * 1000 + r)
                pos = torch.randperm(lk[b], generator=g)[:n].sort().values
                needle_pos[(b, r)] = pos.tolist()
    elif cfg.needles == "query":
        for b in range(cfg.batch):
            for r in range(R):
                if not peaky[b]:
                    needle_pos[(b, r)] = []
                    continue
                g = _gen("cpu", cfg.seed, _TAG["npos"], b * 1000 + r)
                n = min(cfg.needles_per_seq, lk[b])
                pos = torch.randperm(lk[b], generator=g)[:n].sort().values
                needle_pos[(b, r)] = pos.tolist()

    # global (packed) needle rows per KV head, with their direction
    plant = {}  # kv head -> (rows tensor, directions [n, d])
    for (b, r), plist in needle_pos.items():
        if not plist:
            continue
        g_kv = cfg.kv_of(ret[r])
        rows = torch.tensor(plist, dtype=torch.int64) + cu_k[b]
        if topics is not None:
            dirs = topics[r][None, :].expand(len(plist), d)
        else:
            dirs = qdir[cu_q[b], r][None, :].expand(len(plist), d)
        old = plant.get(g_kv)
        if old is None:
            plant[g_kv] = (rows, dirs)
        else:
            plant[g_kv] = (torch.cat([old[0], rows]), torch.cat([old[1], dirs]))

    k = torch.empty((Tk, Hkv, d), dtype=dt, device=device)
    k_pre = torch.empty((Tk, Hkv, d), dtype=dt, device=device)
    v = torch.empty((Tk, Hkv, d), dtype=dt, device=device)
    for c0 in range(0, Tk, CHUNK):
        c1 = min(Tk, c0 + CHUNK)
        x = _randn_chunk(cfg.seed, "k", c0 // CHUNK, (c1 - c0, Hkv, d), device)
        for g_kv, (rows, dirs) in plant.items():
            sel = (rows >= c0) & (rows < c1)
            if bool(sel.any()):
                rr = (rows[sel] - c0).to(device)
                dd = dirs[sel.to(dirs.device)].to(device)
                x[rr, g_kv, :] = _bend(x[rr, g_kv, :], dd, cfg.needle_cos)
        k_pre[c0:c1] = x.to(dt)
        rope_inplace(x, kpos[c0:c1].to(device), cfg.rope_theta)
        k[c0:c1] = x.to(dt)
        del x
        v[c0:c1] = _randn_chunk(cfg.seed, "v", c0 // CHUNK, (c1 - c0, Hkv, d), device).to(dt)

    wq_dev = w_q.to(device)
    wk_dev = wq_dev if w_k is w_q else w_k.to(device)
    return Inputs(
        cfg=cfg, q=q, k=k, v=v, q_pre=q_pre, k_pre=k_pre, w_q=wq_dev, w_k=wk_dev,
        cu_q=torch.tensor(cu_q, dtype=torch.int32, device=device),
        cu_k=torch.tensor(cu_k, dtype=torch.int32, device=device),
        top_p=torch.tensor(_top_p(cfg), dtype=torch.float32, device=device),
        seqlens_q=lq, seqlens_k=lk,
        ret_heads=torch.tensor(ret, dtype=torch.int32),
        needle_pos=needle_pos, peaky=peaky)


def plant_blocks(inp: Inputs, blocks, seed: int = 11, key_scale: float = 4.0, query_mix: float = 3.0,
                 jitter: float = 0.25) -> None:
    """Clustered index scores (in place): every retrieval head's pre-RoPE query gets a
    shared component along a seeded unit direction u (query_mix times its norm), and
    the pre-RoPE keys of the listed 64-key blocks, in every KV group that holds a
    retrieval head, are replaced by key_scale times their norm along u + jitter z / sqrt(d)
    (z standard normal per key, the sum normalised), so that the planted keys score
    highest but not alike (jitter 0: every planted key is key_scale sqrt(d) u, so they
    tie exactly).  Every row's highest indexer scores then sit in those blocks,
    as in selections that gather in a few contiguous spans.  The post-RoPE q and k
    (attention) are left unchanged."""
    cfg = inp.cfg
    g = _gen("cpu", seed, _TAG["topic"], 1)
    d = cfg.head_dim
    u = torch.randn(d, generator=g, dtype=torch.float64)
    u = u / torch.linalg.vector_norm(u)
    dt = inp.q_pre.dtype
    qp = inp.q_pre.to(torch.float64)
    qn = torch.linalg.vector_norm(qp, dim=-1, keepdim=True)
    inp.q_pre.copy_((qp + query_mix * qn * u.to(qp.device)).to(dt))
    rows = torch.cat([torch.arange(64 * b, 64 * b + 64) for b in blocks])
    for gk in sorted({cfg.kv_of(h) for h in cfg.ret_heads}):
        dirs = u + jitter * torch.randn(len(rows), d, generator=g, dtype=torch.float64) / math.sqrt(d)
        dirs = dirs / torch.linalg.vector_norm(dirs, dim=-1, keepdim=True)
        r = rows.to(inp.k_pre.device)
        kn = torch.linalg.vector_norm(inp.k_pre[r, gk].to(torch.float64), dim=-1, keepdim=True)
        if jitter == 0.0:
            kn = torch.full_like(kn, math.sqrt(d))     # identical keys: exact ties
        inp.k_pre[r, gk] = (key_scale * kn * dirs.to(kn.device)).to(dt)


def sample_rows(cfg: Config, n: int, extra: Optional[list] = None) -> List[int]:
    """Seeded uniform query rows in [0, L) plus forced edge rows (prefill)."""
    g = _gen("cpu", cfg.seed, 77, 0)
    L = cfg.seqlen
    rows = set(torch.randint(0, L, (n,), generator=g).tolist())
    for r in extra or []:
        if 0 <= r < L:
            rows.add(int(r))
    return sorted(rows)
