"""Row-level evaluation of the oracle over a packed varlen problem.  TEST INFRASTRUCTURE ONLY.

Applies the definitions of ``rtp_oracle`` to the packed layout the library
uses: q / out [T_q, Hq, 128], k / v / k_pre [T_k, Hkv, 128], q_pre
[T_q, R, 128], cumulative sequence offsets, and query i of sequence b at
position L_k(b) - L_q(b) + i.  GQA groups are contiguous:
kv(h) = floor(h * Hkv / Hq).

Tensors may be numpy arrays or CPU torch tensors of any float dtype; slices
are converted to float64 on first use and cached per (sequence, KV head).
"""
from __future__ import annotations

import dataclasses
from typing import Any, Dict, Optional, Sequence, Tuple

import numpy as np

from . import rtp_oracle as O


def _f64(x) -> np.ndarray:
    if isinstance(x, np.ndarray):
        return x.astype(np.float64, copy=False)
    import torch  # tensors handed over by the tests
    return x.detach().to(torch.float64).cpu().numpy()


@dataclasses.dataclass
class Problem:
    q: Any                   # [T_q, Hq, 128]
    k: Any                   # [T_k, Hkv, 128]
    v: Any
    q_pre: Any               # [T_q, R, 128]
    k_pre: Any               # [T_k, Hkv, 128]
    w_q: Any                 # [R, 16, 128]
    w_k: Any                 # [R, 16, 128]
    cu_q: Sequence[int]
    cu_k: Sequence[int]
    ret_heads: Sequence[int]
    top_p: Sequence[float]   # per sequence
    window: int
    n_sink: int
    dtype: str               # "f32" | "bf16"
    k_idx: Any = None        # [R, T_k, 16] stored index keys (decode inputs), optional
    top_k: Optional[Sequence[int]] = None   # per sequence: fixed top-k instead of top-p
    blocks: bool = False     # the pages' block-granular top-p instead of the token-exact one
    _cache: Dict[Tuple, np.ndarray] = dataclasses.field(default_factory=dict)

    @property
    def n_q_heads(self) -> int:
        return self.q.shape[1]

    @property
    def n_kv_heads(self) -> int:
        return self.k.shape[1]

    def kv_of(self, h: int) -> int:
        return (h * self.n_kv_heads) // self.n_q_heads

    def slot_of(self, h: int) -> int:
        rh = list(self.ret_heads)
        return rh.index(h) if h in rh else -1

    def seq_range_k(self, b: int):
        return int(self.cu_k[b]), int(self.cu_k[b + 1])

    def pos_of(self, b: int, i: int) -> int:
        lq = int(self.cu_q[b + 1]) - int(self.cu_q[b])
        lk = int(self.cu_k[b + 1]) - int(self.cu_k[b])
        return lk - lq + i

    def _kv(self, name: str, b: int, g: int) -> np.ndarray:
        key = (name, b, g)
        if key not in self._cache:
            k0, k1 = self.seq_range_k(b)
            self._cache[key] = _f64(getattr(self, name)[k0:k1, g])
        return self._cache[key]

    def w(self, which: str, r: int) -> np.ndarray:
        key = (which, r)
        if key not in self._cache:
            self._cache[key] = _f64(getattr(self, which)[r])
        return self._cache[key]

    def index_keys(self, b: int, r: int) -> np.ndarray:
        """k_idx rows of sequence b for retrieval slot r ([L_b, 16])."""
        key = ("kidx", b, r)
        if key not in self._cache:
            k0, k1 = self.seq_range_k(b)
            if self.k_idx is not None:
                self._cache[key] = _f64(self.k_idx[r, k0:k1])
            else:
                g = self.kv_of(self.ret_heads[r])
                self._cache[key] = O.project(self._kv("k_pre", b, g), self.w("w_k", r), self.dtype)
        return self._cache[key]

    def q_row(self, qi: int, h: int) -> np.ndarray:
        key = ("q", qi, h)
        if key not in self._cache:
            self._cache[key] = _f64(self.q[qi, h])
        return self._cache[key]

    def q_pre_row(self, qi: int, r: int) -> np.ndarray:
        key = ("qp", qi, r)
        if key not in self._cache:
            self._cache[key] = _f64(self.q_pre[qi, r])
        return self._cache[key]

    def row(self, b: int, i: int, h: int, keys: Optional[np.ndarray] = None) -> O.RowResult:
        """Oracle result of query row i of sequence b on head h."""
        pos = self.pos_of(b, i)
        g = self.kv_of(h)
        K = self._kv("k", b, g)
        V = self._kv("v", b, g)
        qi = int(self.cu_q[b]) + i
        r = self.slot_of(h)
        if r >= 0:
            return O.retrieval_row(self.q_row(qi, h), self.q_pre_row(qi, r), self.w("w_q", r), K, V,
                                   self.index_keys(b, r), pos, float(self.top_p[b]), self.dtype, keys=keys,
                                   k=None if self.top_k is None else int(self.top_k[b]), blocks=self.blocks)
        return O.local_row(self.q_row(qi, h), K, V, pos, self.window, self.n_sink)


def from_inputs(inp, k_idx=None) -> Problem:
    """Build a Problem from ``synth.Inputs`` (tensors are copied to host memory, not converted)."""
    def host(t):
        return t.detach().cpu() if t is not None else None
    cfg = inp.cfg
    return Problem(
        q=host(inp.q), k=host(inp.k), v=host(inp.v), q_pre=host(inp.q_pre), k_pre=host(inp.k_pre),
        w_q=host(inp.w_q), w_k=host(inp.w_k),
        cu_q=inp.cu_q.cpu().tolist(), cu_k=inp.cu_k.cpu().tolist(),
        ret_heads=list(cfg.ret_heads), top_p=[float(x) for x in inp.top_p.cpu().tolist()],
        window=cfg.window, n_sink=cfg.n_sink, dtype=cfg.dtype, k_idx=host(k_idx))
