"""Row-level evaluation of the oracle over a packed varlen problem.  TEST INFRASTRUCTURE ONLY.

Applies the definitions of ``rtp_oracle`` to the packed layout the library
uses: q / out [T_q, Hq, 128], k / v / k_pre [T_k, Hkv, 128], q_pre
[T_q, R, 128], cumulative sequence offsets, and query i of sequence b at
position L_k(b) - L_q(b) + i.  GQA groups are contiguous:
kv(h) = floor(h * Hkv / Hq).
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

from . import rtp_oracle as O


@dataclasses.dataclass
class Problem:
    q: np.ndarray            # [T_q, Hq, 128] float64 (stored values)
    k: np.ndarray            # [T_k, Hkv, 128]
    v: np.ndarray
    q_pre: np.ndarray        # [T_q, R, 128]
    k_pre: np.ndarray        # [T_k, Hkv, 128]
    w_q: np.ndarray          # [R, 16, 128]
    w_k: np.ndarray          # [R, 16, 128]
    cu_q: Sequence[int]
    cu_k: Sequence[int]
    ret_heads: Sequence[int]
    top_p: Sequence[float]   # per sequence
    window: int
    n_sink: int
    dtype: str               # "f32" | "bf16"
    k_idx: Optional[np.ndarray] = None   # [R, T_k, 16] stored index keys (decode inputs)
    _kidx_cache: Dict[Tuple[int, int], np.ndarray] = dataclasses.field(default_factory=dict)

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

    def index_keys(self, b: int, r: int) -> np.ndarray:
        """k_idx rows of sequence b for retrieval slot r ([L_b, 16])."""
        key = (b, r)
        if key not in self._kidx_cache:
            k0, k1 = self.seq_range_k(b)
            if self.k_idx is not None:
                self._kidx_cache[key] = np.asarray(self.k_idx[r, k0:k1], dtype=np.float64)
            else:
                g = self.kv_of(self.ret_heads[r])
                self._kidx_cache[key] = O.project(self.k_pre[k0:k1, g], self.w_k[r], self.dtype)
        return self._kidx_cache[key]

    def all_index_keys(self) -> np.ndarray:
        """[R, T_k, 16] index cache for every retrieval slot (what the decode inputs hold)."""
        R = len(self.ret_heads)
        out = np.zeros((R, self.k.shape[0], O.IDX_DIM))
        for r in range(R):
            g = self.kv_of(self.ret_heads[r])
            out[r] = O.project(self.k_pre[:, g], self.w_k[r], self.dtype)
        return out

    def row(self, b: int, i: int, h: int, keys: Optional[np.ndarray] = None) -> O.RowResult:
        """Oracle result of query row i of sequence b on head h."""
        pos = self.pos_of(b, i)
        k0, k1 = self.seq_range_k(b)
        g = self.kv_of(h)
        K = self.k[k0:k1, g]
        V = self.v[k0:k1, g]
        qi = int(self.cu_q[b]) + i
        r = self.slot_of(h)
        if r >= 0:
            return O.retrieval_row(self.q[qi, h], self.q_pre[qi, r], self.w_q[r], K, V,
                                   self.index_keys(b, r), pos, float(self.top_p[b]),
                                   self.dtype, keys=keys)
        return O.local_row(self.q[qi, h], K, V, pos, self.window, self.n_sink)


def from_inputs(inp, k_idx: Optional[np.ndarray] = None) -> Problem:
    """Build a Problem from ``synth.Inputs`` (torch tensors on any device)."""
    def np64(t):
        return t.detach().float().cpu().numpy().astype(np.float64)
    cfg = inp.cfg
    return Problem(
        q=np64(inp.q), k=np64(inp.k), v=np64(inp.v), q_pre=np64(inp.q_pre),
        k_pre=np64(inp.k_pre), w_q=np64(inp.w), w_k=np64(inp.w),
        cu_q=inp.cu_q.cpu().tolist(), cu_k=inp.cu_k.cpu().tolist(),
        ret_heads=list(cfg.ret_heads), top_p=[float(x) for x in inp.top_p.cpu().tolist()],
        window=cfg.window, n_sink=cfg.n_sink, dtype=cfg.dtype, k_idx=k_idx)
