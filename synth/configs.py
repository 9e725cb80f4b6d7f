"""Workload configurations for the RTPurbo-style sparse-attention hot path.

Each configuration fixes shapes, dtypes, the head split and the structure of
the synthetic inputs.  The numbers follow the five workloads this repository
is measured on; the readings of points the method description leaves open are
written next to the field they set:

* ``n_sink = 4`` everywhere: the local-head pattern of the paper keeps the
  first four tokens as attention sinks ("Full Attention Strikes Back ...",
  paper-graph-ui summary, section 3.4 "Local Head Attention Pattern").
* ``ret_heads``: one retrieval head per KV group (0, 8, 16, 24 with 32 query
  heads over 4 KV heads) for the large workloads, heads {0, 1} for the tiny
  one.  GQA groups are contiguous: kv(h) = floor(h * Hkv / Hq).
* The indexer score is s = (q_idx . k_idx) / sqrt(16).  The workloads use one
  seeded orthonormal 16x128 projection for every retrieval head and for both q
  and k (``proj = "shared"``); ``proj = "distinct"`` draws an independent one
  per retrieval head and per side (W^Q_h, W^K_h), the form the method itself
  trains (section 3.4 "Low-Dimensional Projection Mechanism and Stage-1
  Training").
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Tuple


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    kind: str                      # "prefill" or "decode"
    batch: int
    n_q_heads: int
    n_kv_heads: int
    dtype: str                     # "f32" or "bf16"
    ret_heads: Tuple[int, ...]
    window: int
    top_p: float                   # scalar p (ragged decode draws per-sequence p instead)
    seqlen: int = 0                # prefill length, or decode KV length when not ragged
    head_dim: int = 128
    idx_dim: int = 16
    n_sink: int = 4
    rope_theta: float = 1.0e6
    seed: int = 0
    # needle structure
    needles: str = "none"          # "none" | "topic" (prefill) | "query" (decode)
    needle_frac: float = 0.0       # prefill: fraction of tokens that are needles
    needles_per_seq: int = 0       # decode: needles per (sequence, KV group)
    needle_cos: float = 0.8
    # ragged decode
    ragged: bool = False
    ragged_min: int = 0
    ragged_max: int = 0
    top_p_range: Optional[Tuple[float, float]] = None
    peaky_frac: float = 0.0        # fraction of sequences that carry needles
    # how many query rows the oracle verifies (0 = all)
    verify_rows: int = 0
    # explicit per-sequence KV lengths (prefill: L_q = L_k; decode: L_q = 1)
    seqlens: Optional[Tuple[int, ...]] = None
    # indexer projections: "shared" (one W for every slot, q and k) or "distinct"
    # (an independent W^Q_r and W^K_r per retrieval slot)
    proj: str = "shared"

    @property
    def n_ret(self) -> int:
        return len(self.ret_heads)

    @property
    def local_heads(self) -> Tuple[int, ...]:
        r = set(self.ret_heads)
        return tuple(h for h in range(self.n_q_heads) if h not in r)

    def kv_of(self, h: int) -> int:
        return (h * self.n_kv_heads) // self.n_q_heads


TINY_PREFILL = Config(
    name="tiny_prefill_2k", kind="prefill", batch=1, seqlen=2048,
    n_q_heads=4, n_kv_heads=1, dtype="f32", ret_heads=(0, 1), window=256,
    top_p=0.9, needles="none")

DECODE_32K = Config(
    name="decode_32k_b8", kind="decode", batch=8, seqlen=32768,
    n_q_heads=32, n_kv_heads=4, dtype="bf16", ret_heads=(0, 8, 16, 24),
    window=1024, top_p=0.95, needles="query", needles_per_seq=64)

PREFILL_128K = Config(
    name="prefill_128k", kind="prefill", batch=1, seqlen=131072,
    n_q_heads=32, n_kv_heads=4, dtype="bf16", ret_heads=(0, 8, 16, 24),
    window=2048, top_p=0.9, needles="topic", needle_frac=0.001, verify_rows=512)

PREFILL_1M = Config(
    name="prefill_1m", kind="prefill", batch=1, seqlen=1048576,
    n_q_heads=32, n_kv_heads=4, dtype="bf16", ret_heads=(0, 8, 16, 24),
    window=4096, top_p=0.9, needles="topic", needle_frac=0.001, verify_rows=256)

RAGGED_DECODE = Config(
    name="ragged_decode_b64", kind="decode", batch=64,
    n_q_heads=32, n_kv_heads=4, dtype="bf16", ret_heads=(0, 8, 16, 24),
    window=1024, top_p=0.9, needles="query", needles_per_seq=256,
    ragged=True, ragged_min=4096, ragged_max=262144,
    top_p_range=(0.8, 0.99), peaky_frac=0.5)

ALL = {c.name: c for c in (TINY_PREFILL, DECODE_32K, PREFILL_128K, PREFILL_1M, RAGGED_DECODE)}


def scaled(cfg: Config, **kw) -> Config:
    """A copy of ``cfg`` with some fields replaced (used for reduced-size cases)."""
    return dataclasses.replace(cfg, **kw)


def forced_edge_rows(cfg: Config):
    """Query rows that sit on window / sink edges; always verified."""
    L, W = cfg.seqlen, cfg.window
    rows = {0, 1, W - 2, W - 1, W, W + 3, W + 4, L - 1, cfg.n_sink - 1, cfg.n_sink}
    return sorted(r for r in rows if 0 <= r < L)


def log_uniform_lengths(n: int, lo: int, hi: int, u) -> list:
    """Map uniforms u in [0, 1) to lengths log-uniform in [lo, hi]."""
    a, b = math.log(lo), math.log(hi)
    return [int(round(math.exp(a + (b - a) * float(x)))) for x in u]
