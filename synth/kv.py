"""Seeded synthetic inputs for the 4-bit KV-cache codec and sparse attention.

Test and benchmark infrastructure shared by the oracle and the GPU path; it
draws inputs only (no quantization, no attention arithmetic).

Shapes follow the pages: head_dim 128 with 8 KV heads and 32 query heads
(grouped 4:1), the example structure of the lqnn.cn static review, §3.2; a
128k-token context (the release notes' 4-bit KV cache, release 0.1.8); about
2000 positions selected per query (kongchang.com hands-on, attention
paragraph), taken as 2048; a decode step of 1 token plus 3 drafts.  Keys,
values and queries are float32 N(0, 1) rounded to bf16; each query's
selection is n_sel distinct positions drawn uniformly (the pages do not
describe the indexer, so its output is modelled as a uniform sample).

Draw order: ``SeedSequence(seed).spawn(4)`` -> (keys, values, queries,
selection).
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

from .gen import bf16_bits_from_f32


@dataclass(frozen=True)
class AttnConfig:
    """Sparse attention over a 4-bit KV cache: Tq queries, Hq query heads,
    Hkv KV heads, head_dim D, L cache positions, n_sel selected per query."""

    name: str
    Tq: int
    Hq: int
    Hkv: int
    D: int
    L: int
    n_sel: int
    seed: int

    @property
    def sm_scale(self) -> float:
        return float(1.0 / np.sqrt(self.D))


ATTN_CONFIGS: dict[str, AttnConfig] = {
    # the pages' structure at a 128k context: one decode token plus 3 drafts
    "attn_decode128k": AttnConfig("attn_decode128k", Tq=4, Hq=32, Hkv=8, D=128, L=131072, n_sel=2048, seed=91),
    # a 16-query chunk over the same cache
    "attn_chunk16": AttnConfig("attn_chunk16", Tq=16, Hq=32, Hkv=8, D=128, L=131072, n_sel=2048, seed=92),
    # small: parity element by element, ragged chunk counts
    "attn_small": AttnConfig("attn_small", Tq=3, Hq=32, Hkv=8, D=128, L=5000, n_sel=300, seed=93),
}


def attn_config(name_or_cfg, **overrides) -> AttnConfig:
    cfg = ATTN_CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return replace(cfg, **overrides) if overrides else cfg


@dataclass
class AttnInputs:
    cfg: AttnConfig
    k_bf16: np.ndarray  # uint16 [L, Hkv, D]
    v_bf16: np.ndarray  # uint16 [L, Hkv, D]
    q_bf16: np.ndarray  # uint16 [Tq, Hq, D]
    sel: np.ndarray     # int32 [Tq, n_sel]


def _normal_bf16(seq, shape) -> np.ndarray:
    return bf16_bits_from_f32(np.random.default_rng(seq).standard_normal(shape, dtype=np.float32))


def make_attn_inputs(name_or_cfg, **overrides) -> AttnInputs:
    cfg = attn_config(name_or_cfg, **overrides)
    sk, sv, sq, ss = np.random.SeedSequence(cfg.seed).spawn(4)
    k = _normal_bf16(sk, (cfg.L, cfg.Hkv, cfg.D))
    v = _normal_bf16(sv, (cfg.L, cfg.Hkv, cfg.D))
    q = _normal_bf16(sq, (cfg.Tq, cfg.Hq, cfg.D))
    rng = np.random.default_rng(ss)
    sel = np.stack([rng.choice(cfg.L, size=cfg.n_sel, replace=False) for _ in range(cfg.Tq)]).astype(np.int32)
    return AttnInputs(cfg, k, v, q, sel)
