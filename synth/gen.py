"""Seeded synthetic inputs for the routed MoE FFN layer.

Test and benchmark infrastructure shared by the fp64 oracle and the GPU path.
It draws inputs and prepares them in the storage formats the layer consumes;
it holds none of the layer's own steps (no routing, grouping, dequantization,
matmul, activation or combine).

Storage formats produced here (the formats the C ABI consumes):

* router logits: float32 ``[T, E]``;
* activations ``x``: bfloat16 bit patterns in a uint16 ``[T, H]`` array
  (float32 draw rounded to nearest-even);
* each expert matrix ``W[N, K]`` (gate and up: ``N=I, K=H``; down: ``N=H, K=I``)
  as symmetric 4-bit integers in groups of ``g`` consecutive K elements,
  one fp16 scale per group: ``packed uint8 [E, N, K/2]`` holding the
  offset-binary nibble ``u = q + 8`` with the even K index in the low nibble,
  and ``scales float16 [E, N, K/g]``.

Grouped 4-bit weights with a per-group scale are what the Strata reviews
describe ("源码静态评测：Strata 如何在消费级硬件跑本地大模型" (yfxerp.com),
§3.1; the lqnn.cn static review, §3.1 "量化方案选型", which names group sizes
32/64/128).  The scale rule ``s = fp16(max|w| / 7)`` with symmetric codes is
the workload definition this library is measured on; the pages leave the
rounding of the scale and of the codes open, so both are round-to-nearest-even
here and the oracle and the kernels consume the same ``q`` and ``s``.

Draw order (fixed, so a seed names one input set):
``root = SeedSequence(seed)``; ``root.spawn(4)`` gives the streams for
(logits, x, Zipf ranks, weights); the weight stream spawns one child per
expert, drawing gate ``[I, H]``, up ``[I, H]``, down ``[H, I]`` in that order,
float32 N(0, 0.02) (0.02 is the standard deviation).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

WEIGHT_STD = 0.02


@dataclass(frozen=True)
class MoEConfig:
    """Shape of one MoE FFN layer invocation.

    T tokens, hidden size H, expert intermediate size I, E experts, top-k,
    int4 group size g along K.  ``zipf_s`` set means router logits get a
    per-expert bias ``-zipf_s * ln(rank_e)`` over a seeded rank permutation,
    so that expert popularity follows a Zipf law of exponent ``zipf_s``.
    ``weight_std`` is the standard deviation of the expert weights before
    quantization (0.02 for every workload configuration).  ``fmt`` names the
    weight format (see ``quantize_groups``).  ``draft_sigma`` set means the
    tokens after the first are drafts whose router logits stay close to the
    first token's (its row plus ``draft_sigma`` times an independent N(0, 1)
    row), so that they select mostly the same experts.
    """

    name: str
    T: int
    H: int
    I: int
    E: int
    k: int
    g: int
    seed: int
    zipf_s: float | None = None
    weight_std: float = WEIGHT_STD
    fmt: str = "int4"  # "int4" (symmetric), "int4_asym" (scale + zero point), "int5" (symmetric 5-bit)
    draft_sigma: float | None = None  # tokens 1.. = token 0's logits + draft_sigma * N(0, 1)

    @property
    def pairs(self) -> int:
        return self.T * self.k


CONFIGS: dict[str, MoEConfig] = {
    # tiny layer, single seed
    "tiny": MoEConfig("tiny", T=64, H=256, I=128, E=16, k=2, g=32, seed=0),
    # one decode token plus three speculative drafts verified together
    "decode": MoEConfig("decode", T=4, H=2048, I=512, E=512, k=10, g=64, seed=1),
    # a 512-token prefill batch
    "prefill512": MoEConfig("prefill512", T=512, H=2048, I=512, E=512, k=10, g=64, seed=2),
    # a 6144-token prefill chunk
    "prefill6144": MoEConfig("prefill6144", T=6144, H=2048, I=512, E=512, k=10, g=64, seed=3),
    # skewed, larger-shape prefill: Zipf(1.1) expert popularity
    "zipf6144": MoEConfig("zipf6144", T=6144, H=4096, I=1024, E=256, k=8, g=128, seed=4, zipf_s=1.1),
    # the 6144-token chunk with the other two group sizes the pages name
    "prefill6144_g32": MoEConfig("prefill6144_g32", T=6144, H=2048, I=512, E=512, k=10, g=32, seed=5),
    "prefill6144_g128": MoEConfig("prefill6144_g128", T=6144, H=2048, I=512, E=512, k=10, g=128, seed=6),
    # the 6144-token chunk in the two other weight formats the pages name
    "prefill6144_asym": MoEConfig("prefill6144_asym", T=6144, H=2048, I=512, E=512, k=10, g=64, seed=7,
                                  fmt="int4_asym"),
    "prefill6144_int5": MoEConfig("prefill6144_int5", T=6144, H=2048, I=512, E=512, k=10, g=64, seed=8, fmt="int5"),
    # a decode step in those formats
    "decode_asym": MoEConfig("decode_asym", T=4, H=2048, I=512, E=512, k=10, g=64, seed=9, fmt="int4_asym"),
    "decode_int5": MoEConfig("decode_int5", T=4, H=2048, I=512, E=512, k=10, g=64, seed=10, fmt="int5"),
    # a decode step whose 3 drafts route mostly to the first token's experts
    "decode_shared": MoEConfig("decode_shared", T=4, H=2048, I=512, E=512, k=10, g=64, seed=11, draft_sigma=0.05),
}


def config(name_or_cfg, **overrides) -> MoEConfig:
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    return replace(cfg, **overrides) if overrides else cfg


def weight_bytes_per_expert(cfg: MoEConfig) -> int:
    """Packed bytes of one expert's three matrices plus their side data:
    fp16 scales (all formats), 4-bit zero points (int4_asym), one fifth bit
    per weight (int5)."""
    n = 3 * cfg.H * cfg.I
    extra = {"int4": 0, "int4_asym": n // cfg.g // 2, "int5": n // 8}[cfg.fmt]
    return n // 2 + 2 * (n // cfg.g) + extra


@dataclass
class MoEInputs:
    cfg: MoEConfig
    logits: np.ndarray  # float32 [T, E]
    x_bf16: np.ndarray  # uint16 [T, H]
    weights: dict = field(default_factory=dict)  # see module docstring


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bit patterns."""
    b = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    rounded = (b + (np.uint32(0x7FFF) + ((b >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def quantize_int4_groups(w: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray]:
    """Symmetric int4 group quantization of ``w[N, K]`` along K.

    Returns ``(packed uint8 [N, K/2], scales float16 [N, K/g])`` with
    ``s = fp16(fp32(max|w|)/7)`` per group, ``q = clamp(rint(w / s), -8, 7)``
    (``q = 0`` where ``s = 0``), nibble ``u = q + 8``, even K in the low nibble.
    """
    n, kdim = w.shape
    if kdim % g or kdim % 2:
        raise ValueError(f"K={kdim} must be a multiple of g={g} and of 2")
    grp = np.asarray(w, dtype=np.float32).reshape(n, kdim // g, g)
    amax = np.abs(grp).max(axis=2)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    safe = np.where(s > 0, s, 1.0)
    r = np.where(s > 0, grp.astype(np.float64) / safe, 0.0)
    q = np.clip(np.rint(r), -8, 7).astype(np.int16)
    u = (q + 8).astype(np.uint8).reshape(n, kdim)
    packed = (u[:, 0::2] | (u[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, s16


def quantize_int4_asym_groups(w: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Asymmetric 4-bit group quantization of ``w[N, K]`` along K (each group
    stores a scale and a zero point).

    The group's range is widened to contain 0 (lo = min(min w, 0), hi =
    max(max w, 0)); ``s = fp16(fp32(hi - lo) / 15)``, ``z = clamp(rint(-lo / s),
    0, 15)``, ``u = clamp(rint(w / s) + z, 0, 15)`` (all 0 where s = 0), so
    ``w ~ (u - z) * s``.  Returns ``(packed uint8 [N, K/2], scales float16
    [N, K/g], zeros uint8 [N, K/g/2])`` with u as offset-binary nibbles (even
    K in the low nibble) and the zero points two per byte (group j in byte
    j // 2, even j in the low nibble).
    """
    n, kdim = w.shape
    if kdim % g or (kdim // g) % 2:
        raise ValueError(f"K={kdim} must hold an even number of groups of g={g}")
    grp = np.asarray(w, dtype=np.float32).reshape(n, kdim // g, g)
    lo = np.minimum(grp.min(axis=2), np.float32(0))
    hi = np.maximum(grp.max(axis=2), np.float32(0))
    s16 = ((hi - lo) / np.float32(15.0)).astype(np.float16)
    s = s16.astype(np.float64)
    safe = np.where(s > 0, s, 1.0)
    z = np.where(s > 0, np.clip(np.rint(-lo.astype(np.float64) / safe), 0, 15), 0).astype(np.int16)
    r = np.where(s[..., None] > 0, grp.astype(np.float64) / safe[..., None], 0.0)
    u = np.where(s[..., None] > 0, np.clip(np.rint(r) + z[..., None], 0, 15), 0).astype(np.uint8).reshape(n, kdim)
    packed = (u[:, 0::2] | (u[:, 1::2] << np.uint8(4))).astype(np.uint8)
    zb = z.astype(np.uint8)
    zeros = (zb[:, 0::2] | (zb[:, 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, s16, zeros


def quantize_int5_groups(w: np.ndarray, g: int) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Symmetric 5-bit group quantization of ``w[N, K]`` along K.

    ``s = fp16(fp32(max|w|) / 15)``, ``q = clamp(rint(w / s), -16, 15)`` (0 where
    s = 0), ``u5 = q + 16``.  Returns ``(packed uint8 [N, K/2], scales float16
    [N, K/g], hi uint32 [N, K/32])``: the low four bits of u5 as offset-binary
    nibbles (even K in the low nibble) and the fifth bits in one 32-bit word
    per 32 K values, the fifth bit of K = 32m + 8c + i at bit 4i + c of word m.
    """
    n, kdim = w.shape
    if kdim % g or kdim % 32:
        raise ValueError(f"K={kdim} must be a multiple of g={g} and of 32")
    grp = np.asarray(w, dtype=np.float32).reshape(n, kdim // g, g)
    amax = np.abs(grp).max(axis=2)
    s16 = (amax / np.float32(15.0)).astype(np.float16)
    s = s16.astype(np.float64)[..., None]
    safe = np.where(s > 0, s, 1.0)
    q = np.where(s > 0, np.clip(np.rint(grp.astype(np.float64) / safe), -16, 15), 0).astype(np.int16)
    u5 = (q + 16).reshape(n, kdim)
    u = (u5 & 15).astype(np.uint8)
    packed = (u[:, 0::2] | (u[:, 1::2] << np.uint8(4))).astype(np.uint8)
    b = (u5 >> 4).astype(np.uint32).reshape(n, kdim // 32, 4, 8)  # [n, m, c, i]
    shifts = (4 * np.arange(8)[None, :] + np.arange(4)[:, None]).astype(np.uint32)  # [c, i] -> 4i + c
    hi = (b << shifts[None, None]).sum(axis=(2, 3), dtype=np.uint64).astype(np.uint32)
    return packed, s16, hi


def quantize_groups(w: np.ndarray, g: int, fmt: str) -> dict:
    """Quantize ``w[N, K]`` in format ``fmt``; returns the arrays by suffix:
    "" (packed nibbles), "_scale", and "_zero" (int4_asym) or "_hi" (int5)."""
    if fmt == "int4":
        p, sc = quantize_int4_groups(w, g)
        return {"": p, "_scale": sc}
    if fmt == "int4_asym":
        p, sc, z = quantize_int4_asym_groups(w, g)
        return {"": p, "_scale": sc, "_zero": z}
    if fmt == "int5":
        p, sc, hi = quantize_int5_groups(w, g)
        return {"": p, "_scale": sc, "_hi": hi}
    raise ValueError(f"unknown weight format {fmt!r}")


def _streams(seed: int):
    root = np.random.SeedSequence(seed)
    return root.spawn(4)  # logits, x, zipf ranks, weights


def make_logits(cfg: MoEConfig, seq: np.random.SeedSequence, rank_seq=None) -> np.ndarray:
    rng = np.random.default_rng(seq)
    logits = rng.standard_normal((cfg.T, cfg.E), dtype=np.float32)
    if cfg.zipf_s is not None:
        ranks = np.random.default_rng(rank_seq).permutation(cfg.E) + 1
        bias = (-cfg.zipf_s * np.log(ranks.astype(np.float64))).astype(np.float32)
        logits = logits + bias[None, :]
    if cfg.draft_sigma is not None and cfg.T > 1:
        logits[1:] = logits[0][None, :] + np.float32(cfg.draft_sigma) * logits[1:]
    return np.ascontiguousarray(logits, dtype=np.float32)


def make_x(cfg: MoEConfig, seq: np.random.SeedSequence) -> np.ndarray:
    rng = np.random.default_rng(seq)
    return bf16_bits_from_f32(rng.standard_normal((cfg.T, cfg.H), dtype=np.float32))


def make_router(T: int, H: int, E: int, seed: int) -> tuple[np.ndarray, np.ndarray]:
    """Inputs of the router projection: x bf16 [T][H] ~ N(0, 1) and router
    rows W_r bf16 [E][H] ~ N(0, 1/H), so that the logits x . W_r^T are about
    N(0, 1) like the logits of the layer configurations.  Returns bf16 bit
    patterns (uint16)."""
    sx, sw = np.random.SeedSequence(seed).spawn(2)
    x = np.random.default_rng(sx).standard_normal((T, H), dtype=np.float32)
    w = np.random.default_rng(sw).standard_normal((E, H), dtype=np.float32) * np.float32(1.0 / np.sqrt(H))
    return bf16_bits_from_f32(x), bf16_bits_from_f32(w)


def _expert_weights(cfg: MoEConfig, seq, e: int, out: dict) -> None:
    rng = np.random.default_rng(seq)
    std = np.float32(cfg.weight_std)
    for name, (n, kdim) in (("gate", (cfg.I, cfg.H)), ("up", (cfg.I, cfg.H)), ("down", (cfg.H, cfg.I))):
        w = rng.standard_normal((n, kdim), dtype=np.float32) * std
        for suffix, arr in quantize_groups(w, cfg.g, cfg.fmt).items():
            out[name + suffix][e] = arr


def make_weights(cfg: MoEConfig, seq: np.random.SeedSequence, threads: int | None = None) -> dict:
    E, H, I, g = cfg.E, cfg.H, cfg.I, cfg.g
    out = {
        "gate": np.empty((E, I, H // 2), np.uint8),
        "gate_scale": np.empty((E, I, H // g), np.float16),
        "up": np.empty((E, I, H // 2), np.uint8),
        "up_scale": np.empty((E, I, H // g), np.float16),
        "down": np.empty((E, H, I // 2), np.uint8),
        "down_scale": np.empty((E, H, I // g), np.float16),
    }
    for name, (n, kdim) in (("gate", (I, H)), ("up", (I, H)), ("down", (H, I))):
        if cfg.fmt == "int4_asym":
            out[name + "_zero"] = np.empty((E, n, kdim // g // 2), np.uint8)
        elif cfg.fmt == "int5":
            out[name + "_hi"] = np.empty((E, n, kdim // 32), np.uint32)
    kids = seq.spawn(E)
    threads = threads or min(16, os.cpu_count() or 1)
    if threads <= 1 or E == 1:
        for e in range(E):
            _expert_weights(cfg, kids[e], e, out)
    else:
        with ThreadPoolExecutor(threads) as ex:
            list(ex.map(lambda e: _expert_weights(cfg, kids[e], e, out), range(E)))
    return out


def make_inputs(name_or_cfg, with_weights: bool = True, **overrides) -> MoEInputs:
    cfg = config(name_or_cfg, **overrides)
    s_logits, s_x, s_rank, s_w = _streams(cfg.seed)
    inp = MoEInputs(cfg, make_logits(cfg, s_logits, s_rank), make_x(cfg, s_x))
    if with_weights:
        inp.weights = make_weights(cfg, s_w)
    return inp


def decode_steps(cfg: MoEConfig, steps: int) -> list[tuple[np.ndarray, np.ndarray]]:
    """Independent (logits, x) draws for ``steps`` decode steps over one expert pool.

    Step ``s`` uses ``SeedSequence([seed, 1000 + s])``; the Zipf ranks (if any)
    are those of the layer's own seed, so every step sees the same pool.
    """
    _, _, s_rank, _ = _streams(cfg.seed)
    out = []
    for s in range(steps):
        a, b = np.random.SeedSequence([cfg.seed, 1000 + s]).spawn(2)
        out.append((make_logits(cfg, a, s_rank), make_x(cfg, b)))
    return out
