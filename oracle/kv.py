"""CPU oracle of the 4-bit KV-cache codec and of sparse attention over it.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library's
product path never does.  It imports only NumPy and shares no code with the
HIP kernels.

What is computed, as the pages state it:

* KV-cache quantization: the cache of keys and values can be stored in 4 bits
  per element (an optional 4-bit KV cache: "40天64个版本：Strata如何用发版
  密度定义AI本地推理路线图", first step, release 0.1.8), quantized per head and
  symmetrically, without outlier handling (lqnn.cn static review, §3.1 "量化方
  案选型", the KV-cache branch).  The dequantization is fused into the
  operator that reads the cache, so there is no separate round trip through
  memory (yfxerp.com static review, §4.2).
* Sparse attention: an indexer picks about 2000 cache positions for every
  query and the attention kernel reads only those rows of the cache instead
  of building a full mask ("两天移植，预填充提速8倍：Strata引擎实测"
  (kongchang.com), section "Strata快在哪：不是魔法，是物流", attention
  paragraph; the background note on KV cache beside it).

Readings of points the pages leave open (each also listed in the design
notes):

* "per head": one scale per (position, KV head) vector of head_dim values;
  symmetric codes q in [-8, 7] with s = fp16(max|x| / 7) and q = rint(x / s)
  (nearest-even), stored offset-binary (u = q + 8, even index in the low
  nibble) like the expert weights; an all-zero vector gets s = 0, q = 0.  The
  code decision is taken in fp32 (the division x / s and the scale's max / 7),
  the precision the kernel takes it in; dequantization is exact in fp64.
* the indexer is outside the method's stated steps (the pages give only the
  count): its output, a list of cache positions per query, is an input;
* attention over the selected rows is standard scaled dot-product attention
  with grouped KV heads: query head h reads KV head h // (Hq / Hkv), weights
  softmax over the selected positions of sm_scale * q . k.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "kv_quantize",
    "kv_dequant",
    "sparse_attention",
    "kv_bytes_per_token",
]


def _bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def kv_quantize(x_bf16: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Per-head symmetric 4-bit quantization of key or value vectors.

    ``x_bf16``: bfloat16 bit patterns ``[..., D]`` (one vector per position and
    KV head).  Returns ``(packed uint8 [..., D/2], scale float16 [...])`` with
    ``s = fp16(fp32(max|x|) / 7)``, ``q = clamp(rint(fp32(x) / fp32(s)), -8, 7)``
    (``q = 0`` where ``s = 0``), nibble ``u = q + 8``, even index in the low
    nibble (lqnn.cn static review, §3.1: per-head symmetric quantization of the
    KV cache).
    """
    x = _bf16_to_f32(x_bf16)
    D = x.shape[-1]
    if D % 2:
        raise ValueError("head_dim must be even")
    amax = np.abs(x).max(axis=-1)
    s16 = (amax / np.float32(7.0)).astype(np.float16)
    s32 = s16.astype(np.float32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(s32 > 0, x / np.where(s32 > 0, s32, np.float32(1.0)), np.float32(0.0))
    q = np.clip(np.rint(r), -8, 7).astype(np.int16)
    u = (q + 8).astype(np.uint8)
    packed = (u[..., 0::2] | (u[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, s16


def kv_dequant(packed: np.ndarray, scale: np.ndarray) -> np.ndarray:
    """``x[..., d] = (u_d - 8) * s`` in float64 (exact)."""
    p = np.asarray(packed, dtype=np.uint8)
    q = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.float64)
    q[..., 0::2] = (p & 0x0F).astype(np.float64) - 8.0
    q[..., 1::2] = (p >> 4).astype(np.float64) - 8.0
    return q * np.asarray(scale, dtype=np.float16).astype(np.float64)[..., None]


def sparse_attention(q_bf16: np.ndarray, k_packed: np.ndarray, k_scale: np.ndarray, v_packed: np.ndarray,
                     v_scale: np.ndarray, sel: np.ndarray, sm_scale: float) -> np.ndarray:
    """Attention of each query over its selected cache rows, fp64.

    ``q_bf16 [Tq, Hq, D]`` bf16 bits; cache ``k_packed / v_packed [L, Hkv, D/2]``,
    ``k_scale / v_scale [L, Hkv]``; ``sel [Tq, n]`` cache positions per query
    (kongchang.com hands-on, attention paragraph: only the selected rows are
    read).  ``out[t, h] = sum_i p_i v[sel[t, i], g]`` with ``p = softmax_i(
    sm_scale * q[t, h] . k[sel[t, i], g])`` and ``g = h // (Hq / Hkv)``.
    """
    q = _bf16_to_f32(q_bf16).astype(np.float64)
    Tq, Hq, D = q.shape
    Hkv = k_packed.shape[1]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    out = np.zeros((Tq, Hq, D), dtype=np.float64)
    for t in range(Tq):
        rows = np.asarray(sel[t], dtype=np.int64)
        K = kv_dequant(k_packed[rows], k_scale[rows])  # [n, Hkv, D]
        V = kv_dequant(v_packed[rows], v_scale[rows])
        for h in range(Hq):
            g = h // G
            s = sm_scale * (K[:, g, :] @ q[t, h])
            p = np.exp(s - s.max())
            p /= p.sum()
            out[t, h] = p @ V[:, g, :]
    return out


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, bits: int) -> int:
    """Cache bytes per token for K and V over all layers: fp16 (bits = 16) or
    the 4-bit codec (bits = 4: head_dim / 2 bytes plus one fp16 scale per
    head vector)."""
    if bits == 16:
        per_head = head_dim * 2
    elif bits == 4:
        per_head = head_dim // 2 + 2
    else:
        raise ValueError("bits must be 16 or 4")
    return 2 * layers * kv_heads * per_head
