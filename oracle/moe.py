"""fp64 CPU oracle of the routed mixture-of-experts FFN layer.

TEST INFRASTRUCTURE.  Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module; the library's
product path never does.  It shares no code with the HIP kernels: it imports
neither the package nor its C library, only NumPy.

What the layer computes (the method as the pages state it):

* each layer's router picks a few of a large pool of experts for every token
  (512 experts, about 10 active per token): "两天移植，预填充提速8倍：Strata
  引擎实测" (kongchang.com), section "Strata快在哪：不是魔法，是物流", the MoE
  note; penglei.dev "Strata local MoE", section "原理一：把显存作为专家缓存";
* tokens are grouped by expert, so each expert's weights serve every token
  routed to it in one batch (same section of the kongchang.com hands-on: a
  larger prefill batch means more tokens reuse each expert);
* the expert matmuls run on group-quantized 4-bit weights that are
  dequantized inside the matmul rather than before it (lqnn.cn static review,
  §1.2 and §3.1; kongchang.com hands-on, the MMQ note);
* the expert FFN is SwiGLU, ``down(silu(gate x) * up x)``, and the experts'
  outputs are combined with softmax weights over the selected experts (the
  workload definition this library is measured on; the pages leave the
  gating function open).

Every step here is the plain definition written out in float64 with no
blocking, fusion or reordering; library calls (sort, bincount, cumsum, matmul)
serve as single steps.  Readings of points the pages leave open:

* top-k order: descending logit, equal logits broken toward the lower expert
  index, and -0.0 == +0.0 (IEEE comparison);
* routing weights: softmax over the k selected logits, in fp64;
* order of pairs inside an expert group: ascending pair index p = t*k + j;
* int4 storage: nibble u = q + 8, even K index in the low nibble, one fp16
  scale per g consecutive K elements, ``W = (u - 8) * s``.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "router_logits",
    "route",
    "histogram",
    "exclusive_scan",
    "permutation",
    "unpack_int4",
    "dequant",
    "bf16_to_f64",
    "silu",
    "expert_ffn",
    "ffn_grouped",
    "combine",
    "moe_layer",
    "moe_out_tokens",
]


def router_logits(x_bf16: np.ndarray, w_router_bf16: np.ndarray) -> np.ndarray:
    """Router projection: logits[t][e] = sum_h x[t][h] * W_r[e][h], in fp64.

    The router scores every expert for every token before the top-k picks a
    few (kongchang.com hands-on, section "Strata快在哪：不是魔法，是物流", the
    MoE note; penglei.dev "Strata local MoE", section "原理一").  Inputs are
    bf16 bit patterns (x [T][H], W_r [E][H]), widened exactly; the fp64
    matmul is one step.  Selections made on these logits are compared with
    the library's on its own fp32 logits (the decision is taken in the
    kernel's precision), the logits themselves within an error bound.
    """
    return bf16_to_f64(x_bf16) @ bf16_to_f64(w_router_bf16).T


def route(logits: np.ndarray, k: int) -> tuple[np.ndarray, np.ndarray]:
    """Top-k expert selection and softmax gating per token.

    Router picks a few experts per token: kongchang.com hands-on, section
    "Strata快在哪：不是魔法，是物流" (MoE note); penglei.dev, "原理一".
    Returns ``ids int32 [T, k]`` (descending logit, ties to the lower index)
    and ``w float64 [T, k]`` = softmax of the selected logits.
    """
    logits = np.asarray(logits, dtype=np.float32)
    if logits.ndim != 2:
        raise ValueError("logits must be [T, E]")
    T, E = logits.shape
    if not 1 <= k <= E:
        raise ValueError(f"k={k} must lie in [1, E={E}]")
    if not np.all(np.isfinite(logits)):
        raise ValueError("logits must be finite")
    # Stable sort of -logit keeps ascending index order among equal values;
    # -0.0 and +0.0 compare equal under IEEE ordering.
    order = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")
    ids = order[:, :k].astype(np.int32)
    sel = np.take_along_axis(logits, ids, axis=1).astype(np.float64)
    z = np.exp(sel - sel[:, :1])
    w = z / z.sum(axis=1, keepdims=True)
    return ids, w


def histogram(ids: np.ndarray, E: int) -> np.ndarray:
    """Per-expert count of routed (token, slot) pairs: ``counts[e] = #{p : ids[p] = e}``."""
    flat = np.asarray(ids).reshape(-1).astype(np.int64)
    return np.bincount(flat, minlength=E).astype(np.int32)


def exclusive_scan(counts: np.ndarray) -> np.ndarray:
    """``offsets[0] = 0``, ``offsets[e+1] = offsets[e] + counts[e]`` (length E+1)."""
    out = np.zeros(len(counts) + 1, dtype=np.int64)
    out[1:] = np.cumsum(np.asarray(counts, dtype=np.int64))
    return out.astype(np.int32)


def permutation(ids: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """Group pairs by expert: stable counting-sort order of the flat pair index.

    ``perm[i]`` is the pair index p = t*k + j at grouped position i (pairs of
    expert e occupy ``offsets[e]:offsets[e+1]`` in ascending p);
    ``inv_perm[p]`` is the grouped position of pair p.
    """
    flat = np.asarray(ids).reshape(-1)
    perm = np.argsort(flat, kind="stable").astype(np.int32)
    inv = np.empty_like(perm)
    inv[perm] = np.arange(len(perm), dtype=np.int32)
    return perm, inv


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Offset-binary nibbles to signed codes: ``q = u - 8``, even K from the low nibble."""
    p = np.asarray(packed, dtype=np.uint8)
    lo = (p & 0x0F).astype(np.int16) - 8
    hi = (p >> 4).astype(np.int16) - 8
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def dequant(packed: np.ndarray, scales: np.ndarray, g: int, zeros: np.ndarray | None = None,
            hi: np.ndarray | None = None) -> np.ndarray:
    """Group dequantization ``W[n, kk] = q[n, kk] * s[n, kk // g]`` in float64 (exact).

    Per-group scales: yfxerp.com static review §3.1; lqnn.cn static review §3.1.
    The code q of element kk comes from its nibble u (``unpack_int4`` gives
    u - 8) in one of three formats:

    * symmetric 4-bit (default): ``q = u - 8``;
    * asymmetric 4-bit, one zero point per group (each group stores a scale and
      a zero point: lqnn.cn static review, §3.1): ``q = u - z[n, kk // g]``,
      zero points packed two per byte (group j in byte j // 2, even j in the
      low nibble);
    * symmetric 5-bit blocks (4- and 5-bit block quantization, kongchang.com
      hands-on, MMQ note): ``q = u + 16 * b - 16`` where the fifth bit b of
      element kk = 32m + 8c + i is bit 4i + c of the 32-bit word hi[n, m].
    """
    u = unpack_int4(packed).astype(np.int64) + 8
    if hi is not None:
        words = np.asarray(hi, dtype=np.uint32)
        kk = np.arange(u.shape[-1])
        c, i = (kk % 32) // 8, kk % 8
        # word m = kk // 32 of the row, repeated over its 32 elements
        bit = (np.repeat(words, 32, axis=-1) >> (4 * i + c).astype(np.uint32)) & np.uint32(1)
        q = u + 16 * bit.astype(np.int64) - 16
    elif zeros is not None:
        zb = np.asarray(zeros, dtype=np.uint8)
        z = np.empty(zb.shape[:-1] + (zb.shape[-1] * 2,), dtype=np.int64)
        z[..., 0::2] = zb & 0x0F
        z[..., 1::2] = zb >> 4
        ngr = u.shape[-1] // g
        q = u - np.repeat(z[..., :ngr], g, axis=-1)
    else:
        q = u - 8
    s = np.asarray(scales, dtype=np.float16).astype(np.float64)
    return q.astype(np.float64) * np.repeat(s, g, axis=-1)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float64 exactly."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def silu(z: np.ndarray) -> np.ndarray:
    """``silu(z) = z / (1 + exp(-z))``."""
    return z / (1.0 + np.exp(-z))


def expert_ffn(X: np.ndarray, Wg: np.ndarray, Wu: np.ndarray, Wd: np.ndarray) -> np.ndarray:
    """SwiGLU expert: ``Y = (silu(X Wg^T) * (X Wu^T)) Wd^T`` in float64, no intermediate rounding."""
    G = X @ Wg.T
    U = X @ Wu.T
    return (silu(G) * U) @ Wd.T


def _expert_mats(weights: dict, e: int, g: int):
    """Expert e's gate, up and down matrices.  The format follows from the
    arrays present: per-group zero points ("<name>_zero": asymmetric 4-bit),
    fifth-bit words ("<name>_hi": 5-bit), neither (symmetric 4-bit)."""

    def one(name):
        zeros = weights.get(name + "_zero")
        zeros = None if zeros is None else zeros[e]
        hi = weights.get(name + "_hi")
        hi = None if hi is None else hi[e]
        return dequant(weights[name][e], weights[name + "_scale"][e], g, zeros=zeros, hi=hi)

    return one("gate"), one("up"), one("down")


def ffn_grouped(x_bf16, weights: dict, offsets, perm, k: int, g: int) -> np.ndarray:
    """Expert outputs for every routed pair, in grouped order: ``Y[i] = FFN_e(x[perm[i] // k])``.

    One batch per expert over the rows ``offsets[e]:offsets[e+1]``
    (kongchang.com hands-on, "Strata快在哪": tokens routed to an expert share
    its weights in one batch).  Returns float64 ``[T*k, H]``.
    """
    x = bf16_to_f64(x_bf16)
    E = len(offsets) - 1
    H = x.shape[1]
    Y = np.zeros((len(perm), H), dtype=np.float64)
    for e in range(E):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        if lo == hi:
            continue
        rows = np.asarray(perm[lo:hi]) // k
        Y[lo:hi] = expert_ffn(x[rows], *_expert_mats(weights, e, g))
    return Y


def combine(Y: np.ndarray, inv_perm, w: np.ndarray, k: int) -> np.ndarray:
    """``out[t] = sum_j w[t, j] * Y[inv_perm[t*k + j]]``, summed in j order, float64."""
    T = len(inv_perm) // k
    out = np.zeros((T, Y.shape[1]), dtype=np.float64)
    inv = np.asarray(inv_perm).reshape(T, k)
    for j in range(k):
        out += w[:, j : j + 1] * Y[inv[:, j]]
    return out


def moe_layer(logits, x_bf16, weights: dict, k: int, g: int) -> dict:
    """The whole layer: route, histogram, scan, permutation, grouped FFN, combine."""
    E = np.asarray(logits).shape[1]
    ids, w = route(logits, k)
    counts = histogram(ids, E)
    offsets = exclusive_scan(counts)
    perm, inv = permutation(ids)
    Y = ffn_grouped(x_bf16, weights, offsets, perm, k, g)
    out = combine(Y, inv, w, k)
    return dict(ids=ids, w=w, counts=counts, offsets=offsets, perm=perm, inv_perm=inv, y=Y, out=out)


def moe_out_tokens(tokens, ids, w, x_bf16, weights: dict, g: int) -> np.ndarray:
    """Layer output for a subset of tokens only (for outputs sampled from a large run).

    ``out[t] = sum_j w[t, j] * FFN_{ids[t, j]}(x[t])`` for each t in ``tokens``,
    dequantizing each needed expert once.  Same arithmetic as ``moe_layer``.
    """
    tokens = np.asarray(tokens, dtype=np.int64)
    x = bf16_to_f64(x_bf16)
    k = ids.shape[1]
    need: dict[int, list[tuple[int, int]]] = {}
    for r, t in enumerate(tokens):
        for j in range(k):
            need.setdefault(int(ids[t, j]), []).append((r, j))
    contrib = np.zeros((len(tokens), k, x.shape[1]), dtype=np.float64)
    for e, lst in need.items():
        rows = np.array([tokens[r] for r, _ in lst])
        Y = expert_ffn(x[rows], *_expert_mats(weights, e, g))
        for (r, j), yv in zip(lst, Y):
            contrib[r, j] = yv
    out = np.zeros((len(tokens), x.shape[1]), dtype=np.float64)
    for j in range(k):
        out += w[tokens, j][:, None] * contrib[:, j]
    return out
