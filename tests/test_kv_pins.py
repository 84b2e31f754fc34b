"""CPU pins of the KV-cache codec and sparse-attention oracle (oracle/kv.py).

Each check ties the oracle to something other than itself: a hand-decoded
worked example, the pages' printed cache sizes (tests/golden), closed forms
(a single selected row, zero queries), invariances, a textbook attention
routine from torch on the full selection, and brute-force loops.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(vals):
    return synth.bf16_bits_from_f32(np.asarray(vals, dtype=np.float32))


def test_kv_quantize_hand_decoded_example():
    # max |x| = 7 -> s = 1; 3.5, 2.5 and -3.5 round half to even: 4, 2, -4.
    x = _bf16([[7.0, -7.0, 3.5, 0.0, 1.0, -1.0, 2.5, -3.5]])
    packed, scale = oracle.kv_quantize(x)
    assert scale.dtype == np.float16 and float(scale[0]) == 1.0
    # u = q + 8 = 15, 1, 12, 8, 9, 7, 10, 4; byte = u_even | u_odd << 4
    assert packed[0].tolist() == [0x1F, 0x8C, 0x79, 0x4A]
    assert oracle.kv_dequant(packed, scale)[0].tolist() == [7.0, -7.0, 4.0, 0.0, 1.0, -1.0, 2.0, -4.0]


def test_kv_quantize_zero_vector():
    packed, scale = oracle.kv_quantize(np.zeros((3, 16), np.uint16))
    assert (scale == 0).all() and (packed == 0x88).all()
    assert (oracle.kv_dequant(packed, scale) == 0).all()


def test_kv_quantize_error_bound_and_full_range():
    rng = np.random.default_rng(5)
    x = _bf16(rng.standard_normal((200, 128)) * rng.uniform(0.01, 100, (200, 1)))
    packed, scale = oracle.kv_quantize(x)
    xf = oracle.bf16_to_f64(x)
    d = oracle.kv_dequant(packed, scale)
    s = scale.astype(np.float64)[:, None]
    assert (np.abs(xf - d) <= s / 2 * (1 + 2.0 ** -10) + 1e-300).all()
    q = np.rint(d / s)
    assert (np.abs(q).max(axis=1) == 7).all()  # every row uses the code range
    assert (np.abs(d - q * s) == 0).all()


def test_kv_quantize_scaling_and_sign():
    rng = np.random.default_rng(6)
    x = _bf16(rng.standard_normal((50, 64)))
    p1, s1 = oracle.kv_quantize(x)
    p2, s2 = oracle.kv_quantize(_bf16(oracle.bf16_to_f64(x) * 2))
    assert (s2.astype(np.float64) == 2 * s1.astype(np.float64)).all() and (p1 == p2).all()
    p3, s3 = oracle.kv_quantize(x ^ np.uint16(0x8000))  # negate every element
    assert (s3 == s1).all()
    d1, d3 = oracle.kv_dequant(p1, s1), oracle.kv_dequant(p3, s3)
    assert (d3 == -d1).all()


def test_kv_dequant_matches_elementwise_definition():
    rng = np.random.default_rng(7)
    packed = rng.integers(0, 256, (3, 4), dtype=np.uint8)
    scale = np.array([0.5, 3.0, -0.25], np.float16)
    d = oracle.kv_dequant(packed, scale)
    for r in range(3):
        for j in range(4):
            b = int(packed[r, j])
            assert d[r, 2 * j] == ((b & 15) - 8) * float(scale[r])
            assert d[r, 2 * j + 1] == ((b >> 4) - 8) * float(scale[r])


def test_cache_bytes_match_page_figures():
    g = json.load(open(os.path.join(GOLDEN, "kv_cache_bytes.json")))
    L, D = g["layers"], g["head_dim"]
    fp = g["fp16_bytes_per_token"]
    assert oracle.kv_bytes_per_token(L, 8, D, 16) == fp["kv_heads_8"]
    assert oracle.kv_bytes_per_token(L, 32, D, 16) == fp["kv_heads_32_mha"]
    assert oracle.kv_bytes_per_token(L, 1, D, 16) == fp["kv_heads_1_mqa"]
    assert abs(8192 * oracle.kv_bytes_per_token(L, 8, D, 16) / g["fp16_context_8k_bytes_approx"] - 1) < 0.1
    mb = 1000 * oracle.kv_bytes_per_token(L, 8, D, 4) / 1e6
    lo, hi = g["four_bit_mb_per_1000_tokens_range"]
    assert lo <= mb <= hi, mb


def _cache(inp):
    kp, ks = oracle.kv_quantize(inp.k_bf16)
    vp, vs = oracle.kv_quantize(inp.v_bf16)
    return kp, ks, vp, vs


def test_sparse_attention_full_selection_is_textbook_attention():
    """Selecting every position is dense attention: torch's scaled dot-product
    attention (fp64, CPU) on the dequantized cache, KV heads repeated."""
    torch = pytest.importorskip("torch")
    inp = synth.make_attn_inputs("attn_small", L=96, n_sel=96, Tq=2)
    cfg = inp.cfg
    kp, ks, vp, vs = _cache(inp)
    sel = np.tile(np.arange(cfg.L, dtype=np.int32), (cfg.Tq, 1))
    got = oracle.sparse_attention(inp.q_bf16, kp, ks, vp, vs, sel, cfg.sm_scale)
    G = cfg.Hq // cfg.Hkv
    K = torch.from_numpy(oracle.kv_dequant(kp, ks)).permute(1, 0, 2).repeat_interleave(G, 0)  # [Hq, L, D]
    V = torch.from_numpy(oracle.kv_dequant(vp, vs)).permute(1, 0, 2).repeat_interleave(G, 0)
    Q = torch.from_numpy(oracle.bf16_to_f64(inp.q_bf16)).permute(1, 0, 2)  # [Hq, Tq, D]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=cfg.sm_scale).permute(1, 0, 2).numpy()
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()


def test_sparse_attention_single_row_and_zero_query():
    inp = synth.make_attn_inputs("attn_small", L=64, n_sel=10, Tq=2)
    cfg = inp.cfg
    kp, ks, vp, vs = _cache(inp)
    one = inp.sel[:, :1]
    out = oracle.sparse_attention(inp.q_bf16, kp, ks, vp, vs, one, cfg.sm_scale)
    V = oracle.kv_dequant(vp, vs)
    G = cfg.Hq // cfg.Hkv
    for t in range(cfg.Tq):
        for h in range(cfg.Hq):
            assert (out[t, h] == V[one[t, 0], h // G]).all()
    zq = np.zeros_like(inp.q_bf16)
    out0 = oracle.sparse_attention(zq, kp, ks, vp, vs, inp.sel, cfg.sm_scale)
    for t in range(cfg.Tq):
        for h in range(cfg.Hq):
            mean = V[inp.sel[t], h // G].mean(axis=0)
            assert np.abs(out0[t, h] - mean).max() <= 1e-13 * max(np.abs(mean).max(), 1)


def test_sparse_attention_selection_order_does_not_matter():
    inp = synth.make_attn_inputs("attn_small", L=200, n_sel=37, Tq=2)
    cfg = inp.cfg
    kp, ks, vp, vs = _cache(inp)
    a = oracle.sparse_attention(inp.q_bf16, kp, ks, vp, vs, inp.sel, cfg.sm_scale)
    shuffled = np.stack([np.random.default_rng(t).permutation(r) for t, r in enumerate(inp.sel)])
    b = oracle.sparse_attention(inp.q_bf16, kp, ks, vp, vs, shuffled, cfg.sm_scale)
    assert np.abs(a - b).max() <= 1e-13 * np.abs(a).max()


def test_sparse_attention_bruteforce_loops():
    """Pure-Python loops (math.exp) on a tiny case: 1 query, 4 heads over 2 KV
    heads, head_dim 4, 3 selected rows."""
    rng = np.random.default_rng(9)
    q = _bf16(rng.standard_normal((1, 4, 4)))
    k = _bf16(rng.standard_normal((6, 2, 4)))
    v = _bf16(rng.standard_normal((6, 2, 4)))
    kp, ks = oracle.kv_quantize(k)
    vp, vs = oracle.kv_quantize(v)
    sel = np.array([[4, 0, 2]], np.int32)
    got = oracle.sparse_attention(q, kp, ks, vp, vs, sel, 0.5)
    qf = oracle.bf16_to_f64(q)
    Kd, Vd = oracle.kv_dequant(kp, ks), oracle.kv_dequant(vp, vs)
    for h in range(4):
        g = h // 2
        sc = [0.5 * sum(qf[0, h, d] * Kd[p, g, d] for d in range(4)) for p in (4, 0, 2)]
        m = max(sc)
        e = [math.exp(s - m) for s in sc]
        z = sum(e)
        for d in range(4):
            ref = sum(e[i] / z * Vd[p, g, d] for i, p in enumerate((4, 0, 2)))
            assert abs(got[0, h, d] - ref) <= 1e-13
