"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Brute force on tiny inputs (pure-Python loops written independently of the
oracle's NumPy code), closed forms, invariants, special cases that reduce to a
textbook dense SwiGLU FFN, and the storage figures the pages print.  CPU only.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- routing
def _bruteforce_topk(row, k):
    """Repeated linear scan for the maximum; a strictly larger value replaces the
    current best, so the first (lowest) index wins among equal values."""
    remaining = list(range(len(row)))
    chosen = []
    for _ in range(k):
        best = remaining[0]
        for e in remaining[1:]:
            if float(row[e]) > float(row[best]):
                best = e
        chosen.append(best)
        remaining.remove(best)
    return chosen


def _bruteforce_softmax(vals):
    m = max(vals)
    z = [math.exp(v - m) for v in vals]
    s = sum(z)
    return [v / s for v in z]


# ----------------------------------------------------------------------------- router projection
def test_router_logits_match_bruteforce_loops():
    """x . W_r^T against explicit per-element loops over exactly widened bf16
    values, summed with math.fsum (exactly rounded)."""
    x, w = synth.make_router(3, 16, 5, seed=7)
    got = oracle.router_logits(x, w)

    def widen(b):
        return float(np.array([int(b) << 16], dtype=np.uint32).view(np.float32)[0])

    for t in range(3):
        for e in range(5):
            ref = math.fsum(widen(x[t, h]) * widen(w[e, h]) for h in range(16))
            assert abs(got[t, e] - ref) <= 1e-12 * max(1.0, abs(ref))


def test_router_logits_one_hot_rows_select_x():
    """A router row with a single 1.0 picks one hidden feature exactly."""
    x, _ = synth.make_router(4, 32, 1, seed=8)
    cols = [3, 0, 31, 17, 3]
    w = np.zeros((len(cols), 32), dtype=np.uint16)
    for e, c in enumerate(cols):
        w[e, c] = 0x3F80  # bf16 1.0
    got = oracle.router_logits(x, w)
    xf = oracle.bf16_to_f64(x)
    for e, c in enumerate(cols):
        assert np.array_equal(got[:, e], xf[:, c])


def test_router_logits_scale_exactly_with_router_rows():
    """Doubling every router weight (bf16 exponent + 1, exact) doubles the
    logits exactly, and negating a row negates its column."""
    x, w = synth.make_router(5, 64, 6, seed=9)
    base = oracle.router_logits(x, w)
    w2 = w.copy()
    nz = (w2 & 0x7F80) != 0
    w2[nz] = w2[nz] + 0x0080  # exponent + 1 on normal values (no overflow at these magnitudes)
    assert np.array_equal(oracle.router_logits(x, w2), 2 * base)
    wn = w.copy()
    wn[2] ^= 0x8000
    assert np.array_equal(oracle.router_logits(x, wn)[:, 2], -base[:, 2])


@pytest.mark.parametrize("grid", [None, 0.25, 1.0])
@pytest.mark.parametrize("T,E,k", [(7, 16, 2), (5, 33, 10), (3, 8, 8), (4, 64, 1)])
def test_route_matches_bruteforce(T, E, k, grid):
    rng = np.random.default_rng(100 + T * E + k)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    if grid is not None:  # coarse grid: many exact ties
        logits = (np.round(logits / grid) * grid).astype(np.float32)
    ids, w = oracle.route(logits, k)
    for t in range(T):
        want = _bruteforce_topk(logits[t], k)
        assert list(ids[t]) == want
        ww = _bruteforce_softmax([float(logits[t, e]) for e in want])
        np.testing.assert_allclose(w[t], ww, rtol=1e-14, atol=1e-15)


def test_route_all_equal_row():
    logits = np.full((3, 12), 0.5, np.float32)
    ids, w = oracle.route(logits, 5)
    assert (ids == np.arange(5)).all()
    np.testing.assert_allclose(w, 1.0 / 5, rtol=1e-15)


def test_route_signed_zero_is_a_tie():
    row = np.array([-0.0, 0.0, -0.0, 0.0, -1.0, -0.0], np.float32)
    ids, w = oracle.route(row[None, :], 4)
    assert list(ids[0]) == [0, 1, 2, 3]
    np.testing.assert_allclose(w[0], 0.25, rtol=1e-15)


def test_route_k1_is_argmax_weight_one():
    rng = np.random.default_rng(7)
    logits = rng.standard_normal((50, 40)).astype(np.float32)
    ids, w = oracle.route(logits, 1)
    assert (ids[:, 0] == np.argmax(logits, axis=1)).all()
    assert (w == 1.0).all()


def test_route_k_equals_E_is_full_softmax():
    import scipy.special

    rng = np.random.default_rng(8)
    logits = rng.standard_normal((6, 9)).astype(np.float32)
    ids, w = oracle.route(logits, 9)
    for t in range(6):
        assert list(ids[t]) == sorted(range(9), key=lambda e: (-float(logits[t, e]), e))
        full = scipy.special.softmax(logits[t].astype(np.float64))
        np.testing.assert_allclose(w[t], full[ids[t]], rtol=1e-13)


def test_route_k2_closed_form():
    rng = np.random.default_rng(9)
    logits = rng.standard_normal((40, 16)).astype(np.float32)
    ids, w = oracle.route(logits, 2)
    l0 = np.take_along_axis(logits, ids[:, :1], 1)[:, 0].astype(np.float64)
    l1 = np.take_along_axis(logits, ids[:, 1:2], 1)[:, 0].astype(np.float64)
    np.testing.assert_allclose(w[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-14)
    np.testing.assert_allclose(w.sum(1), 1.0, rtol=1e-15)


def test_route_weights_sum_to_one_and_descend():
    inp = synth.make_inputs("prefill512", with_weights=False)
    ids, w = oracle.route(inp.logits, inp.cfg.k)
    np.testing.assert_allclose(w.sum(1), 1.0, atol=1e-14)
    assert (np.diff(w, axis=1) <= 0).all()
    assert ((ids >= 0) & (ids < inp.cfg.E)).all()
    assert all(len(set(r)) == inp.cfg.k for r in ids)


# ----------------------------------------------------------------------------- grouping
def _bruteforce_grouping(ids, E):
    buckets = [[] for _ in range(E)]
    for p, e in enumerate(np.asarray(ids).reshape(-1).tolist()):
        buckets[e].append(p)
    counts = [len(b) for b in buckets]
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    perm = [p for b in buckets for p in b]
    return counts, offsets, perm


@pytest.mark.parametrize("name", ["tiny", "decode", "prefill512", "zipf6144"])
def test_grouping_matches_bruteforce_and_invariants(name):
    inp = synth.make_inputs(name, with_weights=False)
    cfg = inp.cfg
    ids, _ = oracle.route(inp.logits, cfg.k)
    counts = oracle.histogram(ids, cfg.E)
    offsets = oracle.exclusive_scan(counts)
    perm, inv = oracle.permutation(ids)
    bc, bo, bp = _bruteforce_grouping(ids, cfg.E)
    assert counts.tolist() == bc
    assert offsets.tolist() == bo
    assert perm.tolist() == bp
    P = cfg.T * cfg.k
    assert counts.sum() == P and offsets[-1] == P and offsets[0] == 0
    assert (np.sort(perm) == np.arange(P)).all()  # bijection
    assert (inv[perm] == np.arange(P)).all()
    flat = ids.reshape(-1)
    assert (np.diff(flat[perm]) >= 0).all()  # grouped by expert
    for e in range(cfg.E):
        seg = perm[offsets[e] : offsets[e + 1]]
        assert (np.diff(seg) > 0).all()  # ascending pair index inside a group
        assert (flat[seg] == e).all()


def test_grouping_zipf_is_skewed_with_empty_experts():
    inp = synth.make_inputs("zipf6144", with_weights=False)
    ids, _ = oracle.route(inp.logits, inp.cfg.k)
    counts = oracle.histogram(ids, inp.cfg.E)
    assert (counts == 0).sum() > 10
    assert counts.max() > 10 * inp.cfg.T * inp.cfg.k / inp.cfg.E


# ----------------------------------------------------------------------------- int4 format
def test_unpack_known_bytes():
    # byte = u_even | u_odd << 4, q = u - 8
    packed = np.array([[0x80, 0x0F, 0xF0, 0x78]], np.uint8)
    q = oracle.unpack_int4(packed)
    assert q.tolist() == [[-8, 0, 7, -8, -8, 7, 0, -1]]


def test_dequant_matches_elementwise_definition():
    rng = np.random.default_rng(11)
    N, K, g = 5, 32, 8
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.05, (N, K // g)).astype(np.float16)
    W = oracle.dequant(packed, scales, g)
    for n in range(N):
        for kk in range(K):
            byte = int(packed[n, kk >> 1])
            u = (byte >> 4) if kk & 1 else (byte & 15)
            assert W[n, kk] == (u - 8) * float(scales[n, kk // g])


def test_quantizer_bounds_and_zero_group():
    rng = np.random.default_rng(12)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    w[2, 64:96] = 0.0  # an all-zero group of 32
    packed, s = synth.quantize_int4_groups(w, 32)
    q = oracle.unpack_int4(packed).astype(np.float64).reshape(6, 4, 32)
    sf = s.astype(np.float64)[..., None]
    err = np.abs(w.astype(np.float64).reshape(6, 4, 32) - q * sf)
    assert (err <= sf / 2 * (1 + 2.0**-10) + 1e-30).all()
    nz = sf[..., 0] > 0
    assert (np.abs(q).max(axis=2)[nz] == 7).all()
    assert s[2, 2] == 0 and (q[2, 2] == 0).all()
    assert (packed.reshape(6, 4, 16)[2, 2] == 0x88).all()


def test_bf16_rounding_matches_torch():
    import torch

    rng = np.random.default_rng(13)
    a = np.concatenate([rng.standard_normal(10000).astype(np.float32),
                        np.array([1.0 + 2.0**-8, 1.0 + 3 * 2.0**-8, -0.0, 0.0, 3.0e38], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert (synth.bf16_bits_from_f32(a) == want).all()


def test_storage_ratio_matches_page_figure():
    fx = json.load(open(os.path.join(GOLDEN, "storage_ratio.json")))
    cfg = synth.config("prefill6144")
    assert cfg.g == fx["group"]
    ratio = synth.weight_bytes_per_expert(cfg) / (3 * cfg.H * cfg.I * 2)
    assert abs(ratio - fx["value"]) <= fx["abs_tol"]


def test_int4_model_bytes_match_page_figure():
    fx = json.load(open(os.path.join(GOLDEN, "int4_model_bytes.json")))
    n, g = fx["params"], fx["group"]
    total = n // 2 + 2 * (n // g)
    assert fx["low_bytes"] <= total <= fx["high_bytes"]


# ----------------------------------------------------------------------------- FFN math
def test_silu_values():
    z = np.array([0.0, 1.0, -1.0, 30.0, -30.0])
    s = oracle.silu(z)
    assert s[0] == 0.0
    assert abs(s[1] - 0.7310585786300049) < 1e-15
    assert abs(s[2] + 0.2689414213699951) < 1e-15
    assert abs(s[3] - 30.0) < 1e-10 and abs(s[4]) < 1e-11


def _tiny_cfg(**kw):
    base = dict(name="t", T=6, H=16, I=8, E=4, k=2, g=8, seed=21)
    base.update(kw)
    return synth.MoEConfig(**base)


def _bruteforce_dense_layer(inp):
    """Every token through every expert with explicit loops, masked by the
    brute-force top-k; no grouping or permutation code."""
    cfg, Wt = inp.cfg, inp.weights

    def deq(name, e):
        packed, sc = Wt[name][e], Wt[name + "_scale"][e]
        n, half = packed.shape
        out = [[0.0] * (2 * half) for _ in range(n)]
        for r in range(n):
            for c in range(half):
                b = int(packed[r, c])
                out[r][2 * c] = ((b & 15) - 8) * float(sc[r, (2 * c) // cfg.g])
                out[r][2 * c + 1] = ((b >> 4) - 8) * float(sc[r, (2 * c + 1) // cfg.g])
        return out

    mats = [(deq("gate", e), deq("up", e), deq("down", e)) for e in range(cfg.E)]
    xs = [[float(np.uint32(int(b) << 16).view(np.float32)) for b in row] for row in inp.x_bf16]
    out = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        chosen = _bruteforce_topk(inp.logits[t], cfg.k)
        wts = _bruteforce_softmax([float(inp.logits[t, e]) for e in chosen])
        gate_w = {e: wv for e, wv in zip(chosen, wts)}
        for e in range(cfg.E):
            Wg, Wu, Wd = mats[e]
            h = []
            for i in range(cfg.I):
                gsum = sum(Wg[i][c] * xs[t][c] for c in range(cfg.H))
                usum = sum(Wu[i][c] * xs[t][c] for c in range(cfg.H))
                h.append(gsum / (1.0 + math.exp(-gsum)) * usum)
            y = [sum(Wd[n][i] * h[i] for i in range(cfg.I)) for n in range(cfg.H)]
            mask = gate_w.get(e, 0.0)
            for n in range(cfg.H):
                out[t, n] += mask * y[n]
    return out


@pytest.mark.parametrize("kw", [{}, dict(E=5, k=3, T=7, seed=22), dict(E=3, k=3, seed=23)])
def test_layer_matches_bruteforce_dense(kw):
    inp = synth.make_inputs(_tiny_cfg(**kw))
    ref = _bruteforce_dense_layer(inp)
    got = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    scale = np.abs(ref).max()
    assert np.abs(got - ref).max() <= 1e-12 * scale


def test_single_expert_is_textbook_swiglu():
    import torch

    inp = synth.make_inputs(_tiny_cfg(E=1, k=1, T=9, H=32, I=16, seed=24))
    W = inp.weights

    def tdeq(name):
        p = torch.from_numpy(W[name][0].astype(np.int64))
        q = torch.stack([(p & 15) - 8, (p >> 4) - 8], dim=-1).reshape(p.shape[0], -1).double()
        s = torch.from_numpy(W[name + "_scale"][0].astype(np.float64))
        return q * s.repeat_interleave(inp.cfg.g, dim=1)

    x = torch.from_numpy(inp.x_bf16.view(np.int16).astype(np.int32)).bitwise_left_shift(16)
    x = x.to(torch.int32).view(torch.float32).double()
    ref = torch.nn.functional.silu(x @ tdeq("gate").T) * (x @ tdeq("up").T) @ tdeq("down").T
    got = oracle.moe_layer(inp.logits, inp.x_bf16, W, 1, inp.cfg.g)["out"]
    np.testing.assert_allclose(got, ref.numpy(), rtol=1e-12, atol=1e-14)


def test_zero_input_gives_zero_output():
    inp = synth.make_inputs(_tiny_cfg(seed=25))
    x0 = np.zeros_like(inp.x_bf16)
    out = oracle.moe_layer(inp.logits, x0, inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    assert (out == 0).all()


def test_doubling_down_scales_doubles_output_exactly():
    inp = synth.make_inputs(_tiny_cfg(seed=26))
    a = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    w2 = dict(inp.weights)
    w2["down_scale"] = (inp.weights["down_scale"].astype(np.float32) * 2).astype(np.float16)
    b = oracle.moe_layer(inp.logits, inp.x_bf16, w2, inp.cfg.k, inp.cfg.g)["out"]
    assert (b == 2 * a).all()


def test_token_permutation_permutes_outputs():
    inp = synth.make_inputs(_tiny_cfg(T=11, seed=27))
    a = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    pi = np.random.default_rng(1).permutation(11)
    b = oracle.moe_layer(inp.logits[pi], inp.x_bf16[pi], inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    np.testing.assert_allclose(b, a[pi], rtol=1e-12, atol=1e-15)


def test_expert_relabel_leaves_output_unchanged():
    inp = synth.make_inputs(_tiny_cfg(E=6, k=3, T=10, seed=28))
    a = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, inp.cfg.k, inp.cfg.g)["out"]
    sigma = np.random.default_rng(2).permutation(6)  # new expert e' = position of old
    logits = inp.logits[:, sigma]
    w2 = {n: v[sigma] for n, v in inp.weights.items()}
    b = oracle.moe_layer(logits, inp.x_bf16, w2, inp.cfg.k, inp.cfg.g)["out"]
    np.testing.assert_allclose(b, a, rtol=1e-12, atol=1e-15)


def test_sampled_tokens_match_full_layer():
    inp = synth.make_inputs("tiny")
    cfg = inp.cfg
    full = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    toks = np.array([0, 5, 17, 63])
    part = oracle.moe_out_tokens(toks, full["ids"], full["w"], inp.x_bf16, inp.weights, cfg.g)
    np.testing.assert_allclose(part, full["out"][toks], rtol=1e-12, atol=1e-15)


def test_grouped_rows_are_per_pair_expert_outputs():
    inp = synth.make_inputs("tiny")
    cfg = inp.cfg
    r = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    # grouped row i is FFN_{ids[p]}(x[p // k]) for p = perm[i]: check one row per expert
    for e in range(cfg.E):
        lo, hi = r["offsets"][e], r["offsets"][e + 1]
        if lo == hi:
            continue
        p = int(r["perm"][lo])
        one = oracle.moe_out_tokens([p // cfg.k], r["ids"][:, :], np.eye(cfg.k)[None].repeat(cfg.T, 0)[:, p % cfg.k],
                                    inp.x_bf16, inp.weights, cfg.g)
        np.testing.assert_allclose(r["y"][lo], one[0], rtol=1e-12, atol=1e-15)


# ----------------------------------------------------------------------------- other weight formats
def test_asym_dequant_hand_decoded():
    # u = 1, 2 | 0, 15; zero points 3 (group 0), 5 (group 1); scales 0.5, 2.
    packed = np.array([[0x21, 0xF0]], np.uint8)
    zeros = np.array([[0x53]], np.uint8)
    scales = np.array([[0.5, 2.0]], np.float16)
    W = oracle.dequant(packed, scales, 2, zeros=zeros)
    assert W.tolist() == [[-1.0, -0.5, -10.0, 20.0]]


def test_int5_dequant_hand_decoded():
    # all nibbles 0; fifth bits set for elements 19 (= 8*2 + 3: bit 4*3 + 2)
    # and 15 (= 8*1 + 7: bit 4*7 + 1), so q = -16 except q[19] = q[15] = 0.
    packed = np.zeros((1, 16), np.uint8)
    hi = np.array([[(1 << 14) | (1 << 29)]], np.uint32)
    W = oracle.dequant(packed, np.array([[1.0]], np.float16), 32, hi=hi)
    want = [-16.0] * 32
    want[19] = want[15] = 0.0
    assert W.tolist() == [want]


def test_other_formats_match_elementwise_definition():
    rng = np.random.default_rng(14)
    N, K, g = 3, 64, 16
    packed = rng.integers(0, 256, (N, K // 2), dtype=np.uint8)
    scales = rng.uniform(0.001, 0.05, (N, K // g)).astype(np.float16)
    zeros = rng.integers(0, 256, (N, K // g // 2), dtype=np.uint8)
    hi = rng.integers(0, 2**32, (N, K // 32), dtype=np.uint64).astype(np.uint32)
    Wa = oracle.dequant(packed, scales, g, zeros=zeros)
    W5 = oracle.dequant(packed, scales, g, hi=hi)
    for n in range(N):
        for kk in range(K):
            byte = int(packed[n, kk >> 1])
            u = (byte >> 4) if kk & 1 else (byte & 15)
            grp = kk // g
            zbyte = int(zeros[n, grp >> 1])
            z = (zbyte >> 4) if grp & 1 else (zbyte & 15)
            s = float(scales[n, grp])
            assert Wa[n, kk] == (u - z) * s
            word = int(hi[n, kk // 32])
            c, i = (kk % 32) // 8, kk % 8
            b = (word >> (4 * i + c)) & 1
            assert W5[n, kk] == (u + 16 * b - 16) * s


def test_asym_quantizer_bounds():
    rng = np.random.default_rng(15)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    w[1, :32] = np.abs(w[1, :32]) + 0.01   # an all-positive group
    w[2, 64:96] = 0.0                      # an all-zero group
    w[3, 32:64] = -0.03                    # a constant negative group
    packed, s, zeros = synth.quantize_int4_asym_groups(w, 32)
    W = oracle.dequant(packed, s, 32, zeros=zeros).reshape(6, 4, 32)
    sf = s.astype(np.float64)[..., None]
    err = np.abs(w.astype(np.float64).reshape(6, 4, 32) - W)
    assert (err <= sf * (1 + 2.0**-9) + 1e-30).all()
    assert s[2, 2] == 0 and (W[2, 2] == 0).all()
    assert np.abs(W[3, 1] + 0.03).max() <= float(s[3, 1]) / 2 + 1e-9


def test_int5_quantizer_bounds():
    rng = np.random.default_rng(16)
    w = (rng.standard_normal((6, 128)) * 0.02).astype(np.float32)
    w[4, :64] = 0.0
    packed, s, hi = synth.quantize_int5_groups(w, 64)
    W = oracle.dequant(packed, s, 64, hi=hi).reshape(6, 2, 64)
    sf = s.astype(np.float64)[..., None]
    err = np.abs(w.astype(np.float64).reshape(6, 2, 64) - W)
    assert (err <= sf / 2 * (1 + 2.0**-10) + 1e-30).all()
    q = np.rint(np.where(sf > 0, W / np.where(sf > 0, sf, 1), 0))
    nz = sf[..., 0] > 0
    assert (np.abs(q).max(axis=2)[nz] >= 15).all()
    assert s[4, 0] == 0 and (W[4, 0] == 0).all()


def test_asym_model_bytes_match_page_figure():
    """The lqnn.cn review §3.1: 4-bit weights with a scale and a zero point per
    group come to 2.2-2.4 GB for 4B parameters (10-20 % over 0.5 byte per
    parameter): fp16 scale + 4-bit zero point per 32 weights."""
    fx = json.load(open(os.path.join(GOLDEN, "int4_model_bytes.json")))
    n = fx["params"]
    total = n // 2 + n // 32 * 2 + n // 32 // 2
    assert fx["low_bytes"] <= total <= fx["high_bytes"]
    assert 0.10 <= (total - n / 2) / (n / 2) <= 0.20


@pytest.mark.parametrize("fmt", ["int4_asym", "int5"])
def test_layer_matches_bruteforce_dense_other_formats(fmt):
    inp = synth.make_inputs(_tiny_cfg(H=64, I=32, g=16, fmt=fmt, seed=25))
    cfg = inp.cfg
    Wt = inp.weights

    def deq(name, e):
        packed, sc = Wt[name][e], Wt[name + "_scale"][e]
        n, half = packed.shape
        out = [[0.0] * (2 * half) for _ in range(n)]
        for r in range(n):
            for kk in range(2 * half):
                b = int(packed[r, kk // 2])
                u = (b >> 4) if kk % 2 else (b & 15)
                grp = kk // cfg.g
                if fmt == "int4_asym":
                    zb = int(Wt[name + "_zero"][e][r, grp // 2])
                    q = u - ((zb >> 4) if grp % 2 else (zb & 15))
                else:
                    word = int(Wt[name + "_hi"][e][r, kk // 32])
                    q = u + 16 * ((word >> (4 * (kk % 8) + (kk % 32) // 8)) & 1) - 16
                out[r][kk] = q * float(sc[r, grp])
        return out

    mats = [(deq("gate", e), deq("up", e), deq("down", e)) for e in range(cfg.E)]
    xs = [[float(np.uint32(int(b) << 16).view(np.float32)) for b in row] for row in inp.x_bf16]
    ref = np.zeros((cfg.T, cfg.H))
    for t in range(cfg.T):
        chosen = _bruteforce_topk(inp.logits[t], cfg.k)
        wts = _bruteforce_softmax([float(inp.logits[t, e]) for e in chosen])
        for e, wv in zip(chosen, wts):
            Wg, Wu, Wd = mats[e]
            h = []
            for i in range(cfg.I):
                gs = sum(Wg[i][c] * xs[t][c] for c in range(cfg.H))
                us = sum(Wu[i][c] * xs[t][c] for c in range(cfg.H))
                h.append(gs / (1.0 + math.exp(-gs)) * us)
            for n_ in range(cfg.H):
                ref[t, n_] += wv * sum(Wd[n_][i] * h[i] for i in range(cfg.I))
    got = oracle.moe_layer(inp.logits, inp.x_bf16, Wt, cfg.k, cfg.g)["out"]
    assert np.abs(got - ref).max() <= 1e-12 * np.abs(ref).max()
