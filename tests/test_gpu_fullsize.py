"""GPU parity of the whole-layer call at the full workload sizes, element by
element, plus the ends of the supported envelope.

* ``strata_moe_layer`` exactly as the benchmark times it (one call, fused
  combine, preallocated outputs and workspace) on the four 6144-token
  workloads: routing ids, counts, offsets, perm and inv_perm bit-exact, the
  routing weights within 1e-6, and every element of ``out`` within the output
  tolerance of the fp64 oracle's full layer.
* The general GEMM pipeline on an A operand of more than 4 GiB (row offsets
  past 2^32 bytes), on sampled tokens above and below that boundary.
* The fp16 operand envelope: activations near the fp16 maximum and below the
  smallest fp16 normal, with h and the expert outputs inside fp16's range.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from moe_testutil import W_ATOL, check_close, inputs, to_device

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def qe(gpu_available):
    import quantized_expert_ffn_histogram_amd as qe

    qe.load()
    return qe


def _np(t):
    return t.detach().cpu().numpy()


def _check_routing(res, ref):
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        got = _np(res[key]).reshape(-1)
        assert got.shape == ref[key].reshape(-1).shape, key
        assert (got == ref[key].reshape(-1)).all(), f"{key} differs from the oracle"
    w = _np(res["w"]).astype(np.float64)
    assert np.abs(w - ref["w"]).max() <= W_ATOL
    assert np.abs(w.sum(1) - 1.0).max() <= W_ATOL


@pytest.mark.parametrize("name", ["prefill6144", "zipf6144", "prefill6144_g32", "prefill6144_g128"])
def test_layer_call_full_size_every_element(qe, name):
    """The benchmark's step (LayerRunner, single strata_moe_layer call) on the
    full workload, every output element against the oracle's full layer."""
    import torch

    inp = inputs(name)
    cfg = inp.cfg
    logits, x, ex = to_device(inp)
    run = qe.LayerRunner(ex, cfg.T, cfg.E, cfg.k, fused=True, single_call=True)
    print(f"[full-size] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g}", flush=True)
    run(logits, x)
    torch.cuda.synchronize()
    res = dict(ids=run.ids, w=run.w, counts=run.counts, offsets=run.offsets, perm=run.perm, inv_perm=run.inv,
               out=run.out)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    _check_routing(res, ref)
    stats = check_close(_np(run.out), ref["out"], f"{name} out (all {cfg.T * cfg.H} elements)")
    print(f"[full-size] {name}: {stats}", flush=True)
    # A second call on the same buffers gives the same bits.
    first = run.out.clone()
    run(logits, x)
    torch.cuda.synchronize()
    assert torch.equal(first, run.out)


def test_general_pipeline_a_operand_beyond_4gib(qe):
    """Gate/up GEMM whose A operand (x as fp16, T x H) spans more than 2^32
    bytes: T = 140000 tokens at H = 16384 is 4.59 GB, so rows from 131072 on
    start past 2^32 bytes and run on the general pipeline with 64-bit row
    addresses.  x repeats a block of 1021 distinct rows (131072 mod 1021 =
    384, so a row offset that wrapped at 2^32 would read a different row);
    tokens on both sides of the boundary are compared with the oracle."""
    import torch

    T, H, I, E, k, g = 140000, 16384, 128, 2, 1, 64
    assert T * H * 2 > 2 ** 32 and (131072 % 1021) != 0
    cfg = synth.MoEConfig("beyond4g", T=T, H=H, I=I, E=E, k=k, g=g, seed=71)
    small = synth.make_inputs(dataclasses.replace(cfg, T=1021))
    x_bf16 = np.tile(small.x_bf16, ((T + 1020) // 1021, 1))[:T]
    logits = synth.make_logits(cfg, np.random.SeedSequence([71, 1]))
    dev = torch.device("cuda:0")
    ex = qe.QuantizedExperts.from_numpy(small.weights, g, dev)
    lg = torch.from_numpy(logits).to(dev)
    xd = torch.from_numpy(x_bf16.view(np.int16)).to(dev).view(torch.bfloat16)
    print(f"[beyond4g] T={T} H={H}: A operand {T * H * 2 / 2 ** 30:.2f} GiB", flush=True)
    res = qe.layer(lg, xd, ex, k)
    torch.cuda.synchronize()
    ids, w = oracle.route(logits, k)
    assert (_np(res["ids"]) == ids).all()
    boundary = 2 ** 32 // (2 * H)  # first token row at or past 2^32 bytes
    toks = np.array(sorted({0, 1, 1020, boundary - 1, boundary, boundary + 1, boundary + 383, boundary + 384,
                            T - 2, T - 1} | set(np.random.default_rng(5).integers(boundary, T, 12).tolist())))
    ref = oracle.moe_out_tokens(np.arange(len(toks)), ids[toks], w[toks], x_bf16[toks], small.weights, g)
    out = _np(res["out"][torch.from_numpy(toks).to(dev)])
    check_close(out, ref, "out at tokens around the 2^32-byte boundary")
    del res, xd, ex
    torch.cuda.empty_cache()


def _envelope_inputs(T, seed):
    """x: N(0, 1), one in four tokens with one entry near the fp16 maximum
    (61440 or 65280, random sign) and about 30 % of entries replaced by
    magnitudes in [2^-24, 2^-15] (below the smallest fp16 normal, 2^-14);
    weights drawn with standard deviation 0.0005 so that h and the expert
    outputs stay inside fp16's range."""
    cfg = synth.MoEConfig("fp16_envelope", T=T, H=512, I=256, E=4, k=2, g=64, seed=seed, weight_std=0.0005)
    inp = synth.make_inputs(cfg)
    rng = np.random.default_rng(seed)
    x = oracle.bf16_to_f64(inp.x_bf16)
    tiny = rng.random(x.shape) < 0.3
    mags = 2.0 ** rng.uniform(-24, -15, x.shape)
    x = np.where(tiny, np.sign(rng.standard_normal(x.shape)) * mags, x)
    big_tok = np.arange(0, T, 4)
    big_col = rng.integers(0, cfg.H, len(big_tok))
    x[big_tok, big_col] = rng.choice([-65280.0, -61440.0, 61440.0, 65280.0], len(big_tok))
    inp.x_bf16 = synth.bf16_bits_from_f32(x.astype(np.float32))
    return inp


def _fp16_precondition(inp):
    """Largest |h| and |y| the layer produces on these inputs (fp64)."""
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, inp.cfg.k, inp.cfg.g)
    x = oracle.bf16_to_f64(inp.x_bf16)
    hmax = 0.0
    for e in range(inp.cfg.E):
        lo, hi = int(ref["offsets"][e]), int(ref["offsets"][e + 1])
        if lo == hi:
            continue
        X = x[ref["perm"][lo:hi] // inp.cfg.k]
        G = X @ oracle.dequant(inp.weights["gate"][e], inp.weights["gate_scale"][e], inp.cfg.g).T
        U = X @ oracle.dequant(inp.weights["up"][e], inp.weights["up_scale"][e], inp.cfg.g).T
        hmax = max(hmax, float(np.abs(oracle.silu(G) * U).max()))
    return ref, hmax, float(np.abs(ref["y"]).max())


@pytest.mark.parametrize("T,path", [(600, "auto"), (600, "gemm"), (4, "auto"), (4, "gemv")])
def test_fp16_operand_envelope(qe, T, path, monkeypatch):
    """Activations at both ends of the fp16 operand envelope: entries near
    +-6e4 and below 2^-14 (kept as fp16 subnormals), on the grouped-GEMM
    path (T = 600, 1200 pairs) and on the decode paths (T = 4), through the
    layer call and both combine modes of the separate calls."""
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    inp = _envelope_inputs(T, 81 + T)
    ref, hmax, ymax = _fp16_precondition(inp)
    x = oracle.bf16_to_f64(inp.x_bf16)
    assert np.abs(x).max() >= 61440 and np.abs(x).max() <= 65504
    assert ((np.abs(x) < 2.0 ** -14) & (x != 0)).mean() > 0.2
    assert hmax < 65504 and ymax < 65504, (hmax, ymax)  # inside the precondition
    logits, xd, ex = to_device(inp)
    res = qe.layer(logits, xd, ex, inp.cfg.k)
    _check_routing(res, ref)
    check_close(_np(res["out"]), ref["out"], f"layer out (h max {hmax:.0f}, y max {ymax:.0f})")
    for fused in (True, False):
        r2 = qe.moe_layer(logits, xd, ex, inp.cfg.k, fused=fused)
        check_close(_np(r2["out"]), ref["out"], f"four-call out (fused={fused})")
