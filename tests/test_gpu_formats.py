"""GPU parity of the two other weight formats, asymmetric 4-bit (scale and
zero point per group) and symmetric 5-bit blocks, through the C ABI, against
the fp64 oracle's dequantization (oracle.dequant with zero points or fifth-bit
words).

* Small ragged shapes on the grouped-GEMM path (several tiles and a partial
  tile per expert) and on the decode (GEMV) path, in both combine modes; every
  element of y and out.
* Codes, zero points and fifth bits drawn uniformly over all their bit
  patterns (every nibble, every zero point 0..15, every fifth bit), so no
  code value goes untested.
* The 6144-token prefill chunk (H 2048, I 512, 512 experts, top-10, g 64) in
  each format through the single layer call the benchmark times, every
  output element; the 4-token decode step in each format (the two-kernel
  decode layer), and the GEMV shapes through both combine modes.

Tolerances are those of the symmetric format (the same fp16-operand and
fp32-accumulation envelope): max |err| <= 2e-2 RMS(out), sum |err| / sum |out|
<= 5e-3.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from moe_testutil import W_ATOL, check_close, inputs, to_device

pytestmark = pytest.mark.gpu

FORMATS = ["int4_asym", "int5"]


@pytest.fixture(scope="module")
def qe(gpu_available):
    import quantized_expert_ffn_histogram_amd as qe

    qe.load()
    return qe


def _np(t):
    return t.detach().cpu().numpy()


def _small_cfgs(fmt):
    return [
        synth.MoEConfig(f"ragged64_{fmt}", T=400, H=512, I=256, E=4, k=2, g=64, seed=51, fmt=fmt),
        synth.MoEConfig(f"ragged32_{fmt}", T=333, H=768, I=384, E=5, k=3, g=32, seed=52, fmt=fmt),
        synth.MoEConfig(f"ragged128_{fmt}", T=260, H=1024, I=256, E=3, k=1, g=128, seed=53, fmt=fmt),
        synth.MoEConfig(f"many_{fmt}", T=96, H=256, I=128, E=64, k=6, g=32, seed=54, fmt=fmt),
    ]


def _gemv_cfgs(fmt):
    return [
        synth.MoEConfig(f"gemv_tiny_{fmt}", T=16, H=256, I=128, E=16, k=2, g=32, seed=61, fmt=fmt),
        synth.MoEConfig(f"gemv_t1_{fmt}", T=1, H=2048, I=512, E=64, k=10, g=64, seed=62, fmt=fmt),
        synth.MoEConfig(f"gemv_wide_{fmt}", T=8, H=4096, I=1024, E=32, k=8, g=128, seed=63, fmt=fmt),
    ]


def _all_patterns(inp, seed):
    """The same layer with every weight byte, zero point and fifth bit drawn
    uniformly, and scales small enough to keep h and y inside fp16."""
    cfg = inp.cfg
    rng = np.random.default_rng(seed)
    E, H, I, g = cfg.E, cfg.H, cfg.I, cfg.g
    w = {}
    for name, n, kdim in (("gate", I, H), ("up", I, H), ("down", H, I)):
        w[name] = rng.integers(0, 256, (E, n, kdim // 2), dtype=np.uint8)
        w[name + "_scale"] = rng.uniform(5e-4, 2e-3, (E, n, kdim // g)).astype(np.float16)
        if cfg.fmt == "int4_asym":
            w[name + "_zero"] = rng.integers(0, 256, (E, n, kdim // g // 2), dtype=np.uint8)
        else:
            w[name + "_hi"] = rng.integers(0, 1 << 32, (E, n, kdim // 32), dtype=np.uint32)
    return dataclasses.replace(inp, weights=w)


def _layer(qe, inp, fused):
    logits, x, ex = to_device(inp)
    assert ex.fmt == inp.cfg.fmt
    return qe.moe_layer(logits, x, ex, inp.cfg.k, fused=fused)


def _compare(qe, inp, what):
    cfg = inp.cfg
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    det = _layer(qe, inp, fused=False)
    check_close(_np(det["y"]), ref["y"], f"{what} y")
    check_close(_np(det["out"]), ref["out"], f"{what} out (deterministic)")
    fus = _layer(qe, inp, fused=True)
    check_close(_np(fus["out"]), ref["out"], f"{what} out (fused)")


@pytest.mark.parametrize("path", ["gemm", "auto"])
@pytest.mark.parametrize("cfg", _small_cfgs("int4_asym") + _small_cfgs("int5"), ids=lambda c: c.name)
def test_format_grouped_gemm_ragged(qe, cfg, path, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    _compare(qe, inputs(cfg), cfg.name)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("cfg", _gemv_cfgs("int4_asym") + _gemv_cfgs("int5"), ids=lambda c: c.name)
def test_format_decode_paths(qe, cfg, path, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    _compare(qe, inputs(cfg), cfg.name)


@pytest.mark.parametrize("path", ["gemm", "gemv"])
@pytest.mark.parametrize("fmt", FORMATS)
def test_format_every_bit_pattern(qe, fmt, path, monkeypatch):
    """Uniformly drawn codes, zero points and fifth bits on both paths."""
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    T = 300 if path == "gemm" else 12
    cfg = synth.MoEConfig(f"patterns_{fmt}", T=T, H=512, I=256, E=6, k=3, g=32, seed=71, fmt=fmt)
    _compare(qe, _all_patterns(inputs(cfg), 72), cfg.name)


def _check_routing(res, ref):
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        assert (_np(res[key]).reshape(-1) == ref[key].reshape(-1)).all(), key
    assert np.abs(_np(res["w"]).astype(np.float64) - ref["w"]).max() <= W_ATOL


@pytest.mark.parametrize("name", ["decode_asym", "decode_int5"])
def test_format_decode_layer_call(qe, name):
    """strata_moe_layer on a decode step runs the two-kernel decode layer in
    the other formats too."""
    inp = inputs(name)
    cfg = inp.cfg
    logits, x, ex = to_device(inp)
    qe.timing_enable(True)
    res = qe.layer(logits, x, ex, cfg.k)
    names = qe.timing_kernels()
    qe.timing_enable(False)
    assert "decode_route_gateup" in names and "decode_down_combine" in names, names
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    _check_routing(res, ref)
    check_close(_np(res["out"]), ref["out"], f"{name} out")


@pytest.mark.parametrize("name", ["prefill6144_asym", "prefill6144_int5"])
def test_format_layer_call_full_size(qe, name):
    """The benchmark's single layer call on the 6144-token chunk, every
    output element against the oracle's full layer."""
    import torch

    inp = inputs(name)
    cfg = inp.cfg
    logits, x, ex = to_device(inp)
    run = qe.LayerRunner(ex, cfg.T, cfg.E, cfg.k, fused=True, single_call=True)
    print(f"[formats] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g} {cfg.fmt}", flush=True)
    run(logits, x)
    torch.cuda.synchronize()
    res = dict(ids=run.ids, w=run.w, counts=run.counts, offsets=run.offsets, perm=run.perm, inv_perm=run.inv)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    _check_routing(res, ref)
    stats = check_close(_np(run.out), ref["out"], f"{name} out (all {cfg.T * cfg.H} elements)")
    print(f"[formats] {name}: {stats}", flush=True)


@pytest.mark.parametrize("cfg", _gemv_cfgs("int4_asym") + _gemv_cfgs("int5"), ids=lambda c: c.name)
def test_format_decode_layer_shapes(qe, cfg):
    """The two-kernel decode layer on the GEMV shapes (T = 16, 1, 8; H up to
    4096), and on every bit pattern of codes, zero points and fifth bits."""
    for inp in (inputs(cfg), _all_patterns(inputs(cfg), 73)):
        logits, x, ex = to_device(inp)
        qe.timing_enable(True)
        res = qe.layer(logits, x, ex, cfg.k)
        names = qe.timing_kernels()
        qe.timing_enable(False)
        assert "decode_route_gateup" in names, names
        ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
        _check_routing(res, ref)
        check_close(_np(res["out"]), ref["out"], f"{cfg.name} out")
