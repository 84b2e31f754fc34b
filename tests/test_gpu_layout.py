"""GPU checks of the tiled weight layout (STRATA_L_TILED).

* strata_moe_tile_weights against the layout's definition in the header,
  written out with numpy index arithmetic: every byte, several shapes.
* Every path that reads packed codes (the grouped GEMM's wide and general
  pipelines, the GEMV path, the two-kernel decode layer, the single layer
  call, its no-allocation variant) in all three weight formats: the outputs
  with tiled codes equal those with row-major codes bit for bit (the kernels
  read the same values and do the same arithmetic; only addresses differ),
  and match the fp64 oracle within the layer tolerance.
* The 6144-token prefill chunk in each format and the skewed 6144-token
  layer through the benchmark's single layer call: tiled equals row-major
  on every output element.
* The envelope's edges through the layer call: 1024 experts on the grouped
  GEMM and the decode paths, gate/up rows of K = 8192 and down rows of
  K = 16384 (a block's last tile ends at the end of its buffer range).
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from moe_testutil import check_close, inputs, to_device

pytestmark = pytest.mark.gpu

FORMATS = ["int4", "int4_asym", "int5"]


@pytest.fixture(scope="module")
def qe(gpu_available):
    import quantized_expert_ffn_histogram_amd as qe

    qe.load()
    return qe


def _np(t):
    return t.detach().cpu().numpy()


def _tiled_by_definition(packed: np.ndarray) -> np.ndarray:
    """Byte j of row r (r over all experts' rows) goes to
    ((r/32) * (K/128) + j/64) * 2048 + (r%32) * 64 + j%64."""
    E, N, KB = packed.shape
    rows = E * N
    r, j = np.meshgrid(np.arange(rows), np.arange(KB), indexing="ij")
    dst = ((r // 32) * (KB // 64) + j // 64) * 2048 + (r % 32) * 64 + j % 64
    out = np.zeros(rows * KB, np.uint8)
    out[dst.reshape(-1)] = packed.reshape(-1)
    assert np.unique(dst).size == rows * KB  # a permutation
    return out.reshape(E, N, KB)


@pytest.mark.parametrize("shape", [(1, 32, 128), (3, 64, 256), (2, 96, 2048), (5, 128, 384), (7, 32, 640)])
def test_tile_weights_is_the_documented_permutation(qe, shape):
    import torch

    E, N, K = shape
    packed = np.random.default_rng(K + N).integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    got = _np(qe.tile_weights(torch.from_numpy(packed).cuda()))
    assert np.array_equal(got, _tiled_by_definition(packed))


def _cfgs(fmt):
    # The wide pipeline takes K/g a multiple of 8 (and, for the symmetric
    # format, K/g < 8); the general one the rest.  Gate/up (K = H): K/g = 12,
    # 8, 24, 8, 8 -> general, then wide.  Down (K = I): K/g = 4, 4, 12, 2, 4
    # -> general in every format for 12, in the other two formats for 2 and
    # 4.
    return [
        synth.MoEConfig(f"gen_gateup_{fmt}", T=200, H=768, I=256, E=4, k=2, g=64, seed=85, fmt=fmt),
        synth.MoEConfig(f"ragged64_{fmt}", T=400, H=512, I=256, E=4, k=2, g=64, seed=81, fmt=fmt),
        synth.MoEConfig(f"ragged32_{fmt}", T=333, H=768, I=384, E=5, k=3, g=32, seed=82, fmt=fmt),
        synth.MoEConfig(f"ragged128_{fmt}", T=260, H=1024, I=256, E=3, k=1, g=128, seed=83, fmt=fmt),
        synth.MoEConfig(f"many_{fmt}", T=96, H=256, I=128, E=64, k=6, g=32, seed=84, fmt=fmt),
    ]


def _gemv_cfgs(fmt):
    return [
        synth.MoEConfig(f"gemv_tiny_{fmt}", T=16, H=256, I=128, E=16, k=2, g=32, seed=91, fmt=fmt),
        synth.MoEConfig(f"gemv_t1_{fmt}", T=1, H=2048, I=512, E=64, k=10, g=64, seed=92, fmt=fmt),
        synth.MoEConfig(f"gemv_wide_{fmt}", T=8, H=4096, I=1024, E=32, k=8, g=128, seed=93, fmt=fmt),
    ]


def _both_layouts(inp):
    logits, x, rows = to_device(inp)
    tiled = rows.to_tiled()
    assert tiled.layout == "tiled" and rows.layout == "rows"
    return logits, x, rows, tiled


def _ids(cfgs):
    return [c.name for c in cfgs]


GEMM_CFGS = [c for f in FORMATS for c in _cfgs(f)]
GEMV_CFGS = [c for f in FORMATS for c in _gemv_cfgs(f)]


@pytest.mark.parametrize("cfg", GEMM_CFGS, ids=_ids(GEMM_CFGS))
def test_tiled_grouped_gemm(qe, cfg, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "gemm")
    inp = inputs(cfg)
    logits, x, rows, tiled = _both_layouts(inp)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for fused in (False, True):
        a = qe.moe_layer(logits, x, rows, cfg.k, fused=fused)
        b = qe.moe_layer(logits, x, tiled, cfg.k, fused=fused)
        key = "out"
        assert np.array_equal(_np(a[key]), _np(b[key])), f"{cfg.name} fused={fused}"
        if not fused:
            assert np.array_equal(_np(a["y"]), _np(b["y"])), cfg.name
            check_close(_np(b["y"]), ref["y"], f"{cfg.name} y (tiled)")
        check_close(_np(b["out"]), ref["out"], f"{cfg.name} out (tiled, fused={fused})")


@pytest.mark.parametrize("cfg", GEMV_CFGS, ids=_ids(GEMV_CFGS))
def test_tiled_gemv(qe, cfg, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "gemv")
    inp = inputs(cfg)
    logits, x, rows, tiled = _both_layouts(inp)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for fused in (False, True):
        a = qe.moe_layer(logits, x, rows, cfg.k, fused=fused)
        b = qe.moe_layer(logits, x, tiled, cfg.k, fused=fused)
        assert np.array_equal(_np(a["out"]), _np(b["out"])), f"{cfg.name} fused={fused}"
        check_close(_np(b["out"]), ref["out"], f"{cfg.name} out (tiled, fused={fused})")


@pytest.mark.parametrize("cfg", GEMV_CFGS, ids=_ids(GEMV_CFGS))
def test_tiled_decode_layer(qe, cfg):
    """The single layer call at decode sizes: the two-kernel decode layer."""
    inp = inputs(cfg)
    logits, x, rows, tiled = _both_layouts(inp)
    qe.timing_enable(True)
    a = qe.layer(logits, x, rows, cfg.k)
    b = qe.layer(logits, x, tiled, cfg.k)
    names = qe.timing_kernels()
    qe.timing_enable(False)
    assert "decode_route_gateup" in names and "decode_down_combine" in names, names
    assert np.array_equal(_np(a["out"]), _np(b["out"])), cfg.name
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    check_close(_np(b["out"]), ref["out"], f"{cfg.name} out (tiled)")


@pytest.mark.parametrize("fmt", FORMATS)
def test_tiled_layer_noalloc(qe, fmt):
    """The no-allocation layer call reads the tiled layout too (a prefill
    chunk on the grouped GEMM, then a decode step)."""
    for cfg in (synth.MoEConfig(f"noalloc_{fmt}", T=300, H=512, I=256, E=8, k=2, g=64, seed=95, fmt=fmt),
                _gemv_cfgs(fmt)[0]):
        inp = inputs(cfg)
        logits, x, rows, tiled = _both_layouts(inp)
        a = _np(qe.layer(logits, x, rows, cfg.k)["out"])
        b = _np(qe.layer_noalloc(logits, x, tiled, cfg.k)["out"])
        assert np.array_equal(a, b), cfg.name


@pytest.mark.parametrize("name", ["prefill6144", "prefill6144_asym", "prefill6144_int5", "zipf6144"])
def test_tiled_layer_call_full_size(qe, name):
    """The benchmark's single layer call at full size: tiled codes give the
    row-major outputs on every element (those are checked against the oracle
    by the full-size parity tests)."""
    import torch

    cfg = synth.config(name)
    inp = inputs(name)
    logits, x, rows, tiled = _both_layouts(inp)
    print(f"[layout] {name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g} {cfg.fmt}", flush=True)
    outs = []
    for ex in (rows, tiled):
        run = qe.LayerRunner(ex, cfg.T, cfg.E, cfg.k, fused=True, single_call=True)
        run(logits, x)
        torch.cuda.synchronize()
        outs.append(_np(run.out))
        del run
    assert np.array_equal(outs[0], outs[1]), name
    assert np.isfinite(outs[1]).all()


def test_tiled_descriptor_round_trip(qe):
    cfg = dataclasses.replace(_cfgs("int4")[3], name="desc")
    _, _, rows, tiled = _both_layouts(inputs(cfg))
    assert rows.descriptor().layout == 0 and tiled.descriptor().layout == 1
    assert tiled.to_tiled() is tiled
    assert tiled.gate.shape == rows.gate.shape and tiled.down.shape == rows.down.shape


EDGE_CFGS = [
    # the grouped-GEMM layer call with 1024 experts (1200 pairs: the multi-segment grouping)
    synth.MoEConfig("tiled_fold_e1024", T=150, H=256, I=128, E=1024, k=8, g=32, seed=97),
    # the two-kernel decode layer with 1024 experts and k = 16
    synth.MoEConfig("tiled_decode_e1024", T=3, H=512, I=256, E=1024, k=16, g=64, seed=98),
    # long rows: gate/up K = 8192 (64 stages of the wide pipeline, 64 tiles per 32-row block)
    synth.MoEConfig("tiled_h8192", T=64, H=8192, I=1024, E=4, k=2, g=128, seed=99),
    # down K = 16384: the last tile of a block ends at the end of the block's buffer range
    synth.MoEConfig("tiled_i16384", T=48, H=256, I=16384, E=2, k=1, g=128, seed=100),
]


@pytest.mark.parametrize("cfg", EDGE_CFGS, ids=_ids(EDGE_CFGS))
def test_tiled_edge_shapes_layer_call(qe, cfg):
    """strata_moe_layer at the envelope's edges: tiled equals row-major bit for
    bit, and both match the oracle."""
    inp = inputs(cfg)
    logits, x, rows, tiled = _both_layouts(inp)
    print(f"[layout] {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g}", flush=True)
    a = qe.layer(logits, x, rows, cfg.k)
    b = qe.layer(logits, x, tiled, cfg.k)
    assert np.array_equal(_np(a["out"]), _np(b["out"])), cfg.name
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    assert np.array_equal(_np(b["ids"]).reshape(-1), ref["ids"].reshape(-1))
    check_close(_np(b["out"]), ref["out"], f"{cfg.name} out (tiled)")
