"""GPU parity of every C-ABI call against the fp64 oracle.

Routing ids, counts, offsets and the permutation are compared bit-exactly;
routing weights to 1e-6; layer outputs to max|err| <= 2e-2 * RMS(ref) and
sum|err| / sum|ref| <= 5e-3.  Small layers are compared element by element in
full; the full-size layers on sampled tokens and sampled grouped rows, which
the oracle computes one by one.
"""
import dataclasses

import numpy as np
import pytest

import oracle
import synth
from moe_testutil import W_ATOL, check_close, inputs, to_device

pytestmark = pytest.mark.gpu

FULL = ["tiny", "decode", "prefill512", "prefill6144", "zipf6144"]


@pytest.fixture(scope="module")
def qe(gpu_available):
    import quantized_expert_ffn_histogram_amd as qe

    qe.load()
    return qe


def _np(t):
    return t.detach().cpu().numpy()


# ----------------------------------------------------------------------------- route
def _check_route(qe, logits_np, k):
    import torch

    ids, w = qe.route(torch.from_numpy(np.ascontiguousarray(logits_np, np.float32)).cuda(), k)
    rid, rw = oracle.route(logits_np, k)
    assert (_np(ids) == rid).all(), "routing ids differ from the oracle"
    wg = _np(w).astype(np.float64)
    assert np.abs(wg - rw).max() <= W_ATOL
    assert np.abs(wg.sum(1) - 1.0).max() <= W_ATOL
    return ids, w


@pytest.mark.parametrize("name", FULL)
def test_route_bitexact(qe, name):
    inp = inputs(name)
    _check_route(qe, inp.logits, inp.cfg.k)


@pytest.mark.parametrize(
    "T,E,k,kind",
    [
        (64, 512, 10, "equal"),
        (1000, 512, 10, "grid"),
        (300, 256, 8, "grid_coarse"),
        (50, 16, 4, "signed_zero"),
        (37, 33, 5, "normal"),
        (70, 100, 32, "grid"),
        (45, 1000, 7, "grid"),
        (20, 1024, 32, "normal"),
        (9, 1, 1, "normal"),
        (11, 32, 32, "grid"),
        (3, 64, 1, "huge"),
        (500, 512, 10, "grid_fine"),
        (60, 40, 30, "neg_max"),
    ],
)
def test_route_ties_and_shapes(qe, T, E, k, kind):
    rng = np.random.default_rng(T * 1000 + E + k)
    z = rng.standard_normal((T, E))
    if kind == "equal":
        logits = np.full((T, E), 0.25)
    elif kind == "grid":
        logits = np.round(z * 4) / 4
    elif kind == "grid_coarse":
        logits = np.round(z)
    elif kind == "signed_zero":
        logits = np.where(rng.random((T, E)) < 0.5, -0.0, 0.0)
        logits[:, ::5] = -1.0
    elif kind == "huge":
        logits = z * 1e30
    elif kind == "grid_fine":  # a few ties among the leading candidates
        logits = np.round(z * 32) / 32
    elif kind == "neg_max":  # about half at the most negative float, so some selected ones tie there
        logits = np.where(rng.random((T, E)) < 0.5, np.finfo(np.float32).min, z)
    else:
        logits = z
    _check_route(qe, logits.astype(np.float32), k)


# ----------------------------------------------------------------------------- permute
def _check_permute(qe, ids_np, E):
    import torch

    ids = torch.from_numpy(np.ascontiguousarray(ids_np, np.int32)).cuda()
    counts, offsets, perm, inv = qe.permute(ids, E)
    rc = oracle.histogram(ids_np, E)
    ro = oracle.exclusive_scan(rc)
    rp, ri = oracle.permutation(ids_np)
    assert (_np(counts) == rc).all()
    assert (_np(offsets) == ro).all()
    assert (_np(perm) == rp).all()
    assert (_np(inv) == ri).all()


@pytest.mark.parametrize("name", FULL)
def test_permute_bitexact(qe, name):
    inp = inputs(name)
    ids, _ = oracle.route(inp.logits, inp.cfg.k)
    _check_permute(qe, ids, inp.cfg.E)


@pytest.mark.parametrize(
    "T,E,k,kind",
    [
        (5000, 16, 1, "one_hot"),
        (20000, 1024, 3, "random"),
        (1, 8, 1, "random"),
        (512, 512, 2, "random"),    # 1024 pairs: single-workgroup path, at its limit
        (1025, 300, 1, "random"),   # 1025 pairs: segmented path, ragged last segment
        (3001, 64, 7, "skewed"),
        (2048, 1024, 1, "empty_half"),
        # segments of 1024 pairs; the scan reads each expert's column in
        # batches of 32 segments
        (131072, 512, 1, "random"),  # 128 segments: four whole batches
        (131073, 512, 1, "random"),  # 129 segments: one pair in the last
        (65536, 1024, 1, "random"),  # 64 segments at E = 1024
        (65537, 1024, 1, "random"),  # 65 segments at E = 1024
        (40000, 16, 4, "one_hot"),   # 157 full segments of one expert
        (200000, 8, 5, "skewed"),    # 977 segments
    ],
)
def test_permute_edge_cases(qe, T, E, k, kind):
    rng = np.random.default_rng(T + E + k)
    if kind == "one_hot":
        ids = np.full((T, k), 3, np.int32)
    elif kind == "skewed":
        ids = np.minimum(rng.zipf(1.5, (T, k)) - 1, E - 1).astype(np.int32)
    elif kind == "empty_half":
        ids = (2 * rng.integers(0, E // 2, (T, k))).astype(np.int32)
    else:
        ids = rng.integers(0, E, (T, k)).astype(np.int32)
    _check_permute(qe, ids, E)


def test_zero_tokens(qe):
    import torch

    ids, w = qe.route(torch.zeros((0, 16), dtype=torch.float32, device="cuda"), 2)
    assert ids.shape == (0, 2)
    counts, offsets, perm, inv = qe.permute(ids, 16)
    assert (_np(counts) == 0).all() and (_np(offsets) == 0).all()


# ----------------------------------------------------------------------------- ffn, full compare
SMALL_CFGS = [
    synth.config("tiny"),
    # several 128-row tiles per expert with ragged tails, several column slices
    synth.MoEConfig("ragged64", T=400, H=512, I=256, E=4, k=2, g=64, seed=31),
    synth.MoEConfig("ragged32", T=333, H=768, I=384, E=5, k=3, g=32, seed=32),
    synth.MoEConfig("ragged128", T=260, H=1024, I=256, E=3, k=1, g=128, seed=33),
    synth.MoEConfig("manyexperts", T=96, H=256, I=128, E=64, k=6, g=32, seed=34),
]


def _run_layer(qe, inp, fused):
    logits, x, ex = to_device(inp)
    return qe.moe_layer(logits, x, ex, inp.cfg.k, fused=fused)


@pytest.mark.parametrize("path", ["gemm", "auto"])
@pytest.mark.parametrize("cfg", SMALL_CFGS, ids=lambda c: c.name)
def test_ffn_full_compare(qe, cfg, path, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    inp = inputs(cfg)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    det = _run_layer(qe, inp, fused=False)
    check_close(_np(det["y"]), ref["y"], "y")
    check_close(_np(det["out"]), ref["out"], "out (deterministic)")
    fus = _run_layer(qe, inp, fused=True)
    check_close(_np(fus["out"]), ref["out"], "out (fused)")


GEMV_CFGS = [
    synth.MoEConfig("gemv_tiny", T=16, H=256, I=128, E=16, k=2, g=32, seed=41),
    synth.MoEConfig("gemv_t1", T=1, H=2048, I=512, E=64, k=10, g=64, seed=42),
    synth.MoEConfig("gemv_wide", T=8, H=4096, I=1024, E=32, k=8, g=128, seed=43),
    synth.MoEConfig("gemv_shared", T=12, H=1024, I=256, E=4, k=3, g=64, seed=44),
    # largest envelope: E=1024 experts, k=32, 512 pairs
    synth.MoEConfig("gemv_maxk", T=16, H=256, I=128, E=1024, k=32, g=32, seed=45),
]


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("cfg", GEMV_CFGS, ids=lambda c: c.name)
def test_ffn_decode_paths(qe, cfg, path, monkeypatch):
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    inp = inputs(cfg)
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    det = _run_layer(qe, inp, fused=False)
    check_close(_np(det["y"]), ref["y"], "y")
    fus = _run_layer(qe, inp, fused=True)
    check_close(_np(fus["out"]), ref["out"], "out (fused)")


def test_gemv_fused_repeatable_across_calls(qe, monkeypatch):
    """The decode path's fused output (fp16 y rows in pair order, summed in j
    order) is bitwise repeatable, and a different step in between (other
    experts, other rows) leaves nothing behind that changes the next call."""
    monkeypatch.setenv("STRATA_MOE_FFN_PATH", "gemv")
    cfg = synth.config("decode")
    inp = inputs(cfg)
    steps = synth.decode_steps(cfg, 2)
    a = _run_layer(qe, inp, fused=True)
    other = dataclasses.replace(inp, logits=steps[1][0], x_bf16=steps[1][1])
    mid = _run_layer(qe, other, fused=True)
    ref = oracle.moe_layer(other.logits, other.x_bf16, other.weights, cfg.k, cfg.g)
    check_close(_np(mid["out"]), ref["out"], "decode step 1 out")
    b = _run_layer(qe, inp, fused=True)
    assert (_np(a["out"]) == _np(b["out"])).all()
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    check_close(_np(b["out"]), ref["out"], "decode out")


# ----------------------------------------------------------------------------- ffn, full-size sampled
def _sample_tokens(T, n, seed):
    rng = np.random.default_rng(seed)
    pick = set(rng.choice(T, size=min(n, T), replace=False).tolist()) | {0, T - 1}
    return np.array(sorted(pick))


@pytest.mark.parametrize("name", ["decode", "prefill512", "prefill6144", "zipf6144", "prefill6144_g32",
                                  "prefill6144_g128"])
def test_ffn_full_size_sampled_tokens(qe, name):
    inp = inputs(name)
    cfg = inp.cfg
    res = _run_layer(qe, inp, fused=True)
    ids, w = oracle.route(inp.logits, cfg.k)
    assert (_np(res["ids"]) == ids).all()
    toks = _sample_tokens(cfg.T, 10, cfg.seed)
    ref = oracle.moe_out_tokens(toks, ids, w, inp.x_bf16, inp.weights, cfg.g)
    check_close(_np(res["out"])[toks], ref, f"{name} out[sampled tokens]")


@pytest.mark.parametrize("name", ["prefill6144", "zipf6144", "prefill6144_g32", "prefill6144_g128"])
def test_ffn_full_size_sampled_grouped_rows(qe, name):
    """Deterministic path: grouped rows y[i] of the busiest expert (many tiles,
    ragged last tile) and of a median expert, against the oracle row by row."""
    inp = inputs(name)
    cfg = inp.cfg
    res = _run_layer(qe, inp, fused=False)
    ids, _ = oracle.route(inp.logits, cfg.k)
    counts = oracle.histogram(ids, cfg.E)
    offsets = oracle.exclusive_scan(counts)
    perm, _ = oracle.permutation(ids)
    y = _np(res["y"])
    nz = np.nonzero(counts)[0]
    busiest = int(np.argmax(counts))
    median = int(nz[np.argsort(counts[nz])[len(nz) // 2]])
    x = oracle.bf16_to_f64(inp.x_bf16)
    for e in (busiest, median):
        lo, hi = int(offsets[e]), int(offsets[e + 1])
        rows = np.unique(np.concatenate([np.arange(lo, min(hi, lo + 40)), np.arange(max(lo, hi - 40), hi)]))
        W = [oracle.dequant(inp.weights[m][e], inp.weights[m + "_scale"][e], cfg.g) for m in ("gate", "up", "down")]
        ref = oracle.expert_ffn(x[perm[rows] // cfg.k], *W)
        check_close(y[rows], ref, f"{name} y rows of expert {e} ({hi - lo} rows)")


# ----------------------------------------------------------------------------- determinism
def test_deterministic_path_is_bitwise_repeatable(qe):
    inp = inputs(SMALL_CFGS[1])
    a = _run_layer(qe, inp, fused=False)
    b = _run_layer(qe, inp, fused=False)
    for key in ("ids", "w", "counts", "offsets", "perm", "inv_perm", "y", "out"):
        assert (_np(a[key]) == _np(b[key])).all(), key


def test_one_hot_routing_layer(qe):
    """Every token routed to the same k experts: k experts with T rows each."""
    cfg = synth.MoEConfig("onehot", T=700, H=512, I=256, E=8, k=2, g=64, seed=51)
    inp = synth.make_inputs(cfg)
    inp.logits[:, 5] += 50.0
    inp.logits[:, 2] += 40.0
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    assert ref["counts"][5] == 700 and ref["counts"][2] == 700
    res = _run_layer(qe, inp, fused=True)
    check_close(_np(res["out"]), ref["out"], "one-hot out")


# ----------------------------------------------------------------------------- graph replay
@pytest.mark.parametrize("single", [False, True], ids=["four_calls", "layer_call"])
@pytest.mark.parametrize("name", ["tiny", "decode", "prefill512"])
def test_layer_graph_replay(qe, name, single):
    """A whole layer call (route, permute, fused ffn) captured in a HIP graph
    gives the eager result on every replay.  Between replays the same buffers
    are overwritten by an eager call on other logits and the stream is
    synchronized, so each replay recomputes everything it depends on."""
    import torch

    inp = inputs(name)
    cfg = inp.cfg
    logits, x, experts = to_device(inp)
    run = qe.LayerRunner(experts, cfg.T, cfg.E, cfg.k, fused=True, single_call=single)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for _ in range(2):
            run(logits, x)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(logits, x)
    ref = {k_: getattr(run, k_).clone() for k_ in ("ids", "w", "counts", "offsets", "perm", "out")}
    run(logits, x)
    for k_, v in ref.items():  # capture itself ran nothing: the eager call fills the buffers
        v.copy_(getattr(run, k_))
    oref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    assert (_np(ref["ids"]) == oref["ids"]).all()
    check_close(_np(ref["out"]), oref["out"], f"{name} eager out")
    other = torch.roll(logits, shifts=1, dims=1)
    for rep in range(3):
        run(other, x)
        torch.cuda.synchronize()
        assert not torch.equal(run.ids, ref["ids"])
        graph.replay()
        torch.cuda.synchronize()
        for k_, v in ref.items():
            assert torch.equal(getattr(run, k_), v), f"replay {rep}: {k_} differs from the eager call"


# ----------------------------------------------------------------------------- whole-layer call
LAYER_CFGS = [synth.config("decode"), synth.config("decode_shared")] + GEMV_CFGS + [
    # drafts that share most of the first token's experts, 16 tokens
    synth.MoEConfig("layer_shared16", T=16, H=1024, I=256, E=64, k=8, g=64, seed=50, draft_sigma=0.05),
    synth.MoEConfig("layer_e1024", T=3, H=512, I=256, E=1024, k=16, g=64, seed=46),
    # k * inter at the two-kernel path's limit, one down row per wavefront
    synth.MoEConfig("layer_i2048", T=2, H=256, I=2048, E=8, k=8, g=128, seed=47),
    SMALL_CFGS[1],
    # grouped-GEMM path above 1024 pairs (routing kernel converts x, the scan
    # builds the tile lists): ragged tiles, and 1024 experts of ~1 pair each
    synth.MoEConfig("layer_fold", T=600, H=512, I=256, E=8, k=3, g=64, seed=48),
    synth.MoEConfig("layer_fold_e1024", T=150, H=256, I=128, E=1024, k=8, g=32, seed=49),
]


def _two_kernel_shape(cfg):
    pow2 = lambda v: v & (v - 1) == 0
    return (cfg.T <= 16 and cfg.k <= 16 and cfg.k * cfg.I <= 16384 and cfg.H <= 4096 and pow2(cfg.H)
            and 128 <= cfg.I <= 2048 and pow2(cfg.I))


@pytest.mark.parametrize("path", ["auto", "gemm"])
@pytest.mark.parametrize("cfg", LAYER_CFGS, ids=lambda c: c.name)
def test_layer_call(qe, cfg, path, monkeypatch):
    """strata_moe_layer: routing and grouping outputs bit-exact against the
    oracle and identical to the routing call's, out within the tolerance; the
    decode shapes run as the two fused kernels under the automatic path."""
    import torch

    monkeypatch.setenv("STRATA_MOE_FFN_PATH", path)
    inp = inputs(cfg)
    logits, x, ex = to_device(inp)
    qe.timing_enable(True)
    res = qe.layer(logits, x, ex, cfg.k)
    names = qe.timing_kernels()
    qe.timing_enable(False)
    decode = path == "auto" and _two_kernel_shape(cfg)
    assert ("decode_route_gateup" in names) == decode, names
    # The grouped-GEMM path above 1024 pairs runs without the ffn prologue.
    fold = not decode and cfg.T * cfg.k > 1024
    assert ("route_xconv" in names) == fold, names
    assert not (fold and "ffn_prep" in names), names
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        assert (_np(res[key]) == ref[key]).all(), key
    assert np.abs(_np(res["w"]).astype(np.float64) - ref["w"]).max() <= W_ATOL
    check_close(_np(res["out"]), ref["out"], f"{cfg.name} out")
    ids, w = qe.route(logits, cfg.k)
    assert torch.equal(ids, res["ids"]) and torch.equal(w, res["w"])


@pytest.mark.parametrize("k", list(range(1, 18)) + [32])
def test_layer_call_combine_every_k(qe, k):
    """The grouped-GEMM layer call finishes with the combine of the fp16 y
    rows, which has one kernel instance per k up to 16 and a padded one above:
    each of them against the oracle (ids bit-exact, out within the
    tolerance)."""
    cfg = synth.MoEConfig(f"combine_k{k}", T=120, H=256, I=128, E=max(24, k), k=k, g=32, seed=700 + k)
    inp = inputs(cfg)
    logits, x, ex = to_device(inp)
    qe.timing_enable(True)
    res = qe.layer(logits, x, ex, cfg.k)
    names = qe.timing_kernels()
    qe.timing_enable(False)
    assert "combine" in names and "decode_route_gateup" not in names, names
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        assert (_np(res[key]) == ref[key]).all(), key
    check_close(_np(res["out"]), ref["out"], f"{cfg.name} out")


@pytest.mark.parametrize("k", list(range(1, 17)))
def test_layer_call_decode_every_k(qe, k):
    """The two-kernel decode layer has one down + combine instance per range
    of k (up to 4, 6, 8, 10, 12, 16): each of them against the oracle."""
    cfg = synth.MoEConfig(f"decode_k{k}", T=4, H=256, I=128, E=max(32, k), k=k, g=32, seed=720 + k)
    assert _two_kernel_shape(cfg)
    inp = inputs(cfg)
    logits, x, ex = to_device(inp)
    qe.timing_enable(True)
    res = qe.layer(logits, x, ex, cfg.k)
    names = qe.timing_kernels()
    qe.timing_enable(False)
    assert "decode_down_combine" in names, names
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        assert (_np(res[key]) == ref[key]).all(), key
    check_close(_np(res["out"]), ref["out"], f"{cfg.name} out")


def test_layer_call_repeatable_and_zero_tokens(qe):
    """The two-kernel decode output is bitwise repeatable across calls with a
    different step in between; T = 0 writes zero counts and offsets."""
    import torch

    cfg = synth.config("decode")
    inp = inputs(cfg)
    logits, x, ex = to_device(inp)
    a = qe.layer(logits, x, ex, cfg.k)
    other = torch.roll(logits, shifts=3, dims=1)
    qe.layer(other, x, ex, cfg.k)
    b = qe.layer(logits, x, ex, cfg.k)
    for key in a:
        assert torch.equal(a[key], b[key]), key
    z = qe.layer(logits[:0], x[:0], ex, cfg.k)
    assert int(z["counts"].abs().sum()) == 0 and int(z["offsets"].abs().sum()) == 0


# ----------------------------------------------------------------------------- router projection
ROUTER_CFGS = [
    (6144, 2048, 512, 10, 61),  # the prefill chunk's tokens and expert pool
    (100, 128, 37, 5, 62),      # tokens and experts off the 128 tile, E % 4 != 0
    (1, 64, 1, 1, 63),          # one token, one expert, one K stage
    (70, 448, 130, 4, 65),      # seven K stages: one ring turn of four, then three more
    (130, 16384, 70, 3, 66),    # the largest H: 256 K stages
    (257, 320, 1024, 32, 64),   # largest E and k, odd number of K stages
]


@pytest.mark.parametrize("T,H,E,k,seed", ROUTER_CFGS)
def test_router_projection_then_topk(qe, T, H, E, k, seed):
    """strata_moe_router: fp32 logits within the error bound of fp32
    accumulation of H exact bf16 products (|err| <= H * 2^-24 * sum_h
    |x_h w_h|) of the fp64 projection; the selection bit-exact against the
    oracle's top-k taken on the kernel's own logits (the decision in the
    kernel's precision), weights within the routing tolerance."""
    import torch

    x, w = synth.make_router(T, H, E, seed)
    xd = torch.from_numpy(x.view(np.int16)).cuda().view(torch.bfloat16)
    wd = torch.from_numpy(w.view(np.int16)).cuda().view(torch.bfloat16)
    logits, ids, wts = qe.router(xd, wd, k)
    got = _np(logits)
    ref = oracle.router_logits(x, w)
    mag = np.abs(oracle.bf16_to_f64(x)) @ np.abs(oracle.bf16_to_f64(w)).T
    bound = H * 2.0 ** -24 * mag + 1e-30
    assert (np.abs(got.astype(np.float64) - ref) <= bound).all(), float(np.max(np.abs(got - ref) / bound))
    rid, rw = oracle.route(got, k)
    assert (_np(ids) == rid).all()
    assert np.abs(_np(wts).astype(np.float64) - rw).max() <= W_ATOL
    # The same selection as the routing call on those logits.
    ids2, w2 = qe.route(logits, k)
    assert torch.equal(ids, ids2) and torch.equal(wts, w2)
