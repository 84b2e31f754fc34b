"""strata_moe_layer_noalloc (the layer call on the library's static device
scratch) against strata_moe_layer (the same call on a caller workspace),
through the C ABI.

Both run the same kernels, so every output must be identical bit for bit; the
outputs are also checked against the fp64 oracle (routing bit-exact, out
within the output tolerance).  Two calls in a row on one device: a 512-token
prefill batch (grouped-GEMM path, about 28 MB of scratch) and then a smaller
decode batch (two-kernel path) on the same scratch, whose contents from the
first call must not change the second call's results; a third call repeats
the first and must reproduce it exactly.
"""
import ctypes

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


def _compare(qe, inp, label):
    import torch

    cfg = inp.cfg
    logits, x, ex = to_device(inp)
    need = qe.workspace_size(cfg.T, cfg.E, cfg.k, cfg.H, cfg.I, cfg.g)
    assert need <= 64 << 20, (label, need)
    print(f"[no-alloc] {label}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} g={cfg.g}, "
          f"scratch {need} bytes", flush=True)
    na = qe.layer_noalloc(logits, x, ex, cfg.k)
    torch.cuda.synchronize()
    ws = qe.layer(logits, x, ex, cfg.k)
    torch.cuda.synchronize()
    for key in ("ids", "w", "counts", "offsets", "perm", "inv_perm", "out"):
        assert torch.equal(na[key], ws[key]), f"{label}: {key} differs from strata_moe_layer"
    ref = oracle.moe_layer(inp.logits, inp.x_bf16, inp.weights, cfg.k, cfg.g)
    for key in ("ids", "counts", "offsets", "perm", "inv_perm"):
        assert (_np(na[key]).reshape(-1) == ref[key].reshape(-1)).all(), f"{label}: {key}"
    assert np.abs(_np(na["w"]).astype(np.float64) - ref["w"]).max() <= W_ATOL
    check_close(_np(na["out"]), ref["out"], f"{label} out")
    return na


def test_noalloc_layer_matches_layer_call_twice(qe):
    import torch

    big = inputs("prefill512")
    small = inputs("decode")
    first = _compare(qe, big, "call 1 (prefill512)")
    _compare(qe, small, "call 2 (decode, smaller)")
    # The first input again: the scratch now holds the decode call's data.
    logits, x, ex = to_device(big)
    again = qe.layer_noalloc(logits, x, ex, big.cfg.k)
    torch.cuda.synchronize()
    for key in first:
        assert torch.equal(first[key], again[key]), key


def test_noalloc_rejects_shapes_beyond_the_scratch(qe):
    """The 6144-token chunk needs more scratch than the static array holds:
    refused before anything is enqueued, with both sizes in the message."""
    from quantized_expert_ffn_histogram_amd import _abi

    lib = qe.load()
    cfg = synth.config("prefill6144")
    fake = ctypes.c_void_p(0x10000)
    w = _abi.StrataMoeWeights(fake.value, fake.value, fake.value, fake.value, fake.value, fake.value, cfg.E, cfg.H,
                              cfg.I, cfg.g)
    rc = lib.strata_moe_layer_noalloc(fake, fake, cfg.T, cfg.k, ctypes.byref(w), fake, fake, fake, fake, fake, fake,
                                      fake, None)
    assert rc == 2
    msg = lib.strata_moe_last_error().decode()
    assert "strata_moe_layer_noalloc" in msg and str(64 << 20) in msg, msg
