"""Shared helpers for the GPU parity tests (inputs to device, tolerance checks)."""
from __future__ import annotations

import functools

import numpy as np

import synth

# Output tolerance of the layer against the fp64 oracle (over the compared
# elements): max |err| <= 2e-2 * RMS(ref) and sum |err| / sum |ref| <= 5e-3.
MAX_ERR_REL_RMS = 2e-2
L1_REL = 5e-3
# Routing weights: fp32 softmax of k values against fp64.
W_ATOL = 1e-6


@functools.lru_cache(maxsize=4)
def inputs(name_or_cfg):
    return synth.make_inputs(name_or_cfg)


def to_device(inp, device="cuda"):
    import torch

    import quantized_expert_ffn_histogram_amd as qe

    logits = torch.from_numpy(inp.logits).to(device)
    x = torch.from_numpy(inp.x_bf16.view(np.int16)).to(device).view(torch.bfloat16)
    experts = qe.QuantizedExperts.from_numpy(inp.weights, inp.cfg.g, device) if inp.weights else None
    return logits, x, experts


def check_close(got: np.ndarray, ref: np.ndarray, what: str = "out") -> dict:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    err = np.abs(got - ref)
    rms = float(np.sqrt(np.mean(ref * ref)))
    l1 = float(err.sum() / max(np.abs(ref).sum(), 1e-300))
    stats = dict(max_err_over_rms=float(err.max() / max(rms, 1e-300)), l1_rel=l1)
    assert err.max() <= MAX_ERR_REL_RMS * rms, f"{what}: {stats}"
    assert l1 <= L1_REL, f"{what}: {stats}"
    return stats
