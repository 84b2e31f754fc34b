"""Seeded synthetic inputs for the routed MoE FFN layer (shared by the oracle and the GPU path)."""
from .gen import (  # noqa: F401
    CONFIGS,
    MoEConfig,
    MoEInputs,
    bf16_bits_from_f32,
    config,
    decode_steps,
    make_inputs,
    make_logits,
    make_router,
    make_x,
    quantize_int4_groups,
    weight_bytes_per_expert,
)
