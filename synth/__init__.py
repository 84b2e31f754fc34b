"""Seeded synthetic inputs for the routed MoE FFN layer and the KV-cache attention (shared by the
oracle and the GPU path)."""
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
    quantize_groups,
    quantize_int4_asym_groups,
    quantize_int4_groups,
    quantize_int5_groups,
    weight_bytes_per_expert,
)
from .kv import ATTN_CONFIGS, AttnConfig, AttnInputs, attn_config, make_attn_inputs  # noqa: F401
