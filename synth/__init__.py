"""Seeded synthetic inputs shared by the oracle tests and the GPU path (no method arithmetic)."""
from .workloads import (  # noqa: F401
    WORKLOADS, Workload, ShareInputs, make_share_inputs, make_logits, make_x,
    make_expert_weights, make_local_weights, f32_to_bf16_bits, bf16_bits_to_f32,
    zipf_probs, layer_temperatures,
)
