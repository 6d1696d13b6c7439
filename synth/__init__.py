"""Seeded synthetic inputs for the decode-time int4 MoE expert path.

This package only draws random numbers and lays them out in the host formats
the library and the oracle both accept.  It performs none of the method's
arithmetic (no unpacking, no dequantisation, no routing), so the oracle and the
HIP path can share it without sharing any of the computation they check.
"""

from .configs import CONFIGS, Config, get_config  # noqa: F401
from .gen import (  # noqa: F401
    ExpertWeights,
    LayerInputs,
    TensorHost,
    expert_format,
    gen_activations,
    gen_expert,
    gen_layer,
    gen_norm,
    gen_residual,
    gen_router,
    gen_shared_expert,
    round_f32_to_bf16_bits,
)
