"""Seeded synthetic inputs for the routed MXFP4 MoE layer.

This package produces the *data* that both the fp64 oracle and the HIP path
consume: bf16 activation and router bit patterns, MXFP4 code and scale bytes,
and the optional per-expert logit bias. It holds none of the layer's
arithmetic (no dequantisation, no routing, no FFN).
"""

from .workloads import (  # noqa: F401
    WORKLOADS,
    Workload,
    bank_shapes,
    f64_to_bf16_bits,
    gen_bank,
    gen_expert,
    gen_fp8_bank,
    gen_nvfp4_bank,
    gen_inputs,
    gen_router,
    gen_tokens,
    gen_zipf_bias,
    get,
)
