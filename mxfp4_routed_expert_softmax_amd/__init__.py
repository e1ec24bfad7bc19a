"""Routed MXFP4 mixture-of-experts layer on MI355X (gfx950).

The layer runs in hand-written HIP kernels behind the C ABI of
include/moe_mxfp4.h; this package holds those sources (csrc/), their build
script (build.py) and a ctypes binding (_lib.py) with the same call names.
"""

from ._lib import (  # noqa: F401
    Bank,
    BankTensors,
    Fp8Bank,
    Fp8BankTensors,
    MoeError,
    NvBank,
    NvBankTensors,
    MOE_ERR_HIP,
    MOE_ERR_TIMEOUT,
    MOE_ERR_INVALID_ARG,
    MOE_ERR_UNSUPPORTED,
    MOE_ERR_WORKSPACE,
    MOE_OK,
    header_functions,
    lib,
    moe_combine,
    moe_expert_ffn_fp8,
    moe_expert_ffn_mxfp4,
    moe_expert_ffn_nvfp4,
    moe_last_call_launches,
    moe_launch_name,
    moe_layer_forward,
    moe_layer_forward_fp8_shared,
    moe_layer_forward_mxfp8_act,
    moe_layer_forward_noalloc,
    moe_layer_forward_nvfp4,
    moe_permute,
    moe_quantize_mxfp8,
    moe_router_topk,
    moe_set_kernel_events,
    moe_set_wait_test,
    moe_workspace_status,
    moe_workspace_bytes,
    status_str,
    workspace,
)
