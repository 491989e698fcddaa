"""MI355X-native routed int4 MoE expert layer (HIP kernels behind a C ABI).

The library (``libmoe_q4.so``, built from ``csrc/`` by ``build.py``) computes
router logits and top-k gates, groups token rows by expert, runs the int4
SwiGLU experts (fused-dequant GEMVs for decode, matrix-core grouped GEMMs for
prefill), the gate-weighted combine and the int8 shared expert.  This package is its thin Python
binding: ``_lib`` mirrors the C entry points, ``layer`` holds buffers.
"""
from ._lib import (ASYM_G64, SYM_G128, FP8_B128, NVFP4, WS_DECODE, WS_GROUP, WS_PREFILL, WS_ROUTE, EXPORTS, MoeQ4Error,
                   error_string, layer_struct, lib, moe_q4_decode, moe_q4_dequant, moe_q4_group,
                   moe_q4_prefill, moe_q4_residual_bf16, moe_q4_route, workspace_size,
                   moe_q4_decode_timed, moe_q4_prefill_timed, STAGE_EVENTS, WS_FORWARD, moe_q4_forward,
                   moe_q4_forward_timed, moe_q4_workspace_init, WS_SHARED, SharedExpert, shared_struct,
                   moe_q4_shared, moe_q4_dequant_int8, moe_q4_forward_ex, moe_q4_shared_timed,
                   moe_q4_prefill_pack_size, moe_q4_prefill_pack, prefill_pack,
                   moe_q4_forward_noalloc, NOALLOC_SCRATCH_BYTES, moe_q4_forward_det, WS_FORWARD_DET,
                   FRAME_MAX_LANES, frame_workspace_size, moe_q4_frame)
from .layer import MoeQ4Layer

__all__ = ["ASYM_G64", "SYM_G128", "FP8_B128", "NVFP4", "WS_DECODE", "WS_GROUP", "WS_PREFILL", "WS_ROUTE", "EXPORTS", "MoeQ4Error",
           "error_string", "layer_struct", "lib", "moe_q4_decode", "moe_q4_dequant", "moe_q4_group",
           "moe_q4_prefill", "moe_q4_residual_bf16", "moe_q4_route", "workspace_size", "MoeQ4Layer",
           "moe_q4_decode_timed", "moe_q4_prefill_timed", "STAGE_EVENTS", "WS_FORWARD", "moe_q4_forward",
           "moe_q4_forward_timed", "moe_q4_workspace_init", "WS_SHARED", "SharedExpert", "shared_struct",
           "moe_q4_shared", "moe_q4_dequant_int8", "moe_q4_forward_ex", "moe_q4_shared_timed",
           "moe_q4_prefill_pack_size", "moe_q4_prefill_pack", "prefill_pack",
           "moe_q4_forward_noalloc", "NOALLOC_SCRATCH_BYTES", "moe_q4_forward_det", "WS_FORWARD_DET",
           "FRAME_MAX_LANES", "frame_workspace_size", "moe_q4_frame"]
