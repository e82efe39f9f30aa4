"""gfx950 fused MoE layer forward: Python binding of libmoe.so.

Argument marshalling only. Every step of the layer runs in the HIP kernels
of ``libmoe.so`` (C ABI in ``include/moe.h``); PyTorch supplies device
memory and the current stream. Importing this package fails loudly if the
library has not been built; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes as C
import os

from ._binding import (  # noqa: F401
    ACT_GEGLU, ACT_REGLU, ACT_RELU2, ACT_SWIGLU, ACT_SWIGLU_BOUNDED, ACT_SWIGLU_OAI,
    A_BF16, A_FP8_G128, A_FP8_TOKEN, A_MXFP8_G32, OP_GATEUP_ACT, OP_GATEUP_SWIGLU, OP_PLAIN,
    SCORE_PROBS,
    SCORE_SIGMOID, SCORE_SOFTMAX, W_BF16, W_FP8_BLOCK128, W_FP8_CHANNEL, W_MXFP4, MoeError,
    LayerDesc, Workspace, backward_scratch_size, combine, config_model_params, config_rows,
    dispatch, dispatch_noalloc, expert_backward, grouped_gemm, router_backward,
    layer_forward, library_path, quantize_act, route_topk, symbols)

__all__ = [
    "LayerDesc", "Workspace", "MoeError", "route_topk", "dispatch", "dispatch_noalloc",
    "grouped_gemm",
    "quantize_act", "combine", "layer_forward", "config_rows", "config_model_params", "library_path",
    "symbols", "backward_scratch_size", "expert_backward", "router_backward",
]
