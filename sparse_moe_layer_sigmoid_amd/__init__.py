"""MI355X-native (gfx950) forward pass of one DeepSeekMoE layer: sigmoid routing with the
aux-loss-free bias and its load-driven update, bf16 and FP8 (E4M3, 1x128 / 128x128 tiles with
f32 or power-of-two E8M0 scales) paths.

The compute lives in ``libmoe.so`` (hand-written HIP kernels behind a C ABI, see
``include/moe.h``); ``_lib`` binds it with ctypes and ``layer.MoELayer`` sequences the
calls.  Nothing here falls back to a CPU implementation.
"""
from ._lib import (EXPORTS, LIB_PATH, MoeError, fp8_quant_128x128, fp8_quant_128x128_e8m0,  # noqa: F401
                   fp8_quant_1x128, fp8_quant_1x128_e8m0, lib, moe_bias_update, moe_combine, moe_grouped_gemm,
                   moe_permute, moe_route, moe_route_noalloc)
from .layer import MoELayer  # noqa: F401
from .state import load_bias_state, save_bias_state  # noqa: F401
