"""int8_weight_moe_amd: the forward pass of a mixture-of-experts feed-forward
layer with int8 expert weights (the ExpertsInt8 scheme of the Jamba-1.5
paper) on AMD MI355X (gfx950).

The work is done by hand-written HIP kernels behind the C ABI of
libmoe_int8.so (include/moe_int8.h); `ops` is a thin ctypes binding that
takes torch tensors for device memory and streams.
"""
from ._lib import LIB_PATH, MOE_W_BF16, MOE_W_FP8, MOE_W_INT8, MoeError, load  # noqa: F401
from .ops import (Int8Experts, MoeLayer, moe_combine, moe_expert_down, moe_expert_ffn, moe_expert_gate_up,  # noqa: F401
                  moe_forward, moe_forward_noalloc, moe_mlp_forward, moe_pack_rows, moe_permute, moe_quantize_rows,
                  moe_quantize_pack_rows, moe_quantize_rows_fp8, moe_route, pack_bf16_experts, pack_experts,
                  quantize_experts,
                  quantize_experts_fp8)

__all__ = ["Int8Experts", "MoeLayer", "moe_route", "moe_permute", "moe_expert_ffn", "moe_expert_gate_up", "moe_expert_down", "moe_combine", "moe_forward", "moe_forward_noalloc", "moe_mlp_forward",
           "moe_quantize_rows", "moe_quantize_rows_fp8", "moe_quantize_pack_rows", "quantize_experts_fp8", "moe_pack_rows", "pack_experts", "pack_bf16_experts", "quantize_experts", "MoeError", "load",
           "LIB_PATH", "MOE_W_INT8", "MOE_W_BF16", "MOE_W_FP8"]
