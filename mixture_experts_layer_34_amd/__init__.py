"""DeepSeekMoE layer forward on one AMD MI355X (gfx950).

The compute path is libmoe.so (hand-written HIP, C ABI in include/moe.h);
this package is its ctypes binding plus device-memory plumbing with torch.
Importing it fails when the library is not built.
"""
from ._native import (MOE_BF16, MOE_F32, MOE_MAX_EXPERTS, MOE_MAX_TOPK, MOE_NO_RESIDUAL,
                      MOE_NO_SHARED, MoeError, moe_combine, moe_grouped_ffn, moe_layer_fwd,
                      moe_permute, moe_problem, moe_route, moe_status_str, moe_workspace_bytes,
                      problem)

__all__ = ["MOE_BF16", "MOE_F32", "MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_NO_RESIDUAL",
           "MOE_NO_SHARED", "MoeError", "moe_combine", "moe_grouped_ffn", "moe_layer_fwd",
           "moe_permute", "moe_problem", "moe_route", "moe_status_str", "moe_workspace_bytes",
           "problem"]
