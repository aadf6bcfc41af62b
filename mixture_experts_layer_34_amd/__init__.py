"""DeepSeekMoE layer (forward and backward) on one AMD MI355X (gfx950).

The compute path is libmoe.so (hand-written HIP, C ABI in include/moe.h);
this package is its ctypes binding plus device-memory plumbing with torch.
The binding loads on first use and raises ImportError when the library is
not built (python -m mixture_experts_layer_34_amd.build); there is no
fallback.
"""
import importlib

_EXPORTS = ("MOE_BF16", "MOE_F32", "MOE_MAX_EXPERTS", "MOE_MAX_TOPK", "MOE_NO_RESIDUAL",
            "MOE_NO_SHARED", "MOE_PACKED_WEIGHTS", "MoeError", "moe_combine",
            "moe_grouped_ffn", "moe_layer_fwd", "moe_layer_fwd_marked", "moe_layer_kernels",
            "moe_last_hip_error", "moe_pack_weights", "moe_permute", "moe_problem", "moe_route",
            "moe_status_str", "moe_workspace_bytes", "problem", "moe_layer_bwd",
            "moe_layer_bwd_marked", "moe_layer_bwd_kernels", "moe_bwd_workspace_bytes",
            "moe_train_workspace_bytes", "MOE_SAVE_FOR_BACKWARD", "moe_layer_fwd_noalloc",
            "MOE_NOALLOC_SCRATCH_BYTES", "moe_balance_loss")
__all__ = list(_EXPORTS)


def __getattr__(name):
    if name in _EXPORTS:
        native = importlib.import_module("._native", __name__)
        return getattr(native, name)
    raise AttributeError(name)
