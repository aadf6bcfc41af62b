"""Device-memory plumbing: numpy inputs to torch device tensors and output
buffers for the C ABI.  No layer arithmetic happens here."""
from __future__ import annotations

import numpy as np
import torch

from ._native import moe_problem, moe_workspace_bytes


def to_device(a: np.ndarray | None, device="cuda") -> torch.Tensor | None:
    """bf16 bit patterns (uint16) become bfloat16 tensors, float32 stays."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def to_host_f32(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy()


def torch_dtype(p: moe_problem):
    return torch.bfloat16 if p.dtype == 1 else torch.float32


def workspace(p: moe_problem, device="cuda") -> torch.Tensor:
    nbytes = moe_workspace_bytes(p)
    if nbytes == 0:
        raise ValueError("invalid problem")
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def route_outputs(p: moe_problem, n: int, k: int, device="cuda") -> dict:
    return dict(topk_idx=torch.empty((p.T, k), dtype=torch.int32, device=device),
                topk_gate=torch.empty((p.T, k), dtype=torch.float32, device=device),
                counts=torch.empty(n, dtype=torch.int32, device=device),
                f=torch.empty(n, dtype=torch.float32, device=device),
                P=torch.empty(n, dtype=torch.float32, device=device))
