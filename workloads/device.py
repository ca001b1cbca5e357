"""Moving the seeded inputs to and from the GPU (marshalling only, no arithmetic of the method).

bf16 workloads are already bf16-rounded in float32, so the conversion to torch.bfloat16 is
exact; fp8 workloads are uint8 E4M3 codes and travel unchanged.
"""
from __future__ import annotations

import numpy as np

__all__ = ["to_device", "to_host", "codes_to_device"]


def to_device(a, dtype: str = "bf16"):
    """numpy float32 -> contiguous GPU tensor of dtype "bf16", "f16" or "f32"."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    if dtype == "bf16":
        t = t.to(torch.bfloat16)
    elif dtype == "f16":
        t = t.to(torch.float16)
    elif dtype != "f32":
        raise ValueError(f"unknown dtype {dtype!r}")
    return t.cuda()


def codes_to_device(a):
    """numpy uint8 codes (E4M3) -> contiguous GPU uint8 tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def to_host(t) -> np.ndarray:
    """GPU tensor -> float32 numpy array."""
    return t.detach().float().cpu().numpy()
