"""Host <-> device plumbing for the packed layout (torch is used for memory only)."""
from __future__ import annotations

import numpy as np


def to_device(x: np.ndarray, device="cuda"):
    """numpy float32 -> torch.float32, uint16 bf16 bit patterns -> torch.bfloat16,
    int32 -> torch.int32, on `device`."""
    import torch
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(x)).to(device)


def to_host_f64(t) -> np.ndarray:
    """Any float tensor -> float64 numpy (bf16 widens exactly)."""
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def workspace_view(ws, offset: int, count: int, dtype):
    """Typed view of `count` elements at byte `offset` of a uint8 workspace tensor."""
    import torch
    nbytes = count * torch.empty((), dtype=dtype).element_size()
    return ws[offset:offset + nbytes].view(dtype)
