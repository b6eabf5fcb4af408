"""Host-to-device upload of the seeded inputs (plumbing only)."""
from __future__ import annotations

import numpy as np
import torch

from . import synth


def dev(a: np.ndarray, dtype: str, device: str = "cuda") -> torch.Tensor:
    """float32 array (holding bf16 values when dtype is "bf16") -> device tensor."""
    a = np.ascontiguousarray(a, np.float32)
    if dtype == "bf16":
        bits = synth.bf16_bits(a).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(a).to(device)


def dev32(a, device: str = "cuda"):
    """float32 array -> fp32 device tensor (None stays None)."""
    if a is None:
        return None
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(device)
