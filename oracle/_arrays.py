"""Array plumbing for the oracle: exact widening of inputs, bf16 rounding.

No step of the method lives here.  bf16 values are widened exactly to float64;
rounding float32 -> bf16 uses PyTorch's CPU conversion (round to nearest even).
"""

import numpy as np
import torch


def f64(a):
    """Exact float64 copy of a torch tensor (any float dtype) or numpy array."""
    if isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.float64).numpy()
    return np.asarray(a, dtype=np.float64)


def i64(a):
    if isinstance(a, torch.Tensor):
        return a.detach().to("cpu", torch.int64).numpy()
    return np.asarray(a, dtype=np.int64)


def f32_to_bf16(a32):
    """Round a float32 array to bfloat16 (nearest, ties to even) -> torch tensor."""
    return torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
