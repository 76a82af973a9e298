"""Device buffers for callers of the C ABI: torch allocates, the library
computes.

``dev`` copies a seeded host tensor (``inputs.Tensor``) to the GPU bit for
bit; ``empty`` / ``empty_f32`` allocate uninitialised device tensors of a
library dtype code.  Nothing here computes any part of the method.
"""

import numpy as np

from .inputs import BF16, F16, F32


def torch_dtype(dtype):
    import torch
    return {F32: torch.float32, F16: torch.float16, BF16: torch.bfloat16}[dtype]


def dev(t):
    """inputs.Tensor -> device tensor holding exactly the stored values."""
    import torch
    s = np.ascontiguousarray(t.storage)
    if t.dtype == BF16:
        return torch.from_numpy(s.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(s).cuda()


def empty(shape, dtype):
    import torch
    return torch.empty(shape, dtype=torch_dtype(dtype), device="cuda")


def empty_f32(shape):
    import torch
    return torch.empty(shape, dtype=torch.float32, device="cuda")
