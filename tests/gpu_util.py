"""Helpers shared by the GPU tests: device buffers and host round trips.

Inputs come from attention_fa2_tiles_amd.inputs (seeded, rounded to the
storage dtype); the same stored values, upcast to float64, go to the oracle.
All device work goes through the C ABI (attention_fa2_tiles_amd.lib); torch is
only used to allocate device memory and copy it to and from the host.
"""

import sys

import numpy as np
import pytest

from attention_fa2_tiles_amd import lib
from attention_fa2_tiles_amd.devbuf import dev, empty, empty_f32, torch_dtype  # noqa: F401 (re-exported)
from attention_fa2_tiles_amd.inputs import F16, F32


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    lib.load()  # raises if the HIP library is missing: there is no fallback
    return torch


def filled(shape, dtype, value=float("nan")):
    """Output buffers start as NaN so that an element the kernel never
    writes cannot pass a comparison by accident."""
    t = empty(shape, dtype)
    t.fill_(value)
    return t


GUARD_ELEMS = 4096
_guards = []


def guarded(shape, dtype, value=float("nan")):
    """An output buffer placed between two guard regions of GUARD_ELEMS
    elements filled with a sentinel; check_guards() verifies that no kernel
    wrote outside the buffer."""
    import torch
    n = 1
    for x in shape:
        n *= x
    flat = torch.empty(n + 2 * GUARD_ELEMS, dtype=torch_dtype(dtype), device="cuda")
    flat.fill_(-12345.0 if dtype != F16 else -1234.0)
    t = flat[GUARD_ELEMS:GUARD_ELEMS + n].view(shape)
    t.fill_(value)
    _guards.append(flat)
    return t


def guarded_f32(shape):
    return guarded(shape, F32)


def check_guards():
    import torch
    torch.cuda.synchronize()
    bad = []
    for flat in _guards:
        head = flat[:GUARD_ELEMS].float()
        tail = flat[-GUARD_ELEMS:].float()
        sentinel = head[0].item()
        if not (torch.all(head == sentinel) and torch.all(tail == sentinel)):
            bad.append(flat.numel())
    _guards.clear()
    assert not bad, f"a kernel wrote outside its output buffer ({len(bad)} buffers)"


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()
