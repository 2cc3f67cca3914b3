"""Helpers shared by the GPU parity tests: moving seeded host inputs to the
device and comparing with the oracle."""

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("needs an MI355X GPU")


def dev_tensor(payload, dtype):
    """Host payload from synth.normal (uint16 bf16 bits or float32) -> cuda."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(payload).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(payload, dtype=np.float32))
    return t.cuda()


def host_f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def bits_u16(t):
    """bf16 device tensor -> uint16 bit patterns on the host."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def say(*args):
    print(*args, flush=True)
