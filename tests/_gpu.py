"""Helpers for the GPU parity tests: move seeded numpy inputs to the device,
run the library's calls through the C ABI, bring results back as numpy."""
import sys

import numpy as np


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_mod():
    import torch
    return torch


def to_dev(a):
    """numpy -> cuda tensor.  uint16 arrays are bf16 bit patterns -> bfloat16."""
    torch = torch_mod()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(a).cuda()


def to_host(t, dtype: str = None):
    """cuda tensor -> numpy; bfloat16 comes back as uint16 bit patterns."""
    torch = torch_mod()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()


def filled(shape, dtype, byte: int):
    """A device tensor whose every byte is ``byte`` (to expose unwritten outputs)."""
    torch = torch_mod()
    t = torch.empty(shape, dtype=dtype, device="cuda")
    t.view(torch.uint8).fill_(byte)
    return t


def act_dtype(dtype: str):
    torch = torch_mod()
    return torch.float16 if dtype == "fp16" else torch.bfloat16


def act_host_to_f64(a, dtype):
    import oracle as O
    return O.act_to_f64(a, dtype)
