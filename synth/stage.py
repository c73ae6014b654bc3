"""Copy seeded inputs to the GPU in the layouts the H2O library reads.

prompt  : q, k, v as [B, H, P, d]
decode  : q, k, v as [T, B, H, d], so one decode step's inputs are a contiguous
          [B, H, d] slice.
bf16 workloads travel as their bit patterns and are reinterpreted as
torch.bfloat16 on the device, so the GPU sees exactly the generator's bytes.
"""
import numpy as np

from . import gen
from .configs import Workload


def to_torch(arr: np.ndarray, wl: Workload, device):
    import torch
    if wl.kv_dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(device)
    return torch.from_numpy(arr).to(device)


def stage_prompt(wl: Workload, device, prompt=None):
    P = wl.prompt if prompt is None else prompt
    return tuple(to_torch(x, wl, device) for x in gen.batch_storage(wl, 0, P))


def stage_decode(wl: Workload, s0: int, s1: int, device, prompt=None):
    """Decode-step inputs for steps [s0, s1) (positions prompt+s0 .. prompt+s1-1)."""
    P = wl.prompt if prompt is None else prompt
    out = []
    for x in gen.batch_storage(wl, P + s0, P + s1):
        out.append(to_torch(np.ascontiguousarray(np.moveaxis(x, 2, 0)), wl, device))
    return tuple(out)
