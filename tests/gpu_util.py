"""Host <-> device helpers for the GPU tests (torch only allocates and copies)."""
import numpy as np
import torch

import reduced_query_head_amd as sqa


def to_device(a):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if a.dtype == np.uint16:
        t = t.view(torch.bfloat16)
    return t.to("cuda")


def run(q, k, v, scale, causal, out=None):
    """Run the HIP kernel on host arrays; returns the device output tensor."""
    dq, dk, dv = to_device(q), to_device(k), to_device(v)
    o = sqa.attn_fwd(dq, dk, dv, out=out, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return o


def to_host_f64(t):
    return t.float().cpu().numpy().astype(np.float64)


def to_host_bits(t):
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.cpu().numpy()
