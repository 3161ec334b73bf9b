"""Moving the synthetic inputs onto the GPU (torch supplies the device
memory).  No layer arithmetic: bytes are copied as they are."""
from __future__ import annotations

import numpy as np

from .gen import LayerInputs

__all__ = ["bf16_tensor", "upload_layer"]


def bf16_tensor(bits: np.ndarray, device):
    """bf16 bit patterns (uint16) -> a bfloat16 device tensor of the same shape."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def upload_layer(li: LayerInputs, device):
    """Router, bias, bank and shared record as device tensors.  Records are
    generated one at a time into a pinned staging buffer, so banks larger than
    host memory stream through."""
    import torch
    sh = li.shape
    stride = li.stride
    router = torch.from_numpy(li.router()).to(device)
    bias = li.router_bias()
    bias_t = None if bias is None else torch.from_numpy(bias).to(device)
    bank = torch.empty(sh.n_experts * stride, dtype=torch.uint8, device=device)
    stage = torch.empty(stride, dtype=torch.uint8, pin_memory=True)
    for e in range(sh.n_experts):
        stage.numpy()[:] = li.record(e)
        bank[e * stride:(e + 1) * stride].copy_(stage, non_blocking=False)
    shared = None
    if sh.has_shared:
        shared = torch.from_numpy(li.shared_record()).to(device)
    return dict(router=router, bias=bias_t, bank=bank, stride=stride, shared=shared)
