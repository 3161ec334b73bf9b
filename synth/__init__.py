"""Seeded synthetic inputs for the routed-expert MoE layer.

This package produces the *inputs* of the layer (hidden states, the 8-bit
router matrix, the 4-bit expert records and the optional router logit bias)
as plain bytes in the storage format that ``include/moe.h`` specifies, and
copies them to the GPU.  It holds none of the layer's arithmetic: nothing here
dequantizes, multiplies, selects or combines.  Both the CPU oracle and the GPU
library consume what it writes, and neither imports the other.
"""
from .gen import *  # noqa: F401,F403
from .device import bf16_tensor, upload_layer  # noqa: F401
