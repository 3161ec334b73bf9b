"""MI355X (gfx950) routed-expert MoE layer with 4-bit group-64 affine experts.

The layer runs in the HIP library libqreb_moe.so (built in-tree by
``quantized_routed_expert_bit_amd.build``); this package only marshals
arguments to its C ABI (include/moe.h).
"""
from ._lib import (MOE_BF16, MOE_F32, MOE_F_SHARED, MOE_F_RMSNORM, MOE_F_VERIFY, MOE_OK,  # noqa: F401
                   MOE_EINVAL,
                   MOE_EUNSUPPORTED, MOE_ENOMEM, MOE_EBADRECORD, MOE_ESTATE, MOE_EHIP,
                   LIB_PATH, load, make_config)
from .layer import MoELayer, MoEError, crc32, debug_dequant, rvq_gemv  # noqa: F401
