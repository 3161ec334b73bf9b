"""ctypes view of the C ABI in include/moe.h.  Argument marshalling only."""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, c_char_p, c_float, c_int, c_int32, c_uint32, c_uint64, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libqreb_moe.so")

MOE_OK, MOE_EINVAL, MOE_EUNSUPPORTED, MOE_ENOMEM, MOE_EBADRECORD, MOE_ESTATE, MOE_EHIP = \
    0, -1, -2, -3, -4, -5, -6
MOE_BF16, MOE_F32 = 1, 2
MOE_F_SHARED = 1
MOE_F_RMSNORM = 2
MOE_F_VERIFY = 4
MOE_NOALLOC_SCRATCH_BYTES = 64 << 20

# every function include/moe.h declares
EXPORTED = ("moe_workspace_bytes", "moe_open", "moe_set_weights", "moe_forward",
            "moe_forward_noalloc", "moe_crc32", "moe_set_cache", "moe_cache_stats",
            "moe_rvq_workspace_bytes", "moe_rvq_gemv",
            "moe_router_logits", "moe_set_path_rows", "moe_set_narrow_split", "moe_close",
            "moe_strerror", "moe_last_error", "moe_check_record_header", "moe_debug_dequant",
            "moe_profile_start", "moe_profile_start_slots", "moe_profile_read")
# kernel timing slots of moe_profile_read (the last one is reserved)
PROFILE_SLOTS = ("router", "gemv_up", "gemv_down", "mfma_up", "mfma_down", "combine",
                 "cache", "reserved7")
MOE_CACHE_PREFETCH = 1


def cache_prefetch_top(p):
    """MOE_CACHE_PREFETCH_TOP(p): prefetch depth in bits 8-15 of the cache flags."""
    return (int(p) & 0xFF) << 8
CACHE_STATS = ("forwards", "selected", "demand_hits", "demand_misses", "demand_bytes",
               "prefetched", "prefetch_bytes", "prefetch_used", "prefetch_evicted_unused")


class MoeConfig(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("hidden", c_int32), ("n_experts", c_int32),
                ("top_k", c_int32), ("inter", c_int32), ("shared_inter", c_int32),
                ("group", c_int32), ("max_tokens", c_int32), ("device", c_int32),
                ("flags", c_uint32)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("struct_size", c_uint32), ("router", c_void_p), ("router_bias", c_void_p),
                ("bank", c_void_p), ("record_stride", c_uint64), ("shared_record", c_void_p),
                ("workspace", c_void_p), ("workspace_bytes", c_uint64)]


_lib = None


def load() -> ctypes.CDLL:
    """Load the in-tree HIP library; there is no fallback if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run "
                           "`python -m quantized_routed_expert_bit_amd.build` first")
    lib = ctypes.CDLL(LIB_PATH)
    P = POINTER
    lib.moe_workspace_bytes.argtypes = [P(MoeConfig)]
    lib.moe_workspace_bytes.restype = c_uint64
    lib.moe_open.argtypes = [P(MoeConfig), P(c_void_p)]
    lib.moe_open.restype = c_int
    lib.moe_set_weights.argtypes = [c_void_p, P(MoeWeights), c_void_p]
    lib.moe_set_weights.restype = c_int
    lib.moe_forward.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                c_void_p, c_void_p, c_void_p, c_void_p]
    lib.moe_forward.restype = c_int
    lib.moe_forward_noalloc.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p,
                                        c_void_p, c_void_p, c_void_p]
    lib.moe_forward_noalloc.restype = c_int
    lib.moe_router_logits.argtypes = [c_void_p, c_void_p, c_int32, c_int32, c_void_p, c_void_p]
    lib.moe_router_logits.restype = c_int
    lib.moe_set_path_rows.argtypes = [c_void_p, c_int32, c_int32]
    lib.moe_set_path_rows.restype = c_int
    lib.moe_set_narrow_split.argtypes = [c_void_p, c_int32]
    lib.moe_set_narrow_split.restype = c_int
    lib.moe_close.argtypes = [c_void_p]
    lib.moe_close.restype = None
    lib.moe_strerror.argtypes = [c_int]
    lib.moe_strerror.restype = c_char_p
    lib.moe_last_error.argtypes = [c_void_p]
    lib.moe_last_error.restype = c_char_p
    lib.moe_check_record_header.argtypes = [c_void_p, c_uint64, P(MoeConfig), c_int32, c_uint64]
    lib.moe_check_record_header.restype = c_int
    lib.moe_debug_dequant.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_void_p]
    lib.moe_debug_dequant.restype = c_int
    lib.moe_set_cache.argtypes = [c_void_p, c_void_p, c_uint64, c_int32, c_uint32, c_void_p]
    lib.moe_set_cache.restype = c_int
    lib.moe_cache_stats.argtypes = [c_void_p, P(c_uint64), c_int32, c_void_p]
    lib.moe_cache_stats.restype = c_int
    lib.moe_rvq_workspace_bytes.argtypes = [c_int32, c_int32, c_int32, c_int32]
    lib.moe_rvq_workspace_bytes.restype = c_uint64
    lib.moe_rvq_gemv.argtypes = [c_void_p, c_int32, c_int32, c_int32, c_void_p, c_uint64, c_int32,
                                 c_int32, c_void_p, c_void_p, c_void_p, c_uint64, c_void_p]
    lib.moe_rvq_gemv.restype = c_int
    lib.moe_crc32.argtypes = [c_void_p, c_uint64, P(c_uint32), c_void_p]
    lib.moe_crc32.restype = c_int
    lib.moe_profile_start.argtypes = [c_void_p, c_int32]
    lib.moe_profile_start.restype = c_int
    lib.moe_profile_start_slots.argtypes = [c_void_p, c_int32, c_uint32]
    lib.moe_profile_start_slots.restype = c_int
    lib.moe_profile_read.argtypes = [c_void_p, P(c_float), P(c_int32), c_int32]
    lib.moe_profile_read.restype = c_int
    _lib = lib
    return lib


def make_config(hidden, n_experts, top_k, inter, shared_inter=0, max_tokens=1, device=0,
                rmsnorm=False, verify=False):
    return MoeConfig(ctypes.sizeof(MoeConfig), hidden, n_experts, top_k, inter,
                     shared_inter, 64, max_tokens, device,
                     (MOE_F_SHARED if shared_inter else 0) | (MOE_F_RMSNORM if rmsnorm else 0)
                     | (MOE_F_VERIFY if verify else 0))
