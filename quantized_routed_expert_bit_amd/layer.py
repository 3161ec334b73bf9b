"""MoE layer object over the C ABI.  PyTorch supplies device memory and the
current stream; every step of the layer runs in the HIP library."""
from __future__ import annotations

import ctypes

import torch

from . import _lib as L


class MoEError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{msg} (status {code})")
        self.code = code


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


class MoELayer:
    """One routed-expert layer: router (8-bit), top-k, 4-bit experts, combine."""

    def __init__(self, hidden, n_experts, top_k, inter, shared_inter=0, max_tokens=1,
                 device=0, rmsnorm=False, verify=False):
        self.lib = L.load()
        self.cfg = L.make_config(hidden, n_experts, top_k, inter, shared_inter, max_tokens,
                                 device, rmsnorm, verify)
        self.hidden, self.n_experts, self.top_k = hidden, n_experts, top_k
        self.max_tokens = max_tokens
        self.device = torch.device("cuda", device)
        self.ctx = ctypes.c_void_p()
        rc = self.lib.moe_open(ctypes.byref(self.cfg), ctypes.byref(self.ctx))
        if rc != 0:
            raise MoEError(rc, f"moe_open: {self.lib.moe_strerror(rc).decode()}")
        self.workspace_bytes = int(self.lib.moe_workspace_bytes(ctypes.byref(self.cfg)))
        # the library's defaults
        self.mfma_min_rows, self.wide_min_rows = (3 if hidden >= 4096 else 4), 24
        self._keep = ()

    def _check(self, rc, what):
        if rc != 0:
            msg = self.lib.moe_last_error(self.ctx).decode() or self.lib.moe_strerror(rc).decode()
            raise MoEError(rc, f"{what}: {msg}")

    def set_weights(self, router, bank, record_stride, shared=None, router_bias=None,
                    workspace=None, no_workspace=False):
        """Bind the weights.  `workspace` defaults to a new device tensor;
        with no_workspace=True none is bound and only forward_noalloc runs."""
        if workspace is None and not no_workspace:
            workspace = torch.empty(self.workspace_bytes, dtype=torch.uint8, device=self.device)
        w = L.MoeWeights(ctypes.sizeof(L.MoeWeights), _ptr(router), _ptr(router_bias),
                         _ptr(bank), record_stride, _ptr(shared), _ptr(workspace),
                         0 if workspace is None else workspace.numel())
        self._keep = (router, bank, shared, router_bias, workspace)
        self._stride = record_stride
        self._check(self.lib.moe_set_weights(self.ctx, ctypes.byref(w), _stream()),
                    "moe_set_weights")
        return self

    @staticmethod
    def _dtype(x):
        if x.dtype == torch.bfloat16:
            return L.MOE_BF16
        if x.dtype == torch.float32:
            return L.MOE_F32
        raise TypeError("x must be bfloat16 or float32")

    def forward(self, x, return_selection=False, lookahead=None, y=None, residual=None):
        """y = layer(x), or residual + layer(x); y may be the residual tensor."""
        T = x.shape[0]
        x = x.contiguous()
        if y is None:
            y = torch.empty((T, self.hidden), dtype=torch.float32, device=self.device)
        ids = p = None
        if return_selection:
            ids = torch.empty((T, self.top_k), dtype=torch.int32, device=self.device)
            p = torch.empty((T, self.top_k), dtype=torch.float32, device=self.device)
        nxt = lookahead.ctx if lookahead is not None else None
        self._check(self.lib.moe_forward(self.ctx, _ptr(x), self._dtype(x), T, _ptr(y),
                                         _ptr(residual), _ptr(ids), _ptr(p), nxt, _stream()),
                    "moe_forward")
        return (y, ids, p) if return_selection else y

    __call__ = forward

    def forward_noalloc(self, x, return_selection=False, y=None, residual=None):
        """forward() on the library's static scratch (moe_forward_noalloc):
        the library allocates nothing; y, ids and p are the caller's (created
        here only when not given)."""
        T = x.shape[0]
        x = x.contiguous()
        if y is None:
            y = torch.empty((T, self.hidden), dtype=torch.float32, device=self.device)
        ids = p = None
        if return_selection:
            ids = torch.empty((T, self.top_k), dtype=torch.int32, device=self.device)
            p = torch.empty((T, self.top_k), dtype=torch.float32, device=self.device)
        self._check(self.lib.moe_forward_noalloc(self.ctx, _ptr(x), self._dtype(x), T, _ptr(y),
                                                 _ptr(residual), _ptr(ids), _ptr(p), _stream()),
                    "moe_forward_noalloc")
        return (y, ids, p) if return_selection else y

    def router_logits(self, x):
        T = x.shape[0]
        x = x.contiguous()
        out = torch.empty((T, self.n_experts), dtype=torch.float32, device=self.device)
        self._check(self.lib.moe_router_logits(self.ctx, _ptr(x), self._dtype(x), T, _ptr(out),
                                               _stream()), "moe_router_logits")
        return out

    def profile_start(self, max_calls, slots=None):
        """Kernel timing for the next max_calls forwards: every slot, or only
        the named ones (L.PROFILE_SLOTS names)."""
        if slots is None:
            self._check(self.lib.moe_profile_start(self.ctx, max_calls), "moe_profile_start")
            return
        mask = 0
        for n in slots:
            mask |= 1 << L.PROFILE_SLOTS.index(n)
        self._check(self.lib.moe_profile_start_slots(self.ctx, max_calls, mask),
                    "moe_profile_start_slots")

    def profile_read(self):
        """-> ({slot name: average ms per launch}, number of profiled forwards)."""
        n = len(L.PROFILE_SLOTS)
        arr = (ctypes.c_float * n)()
        calls = ctypes.c_int32()
        self._check(self.lib.moe_profile_read(self.ctx, arr, ctypes.byref(calls), n),
                    "moe_profile_read")
        return ({k: v for k, v in zip(L.PROFILE_SLOTS, list(arr)) if not k.startswith("reserved")},
                calls.value)

    def set_cache(self, n_slots, prefetch=False, slots=None, prefetch_top=None):
        """Give the layer an expert cache of n_slots records in HBM (a new
        device tensor unless `slots` is given); 0 removes it.  prefetch: the
        previous layer's lookahead prefetches into it (prefetch_top: only the
        that many highest-ranked predictions of each token; None: all k)."""
        if n_slots and slots is None:
            slots = torch.empty(n_slots * self._stride, dtype=torch.uint8, device=self.device)
        self._slots = slots
        flags = L.MOE_CACHE_PREFETCH if prefetch else 0
        if prefetch_top is not None:
            flags |= L.cache_prefetch_top(prefetch_top)
        self._check(self.lib.moe_set_cache(self.ctx, _ptr(slots) if n_slots else None,
                                           0 if slots is None else slots.numel(), n_slots, flags,
                                           _stream()),
                    "moe_set_cache")
        return self

    def cache_stats(self):
        """{counter name: value} of the expert cache (moe_cache_stats)."""
        arr = (ctypes.c_uint64 * 16)()
        self._check(self.lib.moe_cache_stats(self.ctx, arr, 16, _stream()), "moe_cache_stats")
        return dict(zip(L.CACHE_STATS, list(arr)))

    def set_path_rows(self, mfma_min_rows, wide_min_rows=None):
        if wide_min_rows is None:
            wide_min_rows = max(mfma_min_rows, self.wide_min_rows)
        self._check(self.lib.moe_set_path_rows(self.ctx, mfma_min_rows, wide_min_rows),
                    "moe_set_path_rows")
        self.mfma_min_rows, self.wide_min_rows = mfma_min_rows, wide_min_rows

    def set_narrow_split(self, min_workgroups):
        """32-row tiles split by columns from min_workgroups workgroups on
        (0: always, 2**31 - 1: never), else by K."""
        self._check(self.lib.moe_set_narrow_split(self.ctx, min_workgroups), "moe_set_narrow_split")

    def close(self):
        if self.ctx:
            self.lib.moe_close(self.ctx)
            self.ctx = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def rvq_gemv(x, mats, rows, codebooks, n_mats=1, mat_stride=0, workspace=None, y=None):
    """y [n_mats, T, rows] = W_m x for 3-bit residual-VQ matrices (moe_rvq_gemv).
    x: bf16 or fp32 [T, K] device tensor; mats: uint8 device tensor holding the
    n_mats tiled matrices at mat_stride bytes; codebooks: fp16 [3, 256, 8]."""
    lib = L.load()
    T, K = x.shape
    x = x.contiguous()
    need = int(lib.moe_rvq_workspace_bytes(T, K, rows, n_mats))
    if need == 0:
        raise MoEError(L.MOE_EINVAL, "moe_rvq_workspace_bytes: invalid shape")
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=x.device)
    if y is None:
        y = torch.empty((n_mats, T, rows), dtype=torch.float32, device=x.device)
    rc = lib.moe_rvq_gemv(_ptr(x), MoELayer._dtype(x), T, K, _ptr(mats), mat_stride, n_mats, rows,
                          _ptr(codebooks), _ptr(y), _ptr(workspace), workspace.numel(), _stream())
    if rc != 0:
        raise MoEError(rc, "moe_rvq_gemv")
    return y


def crc32(t):
    """CRC-32 (zlib's) of a contiguous device tensor's bytes, by the library's
    GPU kernel (moe_crc32)."""
    lib = L.load()
    out = ctypes.c_uint32()
    rc = lib.moe_crc32(_ptr(t), t.numel() * t.element_size(), ctypes.byref(out), _stream())
    if rc != 0:
        raise MoEError(rc, "moe_crc32")
    return out.value


def debug_dequant(tiles, bits, rows, cols):
    lib = L.load()
    out = torch.empty((rows, cols), dtype=torch.float32, device=tiles.device)
    rc = lib.moe_debug_dequant(_ptr(tiles), bits, rows, cols, _ptr(out), _stream())
    if rc != 0:
        raise MoEError(rc, "moe_debug_dequant")
    return out
