"""Shared helpers for GPU parity tests: upload synthetic layers, compare the
HIP path with the oracle.  Tolerances: expert ids equal (as sets) wherever
the oracle's k-th/(k+1)-th logit gap exceeds 1e-3 (elsewhere the GPU's set must
be a valid top-k within that band, and the output is checked against the
oracle evaluated on the GPU's selection); ||y - y*||_F / ||y*||_F <= 5e-3 and
max |y - y*| <= 1e-2 * RMS(y*)."""
from __future__ import annotations

import sys
import time

import numpy as np

import oracle
import synth

GAP = 1e-3
REL_FROB = 5e-3
MAX_ABS_RMS = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bf16_tensor(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def upload_layer(li: synth.LayerInputs, device, pinned_chunk: int = 64):
    """Router, bias, bank and shared record as device tensors (records are
    generated one at a time, so banks larger than host memory stream through)."""
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


def oracle_layer(li: synth.LayerInputs, cache=True):
    sh = li.shape
    recs = {}

    def get(e):
        if not cache:
            return li.record(e)
        if e not in recs:
            recs[e] = li.record(e)
        return recs[e]
    return oracle.OracleLayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter,
                              li.router(), li.router_bias(), get, li.shared_record())


def resolve_ids(ref: dict, gpu_ids: np.ndarray):
    """ids the oracle should be evaluated on: the oracle's where the gap exceeds
    GAP (there they must equal the GPU's as sets), the GPU's elsewhere, after
    checking those are a valid top-k within the GAP band."""
    ids = ref["ids"].copy()
    lg = ref["logits"]
    k = ids.shape[1]
    n_tie = 0
    for t in range(ids.shape[0]):
        g = set(int(v) for v in gpu_ids[t])
        assert len(g) == k, f"token {t}: duplicate ids {gpu_ids[t]}"
        if ref["gap"][t] > GAP:
            assert g == set(int(v) for v in ref["ids"][t]), \
                f"token {t}: gpu ids {sorted(g)} != oracle {sorted(ref['ids'][t])} (gap {ref['gap'][t]:.3g})"
        else:
            n_tie += 1
            kth = np.sort(lg[t])[::-1][k - 1]
            assert min(lg[t, list(g)]) >= kth - GAP, f"token {t}: gpu ids outside the tie band"
            ids[t] = gpu_ids[t]
    return ids, n_tie


def compare_y(y: np.ndarray, y_ref: np.ndarray, what: str = ""):
    err = y.astype(np.float64) - y_ref
    rel = np.linalg.norm(err) / max(np.linalg.norm(y_ref), 1e-300)
    rms = np.sqrt(np.mean(y_ref ** 2))
    mx = np.abs(err).max() / max(rms, 1e-300)
    log(f"  {what} rel_frob={rel:.3e} max_abs/rms={mx:.3e}")
    assert rel <= REL_FROB, f"{what}: rel-Frobenius {rel:.3e} > {REL_FROB}"
    assert mx <= MAX_ABS_RMS, f"{what}: max-abs/RMS {mx:.3e} > {MAX_ABS_RMS}"
    return rel, mx


def check_forward(olayer, x64, y, ids, p, what=""):
    """Full check of one forward against the oracle; returns (rel, max, n_tie)."""
    t0 = time.time()
    ref = olayer.forward(x64)
    use, n_tie = resolve_ids(ref, ids)
    if n_tie:
        ref = olayer.forward(x64, logits=ref["logits"], force_ids=use)
    # p: same experts, compare per expert id
    for t in range(ids.shape[0]):
        m_ref = dict(zip(ref["ids"][t].tolist(), ref["p"][t].tolist()))
        for j in range(ids.shape[1]):
            assert abs(p[t, j] - m_ref[int(ids[t, j])]) <= 1e-5, f"token {t} p mismatch"
    rel, mx = compare_y(y, ref["y"], what)
    log(f"  {what} ties={n_tie} oracle {time.time() - t0:.1f}s")
    return rel, mx, n_tie
