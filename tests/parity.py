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


def oracle_pool():
    """A thread pool for the oracle's expert loop (NumPy releases the GIL in
    its array work), sized to this process's CPU share, at most 16."""
    import os
    from concurrent.futures import ThreadPoolExecutor
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return ThreadPoolExecutor(max(1, min(16, n)))

GAP = 1e-3
REL_FROB = 5e-3
MAX_ABS_RMS = 1e-2


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


bf16_tensor = synth.bf16_tensor
upload_layer = synth.upload_layer


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


def valid_in_band(lg_row: np.ndarray, sel) -> bool:
    """True iff `sel` (k distinct expert ids) is a top-k of the logits up to
    GAP: no unselected expert's logit exceeds a selected one's by more than
    GAP, i.e. min(l[sel]) >= max(l[not sel]) - GAP."""
    sel = np.asarray(sorted(set(int(v) for v in sel)), dtype=np.int64)
    if sel.size == 0 or sel.min() < 0 or sel.max() >= lg_row.size:
        return False
    rest = np.ones(lg_row.size, dtype=bool)
    rest[sel] = False
    if not rest.any():
        return True
    return bool(lg_row[sel].min() >= lg_row[rest].max() - GAP)


def resolve_ids(ref: dict, gpu_ids: np.ndarray):
    """ids the oracle should be evaluated on: the oracle's where the gap exceeds
    GAP (there they must equal the GPU's as sets), the GPU's elsewhere, after
    checking that they are a valid top-k within the GAP band (valid_in_band)."""
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
            assert valid_in_band(lg[t], g), \
                f"token {t}: gpu ids {sorted(g)} are not a top-{k} within {GAP} of the oracle's logits"
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


def check_forward(olayer, x64, y, ids, p, what="", pool=None):
    """Full check of one forward against the oracle; returns (rel, max, n_tie).
    `pool` (an executor) evaluates the oracle's experts concurrently."""
    t0 = time.time()
    ref = olayer.forward(x64, pool=pool)
    use, n_tie = resolve_ids(ref, ids)
    # tokens whose GPU set differs from the oracle's (inside the band only):
    # the oracle is evaluated again on the GPU's selection for those rows
    diff = [t for t in range(ids.shape[0])
            if set(use[t].tolist()) != set(ref["ids"][t].tolist())]
    if diff:
        sub = olayer.forward(x64[diff], logits=ref["logits"][diff], force_ids=use[diff], pool=pool)
        for key in ("y", "ids", "p"):
            ref[key] = ref[key].copy()
            ref[key][diff] = sub[key]
    # p: same experts, compare per expert id
    for t in range(ids.shape[0]):
        m_ref = dict(zip(ref["ids"][t].tolist(), ref["p"][t].tolist()))
        pr = np.array([m_ref[int(e)] for e in ids[t]])
        dp = np.abs(p[t] - pr)
        if dp.max() > 1e-5:
            lg = ref["logits"][t, ids[t]]
            log(f"  {what} token {t}: |dp| max {dp.max():.3e}; ids {ids[t].tolist()}\n"
                f"    p gpu {np.round(p[t], 7).tolist()}\n    p ref {np.round(pr, 7).tolist()}\n"
                f"    logits ref {np.round(lg, 6).tolist()}\n"
                f"    log(p_gpu/p_ref) {np.round(np.log(p[t] / pr), 7).tolist()} gap {ref['gap'][t]:.3e}")
        assert dp.max() <= 1e-5, f"token {t} p mismatch: max |dp| {dp.max():.3e}"
    rel, mx = compare_y(y, ref["y"], what)
    log(f"  {what} ties={n_tie} (other set on {len(diff)}) oracle {time.time() - t0:.1f}s")
    return rel, mx, n_tie
