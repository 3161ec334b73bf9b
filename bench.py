"""Benchmark of the routed-expert MoE layer on one MI355X.

Headline workload: the skewed 8-layer stack at the large-expert shape (hidden
7168, 512 experts, top-16, intermediate 2048, shared expert 2048; 101.5 GB of
expert records, generated on the device), 256 tokens, router logits biased by
the log of a Zipf(1.1) prior, fp32 residual stream, each layer's router also
run on the current input for the next layer (lookahead on).  A step is one
pass of the batch through all eight layers (8 moe_forward calls: router, top-k
and bucketing, gate/up, down, combine with the residual add).  The value is
tokens/s through the stack.

The timed region is K eager steps, bracketed by device synchronisation and
timed with HIP events on the stream they run on; the library's own event pairs
around each kernel in those same steps give the per-kernel durations (a step is
milliseconds of GPU work, so eager launches cost nothing measurable).  The
other workloads (the large decode layer at 1, 8 and 64 tokens, the decode layer
at 1, 4 and 16 tokens, the 2048-token prefill) are reported as extra entries,
each with its fraction of the roofline; they are timed as graph replays, and
their kernels in a separate eager pass.

Prints ONE JSON line (one GPU).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, GB/s
MFMA_F16_PEAK_TFS = 2500.0     # MI355X dense fp16/bf16 MFMA, TFLOP/s
METRIC = "MoE layer tokens/s; decode HBM GB/s and prefill TFLOP/s as % of MI355X peak"
KERNELS = ("router", "gemv_up", "gemv_down", "mfma_up", "mfma_down", "combine")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def record_bytes(h, i):
    """Algorithmic bytes of one expert record: 3*H*I weights at 4.5 bits."""
    return 3 * h * i * 9 // 16


def layer_bytes(sh, T, distinct, x_bytes=2, residual=False):
    """Algorithmic bytes of one forward: the distinct routed records, the
    shared record, the 8-bit router (8.5 bits per weight), x, y (fp32), ids and
    p, and the residual read when the forward adds one."""
    b = distinct * record_bytes(sh.hidden, sh.inter) + sh.n_experts * sh.hidden * 17 / 16
    if sh.has_shared:
        b += record_bytes(sh.hidden, sh.shared_inter)
    b += T * sh.hidden * (x_bytes + 4 + (4 if residual else 0)) + T * sh.top_k * 8
    return b


def layer_flops(sh, T):
    return T * 2 * (sh.top_k * 3 * sh.hidden * sh.inter + 3 * sh.hidden * sh.shared_inter
                    + sh.n_experts * sh.hidden)


def kernel_work(cnt, sh, T, rmin, rwide):
    """Algorithmic bytes and FLOPs per launch of each expert kernel, from the
    rows per expert of one forward.  Experts below wide_min_rows rows (and the
    shared expert below it) run in the streaming launches (gate/up, down),
    which also carry the 32-row matrix-core tiles; the others in the 128-row
    matrix-core launches.  Bytes: each record section once (4.5 bits per
    weight); FLOPs: 2 per weight per row."""
    gu, dn = 2 * sh.hidden * sh.inter, sh.hidden * sh.inter
    w = {k: [0.0, 0.0] for k in ("gemv_up", "gemv_down", "mfma_up", "mfma_down")}
    for c in cnt[cnt > 0]:
        up, down = ("mfma_up", "mfma_down") if c >= rwide else ("gemv_up", "gemv_down")
        w[up][0] += gu * 9 / 16
        w[up][1] += 2 * c * gu
        w[down][0] += dn * 9 / 16
        w[down][1] += 2 * c * dn
    if sh.has_shared:
        gus, dns = 2 * sh.hidden * sh.shared_inter, sh.hidden * sh.shared_inter
        up, down = ("mfma_up", "mfma_down") if T >= rwide else ("gemv_up", "gemv_down")
        w[up][0] += gus * 9 / 16
        w[up][1] += 2 * T * gus
        w[down][0] += dns * 9 / 16
        w[down][1] += 2 * T * dns
    return w


def roofline(kernel, bytes_, flops, us):
    """The kernel's bound is the larger of its two ideal times (bytes at the
    HBM peak, FLOPs at the dense fp16 matrix-core peak)."""
    t_hbm = bytes_ / (HBM_PEAK_GBS * 1e9)
    t_mfma = flops / (MFMA_F16_PEAK_TFS * 1e12)
    if t_mfma > t_hbm:
        ach = flops / (us * 1e-6) / 1e12
        return {"bound": "mfma", "achieved": round(ach, 1), "peak": MFMA_F16_PEAK_TFS,
                "unit": "TFLOP/s", "frac": round(ach / MFMA_F16_PEAK_TFS, 4), "kernel": kernel,
                "flops_per_launch": int(flops), "bytes_per_launch": int(bytes_),
                "avg_launch_us": round(us, 3)}
    ach = bytes_ / (us * 1e-6) / 1e9
    return {"bound": "hbm", "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(ach / HBM_PEAK_GBS, 4), "kernel": kernel, "bytes_per_launch": int(bytes_),
            "flops_per_launch": int(flops), "avg_launch_us": round(us, 3)}


def _code_only(text):
    """C/C++ source without its comments and blank lines, trailing blanks
    stripped (string and character literals kept whole), so that a change to
    the comments alone does not count as a change of the kernels."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            i = n if j < 0 else j + 2
        elif c in "\"'":
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    lines = (ln.rstrip() for ln in "".join(out).splitlines())
    return "\n".join(ln for ln in lines if ln)


def source_sha256():
    """Hash of the kernel sources' code (comments excluded)."""
    h = hashlib.sha256()
    for f in ("moe_kernels.hip", "moe_internal.h"):
        with open(os.path.join(ROOT, "quantized_routed_expert_bit_amd", "csrc", f)) as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()


def measured_traffic(name, path_rows):
    """HBM bytes per launch of a kernel on a workload, from the committed
    rocprofv3 FETCH_SIZE + WRITE_SIZE passes (calibrated against a plain copy);
    None once the kernel sources differ from the ones the counters were taken
    on, or the layers' path thresholds (mfma_min_rows, wide_min_rows: which
    experts the launch carries) differ from the ones they ran with."""
    path = os.path.join(ROOT, "profiles", name)
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ",
                                          "path_rows: ")))
        if source_sha256() != fields["source_sha256"].strip():
            return None
        if [int(v) for v in fields["path_rows"].split()] != [int(v) for v in path_rows]:
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def timed_graph(step, steps):
    """Capture `steps` calls of step(i) in one HIP graph, replay it once
    untimed (upload), then time one replay with HIP events on the stream it
    runs on, between two device synchronisations.  Returns seconds."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    host = time.perf_counter() - t0
    del g
    return e0.elapsed_time(e1) * 1e-3, host


def profiled(layers, step, n_steps, timed=False, slots=None):
    """Average ms per launch of each kernel slot over n_steps eager steps, from
    the library's event pairs (only around the kernels named in `slots`, if
    given; a spin kernel first holds the GPU while the host queues the steps).  Returns ({kernel: ms}, {kernel: launches per step}),
    and with timed=True also the seconds the steps took, from HIP events on the
    current stream around them (after the spin), between synchronisations."""
    import torch
    for m in layers:
        m.profile_start(n_steps * 4, slots)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2.4e9 * 0.05))
    e0.record()
    for i in range(n_steps):
        step(i)
    e1.record()
    torch.cuda.synchronize()
    tot = {k: 0.0 for k in KERNELS}
    n = {k: 0 for k in KERNELS}
    for m in layers:
        avg, calls = m.profile_read()
        for k in KERNELS:
            if avg[k] > 0:
                tot[k] += avg[k] * calls
                n[k] += calls
    out = ({k: tot[k] / n[k] if n[k] else 0.0 for k in KERNELS},
           {k: n[k] / n_steps for k in KERNELS})
    return out + (e0.elapsed_time(e1) * 1e-3,) if timed else out


def host_info():
    info = {"os_cpu_count": os.cpu_count()}
    try:
        info["affinity_cpus"] = len(os.sched_getaffinity(0))
    except AttributeError:
        info["affinity_cpus"] = os.cpu_count()
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                info["cpu_model"] = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        from threadpoolctl import threadpool_info
        info["blas"] = [{k: i.get(k) for k in ("internal_api", "version", "num_threads",
                                                 "threading_layer")}
                        for i in threadpool_info() if i.get("user_api") == "blas"]
    except Exception:
        info["blas"] = None
    return info


# ------------------------------------------------------------- workloads ----

def make_large_layer(dev, cfg, layer, max_tokens, rmsnorm=False):
    """One layer at the large-expert shape, its bank generated on the device."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    wl = synth.WORKLOADS[cfg]
    sh = wl.shape
    bank, stride = synth.gpu_bank(0, cfg, layer, sh.hidden, sh.inter, sh.n_experts, dev)
    shared, _ = synth.gpu_bank(0, cfg, layer, sh.hidden, sh.shared_inter, 1, dev, shared=True)
    router = synth.make_router(0, cfg, layer, sh.hidden, sh.n_experts)
    bias = synth.make_router_bias(0, cfg, layer, sh.n_experts, wl.bias)
    m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max_tokens,
                 rmsnorm=rmsnorm)
    m.set_weights(torch.from_numpy(router).to(dev), bank, stride, shared,
                  None if bias is None else torch.from_numpy(bias).to(dev))
    m._host = dict(router=router, bias=bias, stride=stride)
    return m


def run_stack(args, dev):
    """The 8-layer stack, 256 tokens, lookahead on (the headline)."""
    import torch
    import synth
    wl = synth.WORKLOADS[4]
    sh = wl.shape
    T = wl.batches[0]
    layers = []
    for l in range(wl.layers):
        layers.append(make_large_layer(dev, 4, l, T, rmsnorm=True))
        log(f"  stack layer {l} generated")
    x32 = synth.bf16_tensor(synth.make_hidden(0, 4, T, sh.hidden), dev).float()
    r = torch.empty_like(x32)
    L = len(layers)

    def step(_i):
        # r_1 = x + MoE_0(x); r_{l+1} = r_l + MoE_l(r_l) in place; each layer
        # also runs the next layer's router on its input (lookahead)
        for l, m in enumerate(layers):
            nxt = layers[l + 1] if l + 1 < L else None
            src = x32 if l == 0 else r
            m.forward(src, y=r, residual=src, lookahead=nxt)

    # routing of each layer on the stack's own trajectory
    counts = []
    rr = x32.clone()
    for l, m in enumerate(layers):
        out = torch.empty_like(rr)
        _, ids, _ = m.forward(rr, return_selection=True, y=out, residual=rr)
        counts.append(np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts))
        rr = out
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    # every kernel's duration from an untimed eager pass with the library's
    # event pairs around each launch; the dominant kernel is the one with the
    # largest share of the step
    n_prof = max(4, args.steps // 4)
    kern, per_step = profiled(layers, step, n_prof)
    share = {k: kern[k] * per_step[k] for k in KERNELS}
    dom = max(("gemv_up", "gemv_down", "mfma_up", "mfma_down"), key=lambda k: share[k])
    # the timed region: `steps` eager steps, timed with HIP events on the
    # stream they run on, with event pairs around the dominant kernel only
    # (pairs around all of them cost about 2 % of the step); each step is
    # milliseconds of GPU work, so launching eagerly costs nothing measurable
    kdom, _, el = profiled(layers, step, args.steps, timed=True, slots=(dom,))
    us_step = el * 1e6 / args.steps
    # the same steps captured in one HIP graph and replayed: no launch gaps
    # and no event pairs (the library records no timing events inside a
    # capture), so this is reported beside the headline, not as it
    g_el, _ = timed_graph(step, args.steps)
    rmin, rwide = layers[0].mfma_min_rows, layers[0].wide_min_rows
    work = [kernel_work(c, sh, T, rmin, rwide) for c in counts]
    distinct = [int((c > 0).sum()) for c in counts]
    alg = sum(layer_bytes(sh, T, d, x_bytes=4, residual=True) for d in distinct)
    flops = L * layer_flops(sh, T)
    b = float(np.mean([w[dom][0] for w in work]))
    f = float(np.mean([w[dom][1] for w in work]))
    rl = roofline(dom, b, f, kdom[dom] * 1e3)
    rl["traffic"] = measured_traffic(f"{dom}_stack_hbm_traffic.md", (rmin, rwide))
    res = dict(
        tokens_s=T * args.steps / el, us_per_step=us_step, roofline=rl,
        stack_hbm={"alg_bytes_per_step": int(alg), "GB_s": round(alg / (el / args.steps) / 1e9, 1),
                   "frac": round(alg / (el / args.steps) / 1e9 / HBM_PEAK_GBS, 4)},
        stack_mfma={"flops_per_step": int(flops),
                    "TFLOP_s": round(flops / (el / args.steps) / 1e12, 1),
                    "frac": round(flops / (el / args.steps) / 1e12 / MFMA_F16_PEAK_TFS, 4)},
        kernel_us_per_launch={k: round(v * 1e3, 3) for k, v in kern.items()},
        kernel_us_per_step={k: round(share[k] * 1e3, 2) for k in KERNELS},
        path_rows=[rmin, rwide],
        kernel_timing=f"{n_prof} untimed eager steps with event pairs around every kernel; "
                      f"the roofline kernel ({dom}) from its event pairs in the timed steps",
        graph={"tokens_s": round(T * args.steps / g_el, 1),
               "us_per_step": round(g_el * 1e6 / args.steps, 1),
               "what": f"the same {args.steps} steps captured in one HIP graph, replayed once "
                       "untimed and once timed (HIP events, no kernel event pairs)"},
        distinct_experts_per_layer=distinct,
        rows_top_expert_per_layer=[int(c.max()) for c in counts],
        wide_experts_per_layer=[int((c >= rwide).sum()) for c in counts])
    log(f"stack: {res}")
    return res, layers, x32


def cpu_baseline_stack(layers, x32, n_sample=8):
    """The oracle (fp64 NumPy, as it stands) on a bounded sample of the stack
    workload: layer 0 with its 256-token batch.  Router logits, top-k and
    softmax for all tokens and the shared expert on all tokens are timed in
    full; the routed-expert loop (dequantize a record, run its rows) is timed
    on the first n_sample of the layer's active experts, in the oracle's own
    order, and scaled to all of them; the layer time x 8 layers gives
    tokens/s through the stack.  Timed once with BLAS limited to one thread
    and once with all affinity cores.  Reading the records back from the GPU
    is excluded."""
    import oracle
    import synth
    m = layers[0]
    sh = synth.WORKLOADS[4].shape
    T = x32.shape[0]
    bank, stride, shared = m._keep[1], m._host["stride"], m._keep[2]
    x = oracle.rms_normalize(x32.cpu().numpy().astype(np.float64))
    ol = oracle.OracleLayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter,
                            m._host["router"], m._host["bias"], None, shared.cpu().numpy())
    ids0, _ = oracle.select_topk(ol.logits(x), sh.top_k)
    uniq = np.unique(ids0)
    recs = {int(e): bank[int(e) * stride:(int(e) + 1) * stride].cpu().numpy() for e in uniq[:n_sample]}
    info = host_info()
    try:
        from threadpoolctl import threadpool_limits
    except Exception:
        threadpool_limits = None
    out = {}
    for label, nth in (("1_thread", 1), ("all_cores", info["affinity_cpus"])):
        ctx = threadpool_limits(limits=nth, user_api="blas") if threadpool_limits else None
        try:
            t0 = time.perf_counter()
            lg = ol.logits(x)
            ids, _ = oracle.select_topk(lg, sh.top_k)
            oracle.softmax_selected(lg, ids)
            t_route = time.perf_counter() - t0
            t0 = time.perf_counter()
            for e in uniq[:n_sample]:
                rows, _ = np.nonzero(ids == e)
                oracle.expert_ffn(x[rows], *oracle.expert_matrices(recs[int(e)], sh.hidden, sh.inter))
            t_exp = (time.perf_counter() - t0) / min(n_sample, len(uniq)) * len(uniq)
            t0 = time.perf_counter()
            oracle.expert_ffn(x, *oracle.expert_matrices(ol.shared_record, sh.hidden, sh.shared_inter))
            t_sh = time.perf_counter() - t0
        finally:
            if ctx is not None:
                ctx.__exit__(None, None, None)
        t_layer = t_route + t_exp + t_sh
        out[label] = {"tokens_s": round(T / (len(layers) * t_layer), 5), "threads": nth,
                      "layer_s": round(t_layer, 2), "route_s": round(t_route, 3),
                      "experts_s": round(t_exp, 2), "shared_s": round(t_sh, 2)}
    log(f"cpu baseline: {out}")
    return dict(value=out["all_cores"]["tokens_s"], unit="tokens/s", cores=int(info["affinity_cpus"]),
                kind="oracle",
                sample=(f"layer 0 of the stack, 256 tokens: router, top-k, softmax and the shared "
                        f"expert timed in full; the routed-expert loop timed on {n_sample} of the "
                        f"{len(uniq)} active experts and scaled; x {len(layers)} layers"),
                one_thread=out["1_thread"], all_cores=out["all_cores"], host=info)


def run_large(args, dev, n_inputs=4):
    """The large decode layer (a 12.7 GB bank generated on the device) at 1, 8
    and 64 tokens per forward.  The timed graph rotates over n_inputs token
    batches, so successive forwards read different experts (the active set is
    larger than the 256 MB Infinity Cache)."""
    import torch
    import synth
    wl = synth.WORKLOADS[3]
    sh = wl.shape
    m = make_large_layer(dev, 3, 0, max(wl.batches))
    log("  large layer generated")
    out = {}
    for T in wl.batches:
        xs = [synth.bf16_tensor(synth.make_hidden(0, 3, T, sh.hidden, tag=200 + i), dev)
              for i in range(n_inputs)]
        y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        counts = []
        for x in xs:
            _, ids, _ = m.forward(x, return_selection=True)
            counts.append(np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts))
        for i in range(args.warmup):
            m.forward(xs[i % n_inputs], y=y)
        torch.cuda.synchronize()
        el, _ = timed_graph(lambda i: m.forward(xs[i % n_inputs], y=y), args.steps)
        kern, _ = profiled([m], lambda i: m.forward(xs[i % n_inputs], y=y), min(args.steps, 40))
        us = el * 1e6 / args.steps
        d = float(np.mean([(c > 0).sum() for c in counts]))
        alg = layer_bytes(sh, T, d)
        work = [kernel_work(c, sh, T, m.mfma_min_rows, m.wide_min_rows) for c in counts]
        up_b = float(np.mean([w["gemv_up"][0] for w in work]))
        up_f = float(np.mean([w["gemv_up"][1] for w in work]))
        out[f"T{T}"] = {"tokens_s": round(T / (us * 1e-6), 1), "us_per_step": round(us, 2),
                        "distinct_experts": d, "alg_bytes_per_step": int(alg),
                        "layer_GB_s": round(alg / (us * 1e-6) / 1e9, 1),
                        "layer_frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "gemv_up_roofline": roofline("gemv_up", up_b, up_f, kern["gemv_up"] * 1e3),
                        "kernel_us": {k: round(v * 1e3, 3) for k, v in kern.items()}}
        log(f"large T={T}: {out[f'T{T}']}")
    m.close()
    torch.cuda.empty_cache()
    return out


def run_cache(args, dev, decode_layers, n_slots=16, n_tokens=32):
    """Banks larger than HBM: the decode layers as a residual stack whose banks
    sit in pinned host memory, each layer with an n_slots-record HBM cache
    (the TurboFieldfare setting: 16 slots for a top-8 router over 128
    experts), run token by token.  Against the same stack on resident banks;
    with the next layer's router one residual ahead prefetching into the next
    layer's cache (each token's k predicted experts, or its top 6 as the
    WASTE page prefetches), and without."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    sh = synth.WORKLOADS[1].shape
    L = len(decode_layers)
    res, cac = [], []
    for mm in decode_layers:
        w = mm._w
        hb = torch.empty(w["bank"].numel(), dtype=torch.uint8, pin_memory=True)
        hb.copy_(w["bank"])
        for lst, bank in ((res, w["bank"]), (cac, hb)):
            m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, 1, rmsnorm=True)
            m.set_weights(w["router"], bank, w["stride"], w["shared"], w["bias"])
            m._hb = bank
            lst.append(m)
    xs = [synth.bf16_tensor(synth.make_hidden(0, 1, 1, sh.hidden, tag=900 + t), dev).float()
          for t in range(n_tokens)]
    r = torch.empty_like(xs[0])
    rec = synth.record_layout(sh.hidden, sh.inter)["end"]

    def tok(layers, t, la):
        r.copy_(xs[t % n_tokens])
        for l, m in enumerate(layers):
            m.forward(r, y=r, residual=r, lookahead=layers[l + 1] if la and l + 1 < L else None)

    out = {}
    for mode, layers, la, top in (("resident", res, True, None), ("cache_prefetch", cac, True, None),
                                  ("cache_prefetch_top6", cac, True, 6),
                                  ("cache_no_prefetch", cac, False, None)):
        if layers is cac:
            for l, m in enumerate(layers):
                m.set_cache(n_slots, prefetch=la and l > 0, prefetch_top=top if la and l > 0 else None)
        for t in range(4):
            tok(layers, t, la)
        torch.cuda.synchronize()
        if layers is cac:   # count the timed tokens only
            for l, m in enumerate(layers):
                m.set_cache(n_slots, prefetch=la and l > 0, prefetch_top=top if la and l > 0 else None)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for t in range(n_tokens):
            tok(layers, t, la)
        e1.record()
        torch.cuda.synchronize()
        el = e0.elapsed_time(e1) * 1e-3
        ent = {"tokens_s": round(n_tokens / el, 1), "us_per_token": round(el * 1e6 / n_tokens, 1)}
        if layers is cac:
            st = [m.cache_stats() for m in layers]
            sel = sum(x["selected"] for x in st)
            hits = sum(x["demand_hits"] for x in st)
            moved = sum(x["demand_bytes"] + x["prefetch_bytes"] for x in st)
            ent.update({"demand_hit_rate": round(hits / sel, 4),
                        "hit_rate_layer0": round(st[0]["demand_hits"] / st[0]["selected"], 4),
                        "hit_rate_layers_1_on": round(sum(x["demand_hits"] for x in st[1:]) /
                                                      sum(x["selected"] for x in st[1:]), 4),
                        "records_copied_per_token": round(moved / rec / n_tokens, 2),
                        "bytes_copied_per_token": int(moved / n_tokens),
                        "copy_GB_s": round(moved / el / 1e9, 2),
                        "prefetched": sum(x["prefetched"] for x in st),
                        "prefetch_used": sum(x["prefetch_used"] for x in st)})
        out[mode] = ent
        log(f"cache {mode}: {ent}")
    out["setup"] = (f"{L}-layer residual stack of the decode layer (hidden {sh.hidden}, {sh.n_experts} "
                    f"experts, top-{sh.top_k}), banks in pinned host memory, {n_slots} HBM slots per "
                    f"layer, one token per forward, {n_tokens} tokens timed (eager, HIP events)")
    for m in res + cac:
        m.close()
    return out


def run_rvq(args, dev, n_mats=16, R=4096, K=7168, copies=4, batches=(1, 2, 4, 8)):
    """The 3-bit residual-VQ product (the WASTE page's expert codec) on the
    large layer's gate/up shape: n_mats matrices of R x K (16 experts' gate
    and up rows at one decode token), rotating over `copies` banks so each
    call streams its indices from HBM.  Bytes: the indices, 3 bits per
    weight (the 12 KB of codebooks and the per-token tables are not
    counted)."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import rvq_gemv
    mb = synth.rvq_bytes(R, K)
    stride = -(-mb // 4096) * 4096
    g = torch.Generator(device=dev)
    g.manual_seed(5)
    banks = [torch.randint(0, 256, (n_mats * stride,), dtype=torch.uint8, device=dev, generator=g)
             for _ in range(copies)]
    cb = torch.from_numpy(synth.make_rvq_codebooks(0).view(np.int16)).to(dev)
    out = {}
    for T in batches:
        x = synth.bf16_tensor(synth.make_hidden(0, 3, T, K, tag=600), dev)
        y = torch.empty((n_mats, T, R), dtype=torch.float32, device=dev)
        ws = torch.empty(int(rvq_gemv.__globals__["L"].load().moe_rvq_workspace_bytes(T, K, R, n_mats)),
                         dtype=torch.uint8, device=dev)
        call = lambda i: rvq_gemv(x, banks[i % copies], R, cb, n_mats, stride, ws, y)  # noqa: E731
        for i in range(args.warmup):
            call(i)
        torch.cuda.synchronize()
        n = max(args.steps, 20)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            call(i)
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / n
        b = n_mats * mb
        out[f"T{T}"] = {"us_per_call": round(us, 2), "index_bytes": int(b),
                        "GB_s": round(b / (us * 1e-6) / 1e9, 1),
                        "frac_hbm_peak": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "weights_per_s_T": round(n_mats * R * K / (us * 1e-6) / 1e12, 3)}
        log(f"rvq T={T}: {out[f'T{T}']}")
    out["setup"] = (f"{n_mats} matrices of {R} x {K} at 3 bits per weight ({n_mats * mb / 1e6:.0f} MB), "
                    f"{copies} rotating copies, one call = lookups over tables built in LDS + the K-group reduction")
    del banks
    torch.cuda.empty_cache()
    return out


def run_decode(args, dev, batches=(1, 4, 16), copies=6, keep=False):
    """The decode layer (hidden 2816, 128 experts, top-8, intermediate 704,
    shared expert 2112) at 1, 4 and 16 tokens; forwards rotate over `copies`
    layer copies (2.6 GB of weights), so each streams its experts from HBM."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    wl = synth.WORKLOADS[1]
    sh = wl.shape
    layers = []
    for l in range(copies):
        li = synth.LayerInputs(0, 1, l, sh, wl.bias)
        w = synth.upload_layer(li, dev)
        mm = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max(batches))
        mm.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
        mm._w = w
        layers.append(mm)
    log("  decode layer copies uploaded")
    out = {}
    for T in batches:
        xs = [synth.bf16_tensor(synth.make_hidden(0, 1, T, sh.hidden, tag=100 + l + T), dev)
              for l in range(copies)]
        ys = [torch.empty((T, sh.hidden), dtype=torch.float32, device=dev) for _ in range(copies)]
        counts = []
        for l in range(copies):
            _, ids, _ = layers[l].forward(xs[l], return_selection=True)
            counts.append(np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts))
        step = lambda i: layers[i % copies].forward(xs[i % copies], y=ys[i % copies])  # noqa: E731
        for i in range(args.warmup):
            step(i)
        torch.cuda.synchronize()
        el, _ = timed_graph(step, args.steps)
        kern, _ = profiled(layers, step, min(args.steps, 120))
        us = el * 1e6 / args.steps
        d = float(np.mean([(c > 0).sum() for c in counts]))
        alg = layer_bytes(sh, T, d)
        m0 = layers[0]
        work = [kernel_work(c, sh, T, m0.mfma_min_rows, m0.wide_min_rows) for c in counts]
        up_b = float(np.mean([w["gemv_up"][0] for w in work]))
        up_f = float(np.mean([w["gemv_up"][1] for w in work]))
        dn_b = float(np.mean([w["gemv_down"][0] for w in work]))
        dn_f = float(np.mean([w["gemv_down"][1] for w in work]))
        out[f"T{T}"] = {"tokens_s": round(T / (us * 1e-6), 1), "us_per_step": round(us, 2),
                        "distinct_experts": d, "alg_bytes_per_step": int(alg),
                        "layer_GB_s": round(alg / (us * 1e-6) / 1e9, 1),
                        "layer_frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "gemv_up_roofline": roofline("gemv_up", up_b, up_f, kern["gemv_up"] * 1e3),
                        "gemv_down_roofline": roofline("gemv_down", dn_b, dn_f, kern["gemv_down"] * 1e3),
                        "kernel_us": {k: round(v * 1e3, 3) for k, v in kern.items()},
                        "path_rows": [m0.mfma_min_rows, m0.wide_min_rows]}
        if T == 16:
            rows = (m0.mfma_min_rows, m0.wide_min_rows)
            out["T16"]["gemv_up_roofline"]["traffic"] = measured_traffic("gemv_up_decode_T16_hbm_traffic.md", rows)
            out["T16"]["gemv_down_roofline"]["traffic"] = measured_traffic("gemv_down_decode_T16_hbm_traffic.md", rows)
        log(f"decode T={T}: {out[f'T{T}']}")
    if keep:
        return out, layers
    for mm in layers:
        mm.close()
    del layers
    torch.cuda.empty_cache()
    return out


def run_prefill(args, dev, copies=2):
    """The prefill workload: 16 chunks of 128 tokens (2048) per forward, router
    logit bias N(0, 0.5); the expert GEMMs run on the matrix cores."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    wl = synth.WORKLOADS[2]
    sh = wl.shape
    T = wl.batches[0]
    layers = []
    for l in range(copies):
        li = synth.LayerInputs(0, 2, l, sh, wl.bias)
        w = synth.upload_layer(li, dev)
        mm = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, T)
        mm.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
        mm._w = w
        layers.append(mm)
    xs = [synth.bf16_tensor(synth.make_hidden(0, 2, T, sh.hidden, tag=150 + l), dev) for l in range(copies)]
    ys = [torch.empty((T, sh.hidden), dtype=torch.float32, device=dev) for _ in range(copies)]
    counts = []
    for l in range(copies):
        _, ids, _ = layers[l].forward(xs[l], return_selection=True)
        counts.append(np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts))
    step = lambda i: layers[i % copies].forward(xs[i % copies], y=ys[i % copies])  # noqa: E731
    for i in range(2):
        step(i)
    torch.cuda.synchronize()
    n = max(4, args.steps // 2)
    el, _ = timed_graph(step, n)
    kern, _ = profiled(layers, step, min(n, 8))
    us = el * 1e6 / n
    # the same tokens as 16 sequential forwards of 128 (chunked prefill)
    C = 128

    def chunked(i):
        mm, x, y = layers[i % copies], xs[i % copies], ys[i % copies]
        for c in range(T // C):
            mm.forward(x[c * C:(c + 1) * C], y=y[c * C:(c + 1) * C])
    for i in range(2):
        chunked(i)
    torch.cuda.synchronize()
    el_c, _ = timed_graph(chunked, n)
    us_c = el_c * 1e6 / n
    m0 = layers[0]
    work = [kernel_work(c, sh, T, m0.mfma_min_rows, m0.wide_min_rows) for c in counts]
    wf = float(np.mean([w["mfma_up"][1] + w["mfma_down"][1] for w in work]))
    wb = float(np.mean([w["mfma_up"][0] + w["mfma_down"][0] for w in work]))
    wide_us = (kern["mfma_up"] + kern["mfma_down"]) * 1e3
    fl = layer_flops(sh, T)
    res = {"tokens_s": round(T / (us * 1e-6), 1), "us_per_step": round(us, 2),
           "layer_TFLOP_s": round(fl / (us * 1e-6) / 1e12, 1),
           "layer_frac_mfma_peak": round(fl / (us * 1e-6) / 1e12 / MFMA_F16_PEAK_TFS, 4),
           "wide_roofline": roofline("mfma_up+mfma_down", wb, wf, wide_us) if wide_us else None,
           "mfma_up_roofline": roofline("mfma_up", float(np.mean([w["mfma_up"][0] for w in work])),
                                        float(np.mean([w["mfma_up"][1] for w in work])),
                                        kern["mfma_up"] * 1e3) if kern["mfma_up"] else None,
           "chunked_16x128": {"tokens_s": round(T / (us_c * 1e-6), 1), "us_per_step": round(us_c, 2),
                              "what": "the same 2048 tokens as 16 sequential forwards of 128"},
           "rows_per_expert": {"min": int(counts[0].min()), "median": float(np.median(counts[0])),
                               "max": int(counts[0].max())},
           "distinct_experts": float(np.mean([(c > 0).sum() for c in counts])),
           "kernel_us": {k: round(v * 1e3, 3) for k, v in kern.items()}}
    log(f"prefill: {res}")
    for mm in layers:
        mm.close()
    del layers
    torch.cuda.empty_cache()
    return res


def measure_ceilings(dev):
    """What this GPU reaches on plain work, beside the spec peaks: a 1 GiB
    device-to-device copy (bytes read + written per second) and a dense fp16
    8192^3 matrix product through torch (hipBLASLt)."""
    import torch
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    a = torch.randn(8192, 8192, dtype=torch.float16, device=dev)
    b = torch.randn(8192, 8192, dtype=torch.float16, device=dev)

    def timed(fn, n):
        for _ in range(3):
            fn()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e-3 / n
    t_copy = timed(lambda: dst.copy_(src), 20)
    t_mm = timed(lambda: torch.mm(a, b), 20)
    out = {"copy_GB_s": round(2 * src.numel() / t_copy / 1e9, 1),
           "f16_gemm_TFLOP_s": round(2 * 8192 ** 3 / t_mm / 1e12, 1),
           "what": "1 GiB device-to-device copy (read + write bytes); torch.mm fp16 8192^3"}
    del src, dst, a, b
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", choices=("all", "stack", "large", "decode", "prefill", "cache", "rvq"),
                    default="all",
                    help="all: the stack headline plus every extra entry; stack: the headline "
                         "only; large / decode / prefill / cache / rvq: that workload only")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)
    import torch
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda", 0)
    if args.workload == "large":
        print(json.dumps({"large_decode": run_large(args, dev)}), flush=True)
        return
    if args.workload == "decode":
        print(json.dumps({"decode": run_decode(args, dev)}), flush=True)
        return
    if args.workload == "rvq":
        print(json.dumps({"rvq_gemv": run_rvq(args, dev)}), flush=True)
        return
    if args.workload == "cache":
        dec, layers = run_decode(args, dev, batches=(1,), keep=True)
        print(json.dumps({"expert_cache": run_cache(args, dev, layers)}), flush=True)
        return
    if args.workload == "prefill":
        print(json.dumps({"prefill": run_prefill(args, dev)}), flush=True)
        return
    import synth
    sh = synth.WORKLOADS[4].shape
    res, layers, x32 = run_stack(args, dev)
    out = {
        "metric": METRIC,
        "value": round(res["tokens_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["us_per_step"] * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"skewed 8-layer MoE stack: hidden {sh.hidden}, {sh.n_experts} "
                               f"experts, top-{sh.top_k}, intermediate {sh.inter}, shared expert "
                               f"{sh.shared_inter}, 4-bit g64 experts, 8-bit router, Zipf(1.1) "
                               f"router prior, 256 tokens, fp32 residual, lookahead on",
                   "layers": 8, "tokens_per_step": 256, "launch": "eager",
                   "timing": "HIP events around `steps` eager steps; the roofline kernel's "
                             "duration from the library's event pairs around it in the same steps"},
        "roofline": res["roofline"],
        "stack": {k: v for k, v in res.items() if k not in ("roofline",)},
    }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline_stack(layers, x32)
    for m in layers:
        m.close()
    del layers
    torch.cuda.empty_cache()
    if args.workload == "all":
        out["large_decode"] = run_large(args, dev)
        out["decode"], dec_layers = run_decode(args, dev, keep=True)
        out["expert_cache"] = run_cache(args, dev, dec_layers)
        for mm in dec_layers:
            mm.close()
        del dec_layers
        torch.cuda.empty_cache()
        out["prefill"] = run_prefill(args, dev)
        out["rvq_gemv"] = run_rvq(args, dev)
        c = measure_ceilings(dev)
        c["prefill_layer_frac_of_gemm"] = round(out["prefill"]["layer_TFLOP_s"] / c["f16_gemm_TFLOP_s"], 4)
        c["decode_T16_gemv_up_frac_of_copy"] = round(
            out["decode"]["T16"]["gemv_up_roofline"]["achieved"] / c["copy_GB_s"], 4)
        out["ceilings"] = c
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
