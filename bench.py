"""Benchmark of the routed-expert MoE layer on one MI355X.

Default workload: the decode layer (hidden 2816, 128 experts, top-8,
intermediate 704, shared expert 2112) at 16 tokens per forward.  A step is one
moe_forward: router + top-k + bucketing, gate/up, down, combine.  Steps rotate
over several copies of the layer (distinct weights, like consecutive layers of
a model) so the active weights come from HBM, not from the 256 MB last-level
cache.  The timed region is one HIP graph holding K forwards; HIP events that
the library records around each kernel inside that graph give per-kernel
durations for the roofline line.

Prints ONE JSON line (rank 0, one GPU).
"""
from __future__ import annotations

import argparse
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


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def record_bytes(h, i):
    """Algorithmic bytes of one expert record: 3*H*I weights at 4.5 bits."""
    return 3 * h * i * 9 // 16


def measured_traffic():
    """HBM bytes per launch of the streaming gate/up kernel at this workload,
    from the committed rocprofv3 FETCH_SIZE + WRITE_SIZE passes (calibrated
    against a plain copy); None once the kernel sources differ from the ones
    the counters were taken on."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "gemv_up_decode_T16_hbm_traffic.md")
    try:
        fields = dict(line.split(": ", 1) for line in open(path).read().splitlines()
                      if line.startswith(("traffic_bytes_per_launch: ", "source_sha256: ")))
        h = hashlib.sha256()
        for f in ("moe_kernels.hip", "moe_internal.h"):
            with open(os.path.join(ROOT, "quantized_routed_expert_bit_amd", "csrc", f), "rb") as fh:
                h.update(fh.read())
        if h.hexdigest() != fields["source_sha256"].strip():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def build_layers(wl_index, n_copies, max_tokens, dev):
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    from tests.parity import upload_layer
    wl = synth.WORKLOADS[wl_index]
    sh = wl.shape
    layers = []
    for l in range(n_copies):
        li = synth.LayerInputs(0, wl.index, l, sh, wl.bias)
        w = upload_layer(li, dev)
        m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max_tokens)
        m.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
        m._w, m._li = w, li
        layers.append(m)
        log(f"  layer copy {l} uploaded")
    return wl, layers


def run_case(layers, sh, T, steps, warmup, tag=0):
    """Warm up eagerly, capture `steps` forwards in one graph, replay it once
    (the timed region).  Returns timings and routing stats."""
    import torch
    import synth
    from tests.parity import bf16_tensor
    dev = torch.device("cuda", 0)
    n = len(layers)
    xs = [bf16_tensor(synth.make_hidden(0, layers[l]._li.cfg, T, sh.hidden, tag=100 + l + tag), dev)
          for l in range(n)]
    ys = [torch.empty((T, sh.hidden), dtype=torch.float32, device=dev) for _ in range(n)]
    # routing per copy (deterministic): distinct experts and rows
    distinct, streamed = [], []
    rwide = layers[0].wide_min_rows
    for l in range(n):
        _, ids, _ = layers[l].forward(xs[l], return_selection=True)
        cnt = np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts)
        distinct.append(int((cnt > 0).sum()))
        # experts in the streaming launches: streamed, or in 32-row matrix-core tiles
        streamed.append(int(((cnt > 0) & (cnt < rwide)).sum()))
    for i in range(warmup):
        layers[i % n].forward(xs[i % n], y=ys[i % n])
    torch.cuda.synchronize()
    # timed region: one graph replay of `steps` forwards
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(steps):
            layers[i % n].forward(xs[i % n], y=ys[i % n])
    g.replay()                       # untimed replay (graph upload)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    g.replay()
    torch.cuda.synchronize()
    el = time.perf_counter() - t0
    del g
    # kernel timing pass: the same forwards eagerly, with the library's event
    # pairs around each kernel; a spin kernel holds the GPU while the host
    # queues them, so no kernel waits on the host.
    kp = min(steps, 120)
    per_copy = [(kp + n - 1 - l) // n for l in range(n)]
    for l in range(n):
        layers[l].profile_start(per_copy[l])
    t_first = torch.cuda.Event(enable_timing=True)
    t_last = torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(int(2.4e9 * 0.05))          # ~50 ms of GPU spin
    t_first.record()
    for i in range(kp):
        layers[i % n].forward(xs[i % n], y=ys[i % n])
    t_last.record()
    torch.cuda.synchronize()
    eager_ms = t_first.elapsed_time(t_last) / kp
    prof = [layers[l].profile_read() for l in range(n)]
    kern = {}
    for name in prof[0][0]:
        tot = sum(p[0][name] * p[1] for p in prof)
        cnt = sum(p[1] for p in prof if p[0][name] > 0)
        kern[name] = tot / cnt if cnt else 0.0
    d_avg = float(np.average(distinct, weights=per_copy))
    s_avg = float(np.average(streamed, weights=per_copy))
    return dict(elapsed=el, ms_per_step=el * 1e3 / steps, tok_s=T * steps / el, kern_ms=kern,
                distinct=d_avg, streamed=s_avg, per_copy=per_copy, distinct_per_copy=distinct,
                eager_ms_per_step=eager_ms)


def path_flops(ids, sh, T, rmin, rwide):
    """FLOPs of the expert FFNs on each path, from the actual routing."""
    cnt = np.bincount(ids.reshape(-1), minlength=sh.n_experts)
    per_row = 2 * 3 * sh.hidden * sh.inter
    out = {"stream": 0.0, "narrow": 0.0, "wide": 0.0}
    for c in cnt[cnt > 0]:
        out["stream" if c < rmin else ("narrow" if c < rwide else "wide")] += c * per_row
    if sh.has_shared:
        out["stream" if T < rmin else ("narrow" if T < rwide else "wide")] += \
            T * 2 * 3 * sh.hidden * sh.shared_inter
    return out, cnt


def run_prefill(args, dev):
    """The prefill workload: 16 chunks of 128 tokens (2048) per forward, router
    logit bias N(0, 0.5); bound by the matrix cores."""
    import torch
    import synth
    from tests.parity import bf16_tensor
    wl, layers = build_layers(2, 2, 2048, dev)
    sh = wl.shape
    T = wl.batches[0]
    r = run_case(layers, sh, T, max(4, args.steps // 20), 2, tag=50)
    _, ids, _ = layers[0].forward(bf16_tensor(synth.make_hidden(0, 2, T, sh.hidden, tag=150), dev),
                                  return_selection=True)
    fl, cnt = path_flops(ids.cpu().numpy(), sh, T, layers[0].mfma_min_rows, layers[0].wide_min_rows)
    k = r["kern_ms"]
    wide_ms = k["mfma_up"] + k["mfma_down"]
    total_flops = T * 2 * (sh.top_k * 3 * sh.hidden * sh.inter + 3 * sh.hidden * sh.shared_inter
                           + sh.n_experts * sh.hidden)
    res = {"tokens_s": round(r["tok_s"], 1), "us_per_step": round(r["ms_per_step"] * 1e3, 2),
           "layer_TFLOP_s": round(total_flops / (r["ms_per_step"] * 1e-3) / 1e12, 1),
           "layer_frac_mfma_peak": round(total_flops / (r["ms_per_step"] * 1e-3) / 1e12 / MFMA_F16_PEAK_TFS, 4),
           "wide_mfma_TFLOP_s": round(fl["wide"] / (wide_ms * 1e-3) / 1e12, 1) if wide_ms else None,
           "wide_frac_mfma_peak": round(fl["wide"] / (wide_ms * 1e-3) / 1e12 / MFMA_F16_PEAK_TFS, 4) if wide_ms else None,
           "path_gflop": {kk: round(v / 1e9, 2) for kk, v in fl.items()},
           "rows_per_expert": {"min": int(cnt.min()), "median": float(np.median(cnt)), "max": int(cnt.max())},
           "kernel_us": {kk: round(v * 1e3, 3) for kk, v in k.items()},
           "distinct_experts": r["distinct"]}
    log(f"prefill: {res}")
    for m in layers:
        m.close()
    return res


def cpu_baseline(layer0, sh, T):
    """The oracle (fp64 NumPy) on one forward of the same workload."""
    import oracle
    import synth
    from tests.parity import oracle_layer
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count()
    ol = oracle_layer(layer0._li, cache=True)
    xb = synth.make_hidden(0, layer0._li.cfg, T, sh.hidden, tag=100)
    x64 = oracle.bf16_bits_to_f64(xb)
    ids = ol.forward(x64[:1])["ids"]          # warm: regenerate the records the batch uses
    for e in np.unique(oracle.select_topk(ol.logits(x64), sh.top_k)[0]):
        ol.get_record(int(e))
    t0 = time.perf_counter()
    ol.forward(x64)
    el = time.perf_counter() - t0
    return dict(value=round(T / el, 3), unit="tokens/s", cores=int(threads), kind="oracle",
                sample=f"one oracle forward of the {T}-token batch on layer copy 0 (fp64 dequant "
                       f"of every active record + router, top-k, FFNs, combine; record "
                       f"generation excluded): {el:.2f} s")


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


def run_large(args, dev, n_inputs=4):
    """The large decode layer (hidden 7168, 512 experts, top-16, intermediate
    2048, shared expert 2048; a 12.7 GB bank generated on the device) at 1, 8
    and 64 tokens per forward.  The timed graph rotates over n_inputs token
    batches, so successive forwards read different experts (the active set is
    larger than the 256 MB Infinity Cache)."""
    import torch
    import synth
    from quantized_routed_expert_bit_amd import MoELayer
    from tests.parity import bf16_tensor
    wl = synth.WORKLOADS[3]
    sh = wl.shape
    bank, stride = synth.gpu_bank(0, 3, 0, sh.hidden, sh.inter, sh.n_experts, dev)
    shared, _ = synth.gpu_bank(0, 3, 0, sh.hidden, sh.shared_inter, 1, dev, shared=True)
    router = synth.make_router(0, 3, 0, sh.hidden, sh.n_experts)
    bias = synth.make_router_bias(0, 3, 0, sh.n_experts, wl.bias)
    m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max(wl.batches))
    m.set_weights(torch.from_numpy(router).to(dev), bank, stride, shared,
                  None if bias is None else torch.from_numpy(bias).to(dev))
    log("  large layer uploaded")
    out = {}
    for T in wl.batches:
        xs = [bf16_tensor(synth.make_hidden(0, 3, T, sh.hidden, tag=200 + i), dev) for i in range(n_inputs)]
        y = torch.empty((T, sh.hidden), dtype=torch.float32, device=dev)
        distinct = []
        for x in xs:
            _, ids, _ = m.forward(x, return_selection=True)
            distinct.append(int((np.bincount(ids.cpu().numpy().reshape(-1), minlength=sh.n_experts) > 0).sum()))
        for i in range(args.warmup):
            m.forward(xs[i % n_inputs], y=y)
        torch.cuda.synchronize()
        steps = args.steps
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for i in range(steps):
                m.forward(xs[i % n_inputs], y=y)
        g.replay()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        g.replay()
        torch.cuda.synchronize()
        el = time.perf_counter() - t0
        del g
        kp = min(steps, 40)
        m.profile_start(kp)
        torch.cuda._sleep(int(2.4e9 * 0.05))
        for i in range(kp):
            m.forward(xs[i % n_inputs], y=y)
        torch.cuda.synchronize()
        kern, _ = m.profile_read()
        d = float(np.mean(distinct))
        alg = d * record_bytes(sh.hidden, sh.inter) + record_bytes(sh.hidden, sh.shared_inter) + \
            sh.n_experts * sh.hidden * 17 / 16 + T * sh.hidden * 6 + T * sh.top_k * 8
        us = el * 1e6 / steps
        out[f"T{T}"] = {"tokens_s": round(T * steps / el, 1), "us_per_step": round(us, 2),
                        "distinct_experts": d, "alg_bytes_per_step": int(alg),
                        "layer_GB_s": round(alg / (us * 1e-6) / 1e9, 1),
                        "layer_frac_hbm_peak": round(alg / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                        "kernel_us": {k: round(v * 1e3, 3) for k, v in kern.items()}}
        log(f"large T={T}: {out[f'T{T}']}")
    m.close()
    del bank, shared
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--copies", type=int, default=6, help="layer copies the steps rotate over")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the T=1 and T=4 lines")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 2048-token prefill line")
    ap.add_argument("--workload", choices=("all", "decode", "prefill", "large"), default="all",
                    help="decode: only the 16-token decode line; prefill: only the prefill line; "
                         "large: only the hidden-7168, 512-expert decode layer at 1, 8 and 64 tokens")
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
    if args.workload == "prefill":
        print(json.dumps({"prefill": run_prefill(args, dev)}), flush=True)
        return
    if args.workload == "large":
        print(json.dumps({"large_decode": run_large(args, dev)}), flush=True)
        return
    if args.workload == "decode":
        args.no_extra = args.no_prefill = args.no_cpu_baseline = True
    T = args.batch
    wl, layers = build_layers(1, args.copies, max(T, 16), dev)
    sh = wl.shape
    res = run_case(layers, sh, T, args.steps, args.warmup)
    log(f"T={T}: {res['ms_per_step']*1e3:.1f} us/step, kernels {res['kern_ms']}")

    # dominant kernel: the gate/up launch of the streaming path, which also
    # carries the 32-row matrix-core tiles.  Algorithmic bytes per launch =
    # (routed experts with fewer than wide_min_rows rows, + the shared expert
    # when the batch is below that) * 2*H*I*4.5/8.
    shared_streams = sh.has_shared and T < layers[0].wide_min_rows
    up_bytes = res["streamed"] * 2 * sh.hidden * sh.inter * 9 / 16 + \
        (2 * sh.hidden * sh.shared_inter * 9 / 16 if shared_streams else 0)
    up_ms = res["kern_ms"]["gemv_up"]
    achieved = up_bytes / (up_ms * 1e-3) / 1e9
    layer_bytes = res["distinct"] * record_bytes(sh.hidden, sh.inter) + \
        (record_bytes(sh.hidden, sh.shared_inter) if sh.has_shared else 0) + \
        sh.n_experts * sh.hidden * 17 / 16 + T * sh.hidden * 6 + T * sh.top_k * 8
    out = {
        "metric": METRIC,
        "value": round(res["tok_s"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(res["ms_per_step"], 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": f"decode MoE layer: hidden {sh.hidden}, {sh.n_experts} experts, "
                               f"top-{sh.top_k}, intermediate {sh.inter}, shared expert "
                               f"{sh.shared_inter}, {T} tokens per forward, 4-bit g64 experts, "
                               f"8-bit router, {args.copies} rotating layer copies",
                   "tokens_per_step": T, "layer_copies": args.copies, "launch": "hip_graph"},
        "roofline": {"bound": "hbm", "kernel": "gemv_up", "achieved": round(achieved, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic() if T == 16 else None,
                     "bytes_per_launch": int(up_bytes),
                     "avg_launch_us": round(up_ms * 1e3, 3)},
        "layer_hbm": {"alg_bytes_per_step": int(layer_bytes),
                      "GB_s": round(layer_bytes / (res["ms_per_step"] * 1e-3) / 1e9, 1),
                      "frac": round(layer_bytes / (res["ms_per_step"] * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "kernel_us": {k: round(v * 1e3, 3) for k, v in res["kern_ms"].items()},
        "eager_us_per_step": round(res["eager_ms_per_step"] * 1e3, 2),
        "distinct_experts": res["distinct"],
        "streamed_experts": res["streamed"],
    }
    if not args.no_extra:
        extra = {}
        for Tx in (1, 4):
            r = run_case(layers, sh, Tx, args.steps, args.warmup, tag=Tx)
            ub = r["streamed"] * 2 * sh.hidden * sh.inter * 9 / 16 + \
                (2 * sh.hidden * sh.shared_inter * 9 / 16
                 if sh.has_shared and Tx < layers[0].wide_min_rows else 0)
            extra[f"T{Tx}"] = {"tokens_s": round(r["tok_s"], 1), "us_per_step": round(r["ms_per_step"] * 1e3, 2),
                               "gemv_up_GB_s": round(ub / (r["kern_ms"]["gemv_up"] * 1e-3) / 1e9, 1),
                               "kernel_us": {k: round(v * 1e3, 3) for k, v in r["kern_ms"].items()},
                               "distinct_experts": r["distinct"]}
            log(f"T={Tx}: {extra[f'T{Tx}']}")
        out["extra"] = extra
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(layers[0], sh, T)
    if not args.no_extra:
        c = measure_ceilings(dev)
        c["gemv_up_frac_of_copy"] = round(achieved / c["copy_GB_s"], 4)
        out["ceilings"] = c
    if not args.no_prefill:
        for m in layers:
            m.close()
        del layers
        torch.cuda.empty_cache()
        out["prefill"] = run_prefill(args, dev)
        if "ceilings" in out:
            out["ceilings"]["prefill_layer_frac_of_gemm"] = round(
                out["prefill"]["layer_TFLOP_s"] / out["ceilings"]["f16_gemm_TFLOP_s"], 4)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
