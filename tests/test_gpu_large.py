"""Full-size workloads on the GPU, every token checked against the oracle:

* the large-expert decode layer (hidden 7168, 512 experts, top-16,
  intermediate 2048, shared 2048; a 12.7 GB bank) at 1, 8 and 64 tokens;
* the 8-layer stack at that shape (101.5 GB of banks), 256 tokens, Zipf(1.1)
  router prior, fp32 residual stream updated by the library, each layer's
  input RMS-normalized (without it, random-weight SwiGLU layers square the
  activation scale each layer and the stack overflows), with the next layer's
  router run one residual ahead: on and off must give bitwise equal outputs
  and selections.  Two whole layers (all 256 tokens) are checked on the
  residual the GPU's own stack fed them, and 16 tokens on every one of the
  eight layers the same way; the stack's end-to-end drift from the oracle's
  own fp64 stack is reported.

Banks are generated on the device by synth.gpu_bank; the oracle reads the
records it needs back from the bank (the kernels never write it) and
evaluates experts on a thread pool."""
import threading

import numpy as np
import pytest

import oracle
import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


class _Records:
    """Record bytes read back from a device bank, one copy per request
    (thread-safe: the oracle's pool asks from several threads)."""

    def __init__(self, bank, stride):
        self.bank, self.stride, self.lock = bank, stride, threading.Lock()

    def __call__(self, e):
        with self.lock:
            return self.bank[e * self.stride:(e + 1) * self.stride].cpu().numpy()


def _large_layer(dev, cfg, layer, max_tokens, rmsnorm=False):
    import torch
    from quantized_routed_expert_bit_amd import MoELayer
    wl = synth.WORKLOADS[cfg]
    sh = wl.shape
    bank, stride = synth.gpu_bank(0, cfg, layer, sh.hidden, sh.inter, sh.n_experts, dev)
    shared, sstride = synth.gpu_bank(0, cfg, layer, sh.hidden, sh.shared_inter, 1, dev, shared=True)
    router = synth.make_router(0, cfg, layer, sh.hidden, sh.n_experts)
    bias = synth.make_router_bias(0, cfg, layer, sh.n_experts, wl.bias)
    m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max_tokens,
                 rmsnorm=rmsnorm)
    m.set_weights(torch.from_numpy(router).to(dev), bank, stride, shared,
                  None if bias is None else torch.from_numpy(bias).to(dev))
    ol = oracle.OracleLayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, router,
                            bias, _Records(bank, stride), shared.cpu().numpy())
    return m, ol


@pytest.fixture(scope="module")
def large_layer(torch_dev):
    P.log("large decode layer: generating the 12.7 GB bank on the device")
    m, ol = _large_layer(torch_dev, 3, 0, 64)
    yield m, ol
    m.close()


@pytest.mark.timeout(600)
@pytest.mark.parametrize("T", [1, 8, 20, 24, 64])
def test_large_decode_layer_every_token(torch_dev, large_layer, T):
    """Every token of each batch; from 8 tokens the routed experts with 3 to
    23 rows run as 32-row matrix-core tiles over a 112-group K chain (split by
    K at 8 tokens, by columns at 20, 24 and 64), the ones with 1 or 2 rows on
    the streaming path.  At 20 tokens the shared expert's 20 rows take those
    tiles too; from 24 it runs as a 128-row tile on the wide kernels, beside
    the streaming launches, as does every routed expert with 24 or more rows."""
    m, ol = large_layer
    H = synth.WORKLOADS[3].shape.hidden
    P.log(f"large decode T={T}: all tokens")
    xb = synth.make_hidden(0, 3, T, H)
    y, ids, p = m.forward(P.bf16_tensor(xb, torch_dev), return_selection=True)
    ids_np = ids.cpu().numpy()
    cnt = np.bincount(ids_np.reshape(-1), minlength=512)
    P.log(f"  {int((cnt > 0).sum())} experts, rows per expert max {cnt.max()}, "
          f"{int(((cnt >= m.mfma_min_rows) & (cnt < m.wide_min_rows)).sum())} on 32-row tiles, "
          f"{int((cnt >= m.wide_min_rows).sum())} on 128-row tiles")
    with P.oracle_pool() as pool:
        P.check_forward(ol, oracle.bf16_bits_to_f64(xb), y.cpu().numpy(), ids_np,
                        p.cpu().numpy(), f"large T={T}", pool=pool)


@pytest.fixture(scope="module")
def stack(torch_dev):
    """The eight layers and the GPU stack run without lookahead: the residual
    r_l each layer received, its ids, and r_8."""
    import torch
    wl = synth.WORKLOADS[4]
    sh = wl.shape
    T = wl.batches[0]
    layers = []
    for l in range(wl.layers):
        P.log(f"stack: generating layer {l}")
        layers.append(_large_layer(torch_dev, 4, l, T, rmsnorm=True))
    xb = synth.make_hidden(0, 4, T, sh.hidden)
    r0 = P.bf16_tensor(xb, torch_dev).float()
    yield dict(layers=layers, xb=xb, r0=r0, T=T, H=sh.hidden)
    for m, _ in layers:
        m.close()


def _run_stack(st, lookahead):
    import torch
    layers = st["layers"]
    r = st["r0"].clone()
    ids_all, rs = [], []
    for l, (m, _) in enumerate(layers):
        nxt = layers[l + 1][0] if lookahead and l + 1 < len(layers) else None
        out = torch.empty_like(r)
        rs.append(r)
        _, ids, _ = m.forward(r, return_selection=True, lookahead=nxt, y=out, residual=r)
        ids_all.append(ids)
        r = out
    torch.cuda.synchronize()
    return r, ids_all, rs


@pytest.mark.timeout(600)
def test_stack_8_layers_lookahead_invariance(torch_dev, stack):
    import torch
    r_off, ids_off, _ = _run_stack(stack, False)
    r_rep, _, _ = _run_stack(stack, False)
    assert torch.equal(r_rep, r_off), "two runs without lookahead differ"
    r_on, ids_on, _ = _run_stack(stack, True)
    assert torch.equal(r_on, r_off), "lookahead changed the output"
    for a, b in zip(ids_on, ids_off):
        assert torch.equal(a, b), "lookahead changed the selected experts"
    P.log("stack: lookahead on/off bitwise equal")
    r = stack["r0"].clone()
    for m, _ in stack["layers"]:
        m.forward(r, y=r, residual=r)
    assert torch.equal(r, r_off), "in-place residual update differs"


@pytest.mark.timeout(600)
@pytest.mark.parametrize("layer", [0, 5])
def test_stack_full_layer_on_gpu_residual(torch_dev, stack, layer):
    """All 256 tokens of one layer, fed the residual r_l of the GPU's own stack
    run; the oracle takes the same r_l (fp32 -> fp64, exact) through its RMS
    norm."""
    _, _, rs = _run_stack(stack, False)
    m, ol = stack["layers"][layer]
    r = rs[layer]
    y, ids, p = m.forward(r, return_selection=True)
    ids_np = ids.cpu().numpy()
    cnt = np.bincount(ids_np.reshape(-1), minlength=512)
    P.log(f"stack layer {layer}: {int((cnt > 0).sum())} experts, top expert {cnt.max()} rows, "
          f"{int((cnt >= m.wide_min_rows).sum())} on 128-row tiles")
    xin = oracle.rms_normalize(r.cpu().numpy().astype(np.float64))
    lg = m.router_logits(r).cpu().numpy()
    dl = np.abs(lg - ol.logits(xin))
    P.log(f"  router logits: max |err| {dl.max():.3e}, mean {dl.mean():.3e}, "
          f"|x| max {np.abs(xin).max():.2f}, |r| max {float(r.abs().max()):.2f}")
    assert dl.max() < 1e-5
    with P.oracle_pool() as pool:
        P.check_forward(ol, xin, y.cpu().numpy(), ids_np, p.cpu().numpy(),
                        f"stack layer {layer}, 256 tokens", pool=pool)


@pytest.fixture(scope="module")
def stack16(stack):
    """The stack's 256-token run without lookahead and 16 sampled tokens
    (every 16th of the batch)."""
    r_off, ids_off, rs = _run_stack(stack, False)
    return dict(r_off=r_off, ids_off=ids_off, rs=rs, sample=list(range(0, stack["T"], 16)))


@pytest.mark.parametrize("l", range(8))
def test_stack_16_tokens_layer(torch_dev, stack, stack16, l):
    """16 tokens through all 8 layers, one layer per test: the layer's
    output, ids and weights on the input the GPU's stack fed it (the
    256-token forward of that layer, the sampled rows), against the oracle's
    layer on the same input, by the same rules as every other forward (ids
    where the gap exceeds 1e-3, y to the output tolerances)."""
    m, ol = stack["layers"][l]
    sample = stack16["sample"]
    y, ids, p = m.forward(stack16["rs"][l], return_selection=True)
    xin = oracle.rms_normalize(stack16["rs"][l].cpu().numpy()[sample].astype(np.float64))
    with P.oracle_pool() as pool:
        P.check_forward(ol, xin, y.cpu().numpy()[sample], ids.cpu().numpy()[sample],
                        p.cpu().numpy()[sample], f"stack layer {l}, 16 tokens", pool=pool)


@pytest.mark.parametrize("sel", ["own", "gpu"])
def test_stack_16_tokens_end_to_end(torch_dev, stack, stack16, sel):
    """The stack end to end against the oracle's own fp64 stack, on the
    oracle's own selections or forced onto the GPU's.  Reported, with the
    drift per layer; the per-layer bar is held by test_stack_16_tokens_layer.
    The stack amplifies any per-layer difference (the residual grows to
    |r| ~ 900 by layer 5; a relative residual drift of a few 1e-4 moves logits
    by a few 1e-2 and grows layer by layer), so only a loose sanity bound is
    asserted here: r_8 within 5e-2 relative (measured a few 1e-3)."""
    sample = stack16["sample"]
    layers = [ol for _, ol in stack["layers"]]
    gpu_ids = [stack16["ids_off"][l].cpu().numpy()[sample] for l in range(len(layers))]
    x0 = oracle.bf16_bits_to_f64(stack["xb"])[sample]
    with P.oracle_pool() as pool:
        ref = oracle.oracle_stack(layers, x0, norm=True, pool=pool,
                                  force_ids=gpu_ids if sel == "gpu" else None)
    n_diff = 0
    for l, lr in enumerate(ref["layers"]):
        rl = stack16["rs"][l].cpu().numpy()[sample]
        rd = np.linalg.norm(rl - lr["input"]) / np.linalg.norm(lr["input"])
        diff = [(sample[i], round(float(lr["gap"][i]), 4)) for i in range(len(sample))
                if lr["gap"][i] > P.GAP and set(gpu_ids[l][i].tolist()) != set(lr["ids"][i].tolist())]
        n_diff += len(diff)
        P.log(f"  layer {l}: residual drift from the oracle's stack ({sel} selections) {rd:.2e}; "
              f"selections that differ there (token, gap): {diff}")
    err = stack16["r_off"].cpu().numpy()[sample] - ref["out"]
    rel = np.linalg.norm(err) / np.linalg.norm(ref["out"])
    P.log(f"stack end to end, oracle on {sel} selections: r_8 rel {rel:.3e}, "
          f"max/rms {np.abs(err).max() / np.sqrt(np.mean(ref['out'] ** 2)):.3e}; "
          f"{n_diff} token-layers select differently")
    assert np.isfinite(err).all() and rel < 5e-2
