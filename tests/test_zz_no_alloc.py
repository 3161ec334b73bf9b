"""moe_forward_noalloc (the allocation-free entry point) against moe_forward,
through the C ABI: bitwise equal y, ids and p on two calls in a row (the
second with a smaller batch), after another context's call has left its state
in the shared scratch, and on a batch large enough for the 128-row
matrix-core kernels; its errors (a forward too large for the scratch, the
bound-workspace calls on a context without a workspace)."""
import numpy as np
import pytest

import synth
from tests import parity as P

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def _pair(dev, wl_index, max_tokens):
    """Two contexts on the same weights: one with a bound workspace, one
    without (it can only run the allocation-free forward)."""
    from quantized_routed_expert_bit_amd import MoELayer
    wl = synth.WORKLOADS[wl_index]
    sh = wl.shape
    w = synth.upload_layer(synth.layer_inputs(wl), dev)
    ref = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max_tokens)
    ref.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
    na = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, max_tokens)
    na.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"], no_workspace=True)
    return ref, na, w


def _same(dev, ref, na, wl_index, T, tag):
    import torch
    xb = synth.make_hidden(0, wl_index, T, ref.hidden, tag=tag)
    x = P.bf16_tensor(xb, dev)
    y0, i0, p0 = ref.forward(x, return_selection=True)
    y1, i1, p1 = na.forward_noalloc(x, return_selection=True)
    torch.cuda.synchronize()
    assert torch.equal(i0, i1), f"T={T}: ids differ"
    assert torch.equal(p0, p1), f"T={T}: p differs"
    assert torch.equal(y0, y1), f"T={T}: y differs (max {float((y0 - y1).abs().max()):.3e})"
    P.log(f"  noalloc T={T}: bitwise equal to moe_forward")


def test_noalloc_matches_forward(torch_dev):
    import torch
    from quantized_routed_expert_bit_amd import MoEError
    ref, na, _ = _pair(torch_dev, 1, 64)
    _same(torch_dev, ref, na, 1, 16, 31)         # decode batch
    _same(torch_dev, ref, na, 1, 4, 32)          # then a smaller one
    # another context's call leaves its own state in the shared scratch
    ref0, na0, _ = _pair(torch_dev, 0, 4)
    _same(torch_dev, ref0, na0, 0, 4, 33)
    _same(torch_dev, ref, na, 1, 64, 34)         # 128-row matrix-core kernels (side stream)
    _same(torch_dev, ref, na, 1, 1, 35)
    # residual fused into the combine, y aliasing the residual
    x = P.bf16_tensor(synth.make_hidden(0, 1, 8, ref.hidden, tag=36), torch_dev)
    r = torch.randn(8, ref.hidden, device=torch_dev)
    a = r.clone()
    b = r.clone()
    ref.forward(x, y=a, residual=a)
    na.forward_noalloc(x, y=b, residual=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # the bound-workspace calls refuse on a context without a workspace
    with pytest.raises(MoEError) as ei:
        na.forward(x)
    assert ei.value.code == -5
    with pytest.raises(MoEError) as ei:
        na.router_logits(x)
    assert ei.value.code == -5
    with pytest.raises(MoEError) as ei:
        ref.forward(x, lookahead=na)
    assert ei.value.code == -1
    for m in (ref, na, ref0, na0):
        m.close()


def test_noalloc_refuses_a_batch_beyond_the_scratch(torch_dev):
    """2048 tokens of the decode layer need ~230 MB of workspace, more than the
    64 MiB scratch: MOE_ENOMEM, and nothing is launched."""
    import ctypes
    import torch
    from quantized_routed_expert_bit_amd import MoEError, make_config, load
    lib = load()
    sh = synth.WORKLOADS[1].shape
    c = make_config(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, 2048)
    assert lib.moe_workspace_bytes(ctypes.byref(c)) > 64 << 20
    ref, na, _ = _pair(torch_dev, 2, 2048)
    x = P.bf16_tensor(synth.make_hidden(0, 2, 2048, sh.hidden), torch_dev)
    with pytest.raises(MoEError) as ei:
        na.forward_noalloc(x)
    assert ei.value.code == -3
    # a batch that fits still runs on that context
    _same(torch_dev, ref, na, 2, 128, 37)
    ref.close()
    na.close()
