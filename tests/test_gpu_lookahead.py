"""Lookahead at decode sizes, on every single-workgroup top-k variant: layer l
also runs layer l+1's router on its own input and hands the prediction to
l+1, which only orders its expert work by it (the real router still decides,
as in [WASTE] "Önceden okuma ve router tahmini").  Outputs, selections and
weights of both layers must be bitwise equal with the lookahead on and off,
and layer l+1 must match the oracle on the residual it received.  (The
256-token stack checks the same on the multi-workgroup top-k.)"""
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


SHAPES = [
    dict(H=256, E=128, k=8, I=128, Is=128, T=16),   # 16-lane groups, 4 tokens per wave
    dict(H=256, E=512, k=16, I=128, Is=128, T=1),   # a wave per token, partials in one round
    dict(H=256, E=512, k=16, I=128, Is=128, T=8),   # 1024 threads, a wave per token
    dict(H=128, E=1000, k=32, I=64, Is=0, T=3),     # 16 logits per lane
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"E{s['E']}k{s['k']}T{s['T']}")
def test_lookahead_on_off_bitwise(torch_dev, shape):
    import torch
    from quantized_routed_expert_bit_amd import MoELayer
    H, E, k, I, Is, T = (shape[n] for n in ("H", "E", "k", "I", "Is", "T"))
    P.log(f"lookahead: {shape}")
    sh = synth.LayerShape(H, E, k, I, Is)
    lis = [synth.LayerInputs(31, 88, l, sh, "normal0.5") for l in (0, 1)]
    layers = []
    for li in lis:
        w = P.upload_layer(li, torch_dev)
        m = MoELayer(H, E, k, I, Is, T)
        m.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
        m._w = w
        layers.append(m)
    m0, m1 = layers
    x = P.bf16_tensor(synth.make_hidden(31, 88, T, H), torch_dev).float()
    runs = []
    for la in (False, True, False, True):
        r1 = torch.empty_like(x)
        _, i0, p0 = m0.forward(x, return_selection=True, y=r1, residual=x,
                               lookahead=m1 if la else None)
        y1, i1, p1 = m1.forward(r1, return_selection=True)
        torch.cuda.synchronize()
        runs.append((r1, i0, p0, y1, i1, p1))
    for run in runs[1:]:
        for a, b in zip(runs[0], run):
            assert torch.equal(a, b), "lookahead on/off or a repeat changed a result"
    r1, _, _, y1, i1, p1 = runs[1]
    P.check_forward(P.oracle_layer(lis[1]), r1.cpu().numpy().astype(np.float64),
                    y1.cpu().numpy(), i1.cpu().numpy(), p1.cpu().numpy(), f"lookahead {shape}")
    for m in layers:
        m.close()
