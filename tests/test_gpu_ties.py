"""Exact logit ties on the GPU: the selection rule orders experts by (logit
descending, index ascending), so among equal logits the lowest expert index
wins.  A zero router (every code 128 with bias -128 * scale, so every weight
is exactly 0) makes every logit equal to the router bias, exactly, on both
sides; the GPU's ids must then equal the oracle's element by element, in
order, and p the softmax of the selected biases.  Covers each top-k variant
(16-lane groups for up to 128 experts, the whole wave up to 512 (one
workgroup of 1024 threads for 5 to 16 tokens), 16 logits per lane beyond)
and the multi-workgroup bucketing pass."""
import numpy as np
import pytest

import oracle
import synth
from tests import parity as P
from tests import tilebytes as tb

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch_dev():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda", 0)


def zero_router(hidden, n_experts):
    """Tiled 8-bit router whose every weight is 0: codes 128, s = 2^-10,
    b = -128 * 2^-10 (all tiles identical)."""
    q = np.full((64, 64), 128)
    s = tb.f16bits(np.full((64, 1), 2.0 ** -10))
    b = tb.f16bits(np.full((64, 1), -128 * 2.0 ** -10))
    tile = np.frombuffer(bytes(tb.q8_tiles(q, s, b)), dtype=np.uint8)
    n_tiles = (-(-n_experts // 64)) * (hidden // 64)
    return np.tile(tile, n_tiles)


SHAPES = [
    dict(H=512, E=16, k=4, I=256, Is=0, T=4),          # one workgroup buckets itself
    dict(H=2816, E=128, k=8, I=704, Is=2112, T=16),    # the decode layer's shape
    dict(H=256, E=128, k=8, I=128, Is=128, T=300),     # several top-k workgroups + bucketing pass
    dict(H=256, E=512, k=16, I=128, Is=128, T=8),      # whole-wave groups
    dict(H=256, E=256, k=8, I=128, Is=128, T=16),      # a wave per token, 16 waves
    dict(H=128, E=1000, k=32, I=64, Is=0, T=5),        # 16 logits per lane
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"E{s['E']}k{s['k']}T{s['T']}")
@pytest.mark.parametrize("bias", ["none", "repeated"])
def test_exact_ties_lowest_index_wins(torch_dev, shape, bias):
    import torch
    from quantized_routed_expert_bit_amd import MoELayer
    H, E, k, I, Is, T = (shape[n] for n in ("H", "E", "k", "I", "Is", "T"))
    P.log(f"ties: {shape} bias={bias}")
    li = synth.LayerInputs(21, 89, 0, synth.LayerShape(H, E, k, I, Is), None)
    router = zero_router(H, E)
    beta = None
    if bias == "repeated":   # four distinct values: long runs of equal logits
        beta = (np.random.default_rng(E + k).integers(0, 4, E) * 0.25).astype(np.float32)
    w = P.upload_layer(li, torch_dev)
    m = MoELayer(H, E, k, I, Is, T)
    m.set_weights(torch.from_numpy(router).to(torch_dev), w["bank"], w["stride"], w["shared"],
                  None if beta is None else torch.from_numpy(beta).to(torch_dev))
    xb = synth.make_hidden(21, 89, T, H)
    y, ids, p = m.forward(P.bf16_tensor(xb, torch_dev), return_selection=True)
    ids, p = ids.cpu().numpy(), p.cpu().numpy()
    ol = oracle.OracleLayer(H, E, k, I, Is, router, beta, li.record, li.shared_record())
    x64 = oracle.bf16_bits_to_f64(xb)
    lg = ol.logits(x64)
    assert np.array_equal(lg, np.tile(np.zeros(E) if beta is None else beta.astype(np.float64),
                                      (T, 1)))
    ref_ids, _ = oracle.select_topk(lg, k)
    assert np.array_equal(ids, ref_ids), f"first mismatch at token {np.argwhere(ids != ref_ids)[0]}"
    if beta is None:
        assert np.array_equal(ids, np.tile(np.arange(k), (T, 1)))
        assert np.all(np.abs(p - 1.0 / k) <= 1e-7)
    else:
        assert np.all(np.abs(p - oracle.softmax_selected(lg, ref_ids)) <= 1e-6)
    ref = ol.forward(x64, pool=None)
    P.compare_y(y.cpu().numpy(), ref["y"], f"ties {bias}")
    m.close()


@pytest.mark.parametrize("H", [256, 4096])   # mfma_min_rows 4, and 3 from hidden 4096
def test_path_boundaries_exact_rows(torch_dev, H):
    """The zero router sends every token to experts 0..k-1, so each of them,
    and the shared expert, has exactly T rows: T runs across each path
    boundary at the layer's own thresholds (streaming below mfma_min_rows,
    32-row tiles below wide_min_rows, then 128-row tiles, one full tile and a
    second one of a single row), every token against the oracle."""
    import torch
    from quantized_routed_expert_bit_amd import MoELayer
    E, k, I, Is = 64, 4, 128, 128
    li = synth.LayerInputs(21, 87, 0, synth.LayerShape(H, E, k, I, Is), None)
    router = zero_router(H, E)
    w = P.upload_layer(li, torch_dev)
    m = MoELayer(H, E, k, I, Is, 129)
    m.set_weights(torch.from_numpy(router).to(torch_dev), w["bank"], w["stride"], w["shared"], None)
    R, W = m.mfma_min_rows, m.wide_min_rows
    ol = oracle.OracleLayer(H, E, k, I, Is, router, None, li.record, li.shared_record())
    for T in (R - 1, R, W - 1, W, W + 1, 128, 129):
        P.log(f"path boundaries: T={T} (R={R}, W={W})")
        xb = synth.make_hidden(21, 87, T, H)
        y, ids, p = m.forward(P.bf16_tensor(xb, torch_dev), return_selection=True)
        assert np.array_equal(ids.cpu().numpy(), np.tile(np.arange(k), (T, 1)))
        assert np.all(np.abs(p.cpu().numpy() - 1.0 / k) <= 1e-7)
        ref = ol.forward(oracle.bf16_bits_to_f64(xb), pool=None)
        P.compare_y(y.cpu().numpy(), ref["y"], f"boundary T={T}")
    m.close()
