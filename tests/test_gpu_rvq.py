"""The 3-bit residual-VQ product on the GPU (tables of partial inner
products, three lookups per 8-weight run) against the oracle, which
reconstructs the matrix and multiplies in fp64.  Shapes cover one tile, a
row count past a workgroup's rows with a short last K group, several
matrices at a stride, every kind of token pass (1, 2, 4, and 4 carrying 3),
fp32 input, the large layer's gate/up and the decode layer's down shapes,
and enough matrices for K groups larger than 4 tiles.

Tolerance: the GPU's tables and sums are fp32 (x converts exactly, codebook
entries are fp16, products and sums round once each); with K/8 runs of three
terms per output the expected error is a few 1e-7 of the output, so the bar
is rel-Frobenius 1e-5 and max-abs 1e-4 of the output RMS."""
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


CASES = [
    dict(R=64, K=64, T=1, n=1, f32=False),
    dict(R=1088, K=192, T=2, n=3, f32=False),     # ragged row block, a group of 3 tiles
    dict(R=320, K=640, T=5, n=2, f32=True),       # passes of 4 and 1 tokens, fp32 input
    dict(R=2816, K=704, T=4, n=1, f32=False),     # the decode layer's down shape
    dict(R=4096, K=7168, T=1, n=2, f32=False),    # the large layer's gate+up rows
    dict(R=192, K=256, T=3, n=1, f32=False),      # 3 tokens: one pass of 4 with a zero slot
    dict(R=128, K=320, T=6, n=2, f32=True),       # passes of 4 and 2
    dict(R=64, K=128, T=7, n=1, f32=False),       # passes of 4 and 4 (the second with 3)
    # 16 matrices: on 256 CUs the K groups take 7 tiles (one round of 240
    # workgroups), the last group 2 tiles
    dict(R=256, K=6400, T=2, n=16, f32=False),
]


@pytest.mark.parametrize("c", CASES, ids=lambda c: f"R{c['R']}K{c['K']}T{c['T']}n{c['n']}")
def test_rvq_gemv_matches_oracle(torch_dev, c):
    import torch
    from quantized_routed_expert_bit_amd import rvq_gemv
    R, K, T, n = c["R"], c["K"], c["T"], c["n"]
    mb = synth.rvq_bytes(R, K)
    stride = -(-mb // 4096) * 4096
    bank = np.zeros(n * stride, dtype=np.uint8)
    for m in range(n):
        bank[m * stride: m * stride + mb] = synth.make_rvq_matrix(9, R, K, tag=m)
    cb = synth.make_rvq_codebooks(9)
    rng = np.random.default_rng(R + K)
    if c["f32"]:
        x32 = (rng.standard_normal((T, K)) * 1.5).astype(np.float32)
        x = torch.from_numpy(x32).to(torch_dev)
        x64 = x32.astype(np.float64)
    else:
        xb = synth.bf16_bits_from_f32(rng.standard_normal((T, K)).astype(np.float32))
        x = P.bf16_tensor(xb, torch_dev)
        x64 = oracle.bf16_bits_to_f64(xb)
    y = rvq_gemv(x, torch.from_numpy(bank).to(torch_dev), R,
                 torch.from_numpy(cb.view(np.int16)).to(torch_dev), n_mats=n, mat_stride=stride)
    y = y.cpu().numpy().astype(np.float64)
    for m in range(n):
        ref = oracle.rvq_gemv(bank, m * stride, R, K, cb, x64)
        err = y[m] - ref
        rel = np.linalg.norm(err) / np.linalg.norm(ref)
        mx = np.abs(err).max() / np.sqrt(np.mean(ref ** 2))
        P.log(f"rvq {c} m={m}: rel {rel:.2e} max/rms {mx:.2e}")
        assert rel <= 1e-5 and mx <= 1e-4


def test_rvq_gemv_errors(torch_dev):
    import torch
    from quantized_routed_expert_bit_amd import MoEError, rvq_gemv
    x = torch.zeros((1, 96), dtype=torch.float32, device=torch_dev)
    mats = torch.zeros(4096, dtype=torch.uint8, device=torch_dev)
    cb = torch.zeros((3, 256, 8), dtype=torch.float16, device=torch_dev)
    with pytest.raises(MoEError):
        rvq_gemv(x, mats, 64, cb)                    # K = 96 is not a multiple of 64
    x = torch.zeros((1, 64), dtype=torch.float32, device=torch_dev)
    with pytest.raises(MoEError) as ei:
        rvq_gemv(x, mats, 64, cb, workspace=torch.empty(512, dtype=torch.uint8, device=torch_dev)[:128])
    assert ei.value.code == -3
    # y must be 4-byte aligned
    y = torch.empty(258, dtype=torch.uint8, device=torch_dev)[2:]
    with pytest.raises(MoEError) as ei:
        rvq_gemv(x, mats, 64, cb, y=y)
    assert ei.value.code == -1
