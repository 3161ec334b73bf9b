"""Record integrity on the GPU: the library's CRC-32 kernel against zlib's
crc32 on the host (the reference implementation of the checksum), and
MOE_F_VERIFY at bind time: every record of a bank with checksums passes, a
single flipped payload bit anywhere in one record (or in the shared record)
is refused naming that record, and a record without a checksum is refused."""
import time
import zlib

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


@pytest.mark.parametrize("n", [0, 1, 15, 16, 17, 255, 4096, 65537, (1 << 20) + 3, 50_000_007])
def test_crc32_matches_zlib(torch_dev, n):
    import torch
    from quantized_routed_expert_bit_amd import crc32
    g = torch.Generator(device=torch_dev)
    g.manual_seed(n)
    buf = torch.randint(0, 256, (max(n, 1),), dtype=torch.uint8, device=torch_dev, generator=g)[:n]
    want = zlib.crc32(buf.cpu().numpy().tobytes())
    got = crc32(buf)
    P.log(f"crc32 n={n}: gpu {got:08x} zlib {want:08x}")
    assert got == want


def _layer(dev, li, verify, bank=None, shared=None):
    from quantized_routed_expert_bit_amd import MoELayer
    sh = li.shape
    w = synth.upload_layer(li, dev)
    m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, sh.shared_inter, 16, verify=verify)
    return m, w


def test_verify_accepts_a_checked_bank_and_refuses_flipped_bits(torch_dev):
    import torch
    from quantized_routed_expert_bit_amd import MoEError
    wl = synth.WORKLOADS[1]
    li = synth.layer_inputs(wl)
    m, w = _layer(torch_dev, li, verify=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    m.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
    dt = time.perf_counter() - t0
    nbytes = wl.shape.n_experts * w["stride"] + w["shared"].numel()
    P.log(f"verify: {wl.shape.n_experts} records + shared ({nbytes / 1e6:.0f} MB) in {dt * 1e3:.1f} ms "
          f"(header copy, checks and CRCs: {nbytes / dt / 1e9:.1f} GB/s)")
    # the verified context computes the same layer as an unverified one
    ref, _ = _layer(torch_dev, li, verify=False)
    ref.set_weights(w["router"], w["bank"], w["stride"], w["shared"], w["bias"])
    x = P.bf16_tensor(synth.make_hidden(0, 1, 16, wl.shape.hidden), torch_dev)
    assert torch.equal(m.forward(x), ref.forward(x))
    lay = synth.record_layout(wl.shape.hidden, wl.shape.inter)
    rng = np.random.default_rng(3)
    for e, sec in ((77, "down"), (0, "gate"), (127, "up")):
        off = e * w["stride"] + lay[sec] + int(rng.integers(0, lay["end"] - lay["down"]))
        bank = w["bank"].clone()
        bank[off] ^= 1 << int(rng.integers(0, 8))
        with pytest.raises(MoEError) as ei:
            m.set_weights(w["router"], bank, w["stride"], w["shared"], w["bias"])
        assert ei.value.code == -4 and f"record {e}:" in str(ei.value), str(ei.value)
        with pytest.raises(MoEError) as ei:
            m.forward(x)
        assert ei.value.code == -5                       # a refused bind keeps no weights
        del bank
    shared = w["shared"].clone()
    shared[lay["up"] + 12345] ^= 0x80
    with pytest.raises(MoEError) as ei:
        m.set_weights(w["router"], w["bank"], w["stride"], shared, w["bias"])
    assert ei.value.code == -4 and "shared record" in str(ei.value)
    # the unverified context binds the flipped bank (the header check cannot see it)
    bank = w["bank"].clone()
    bank[77 * w["stride"] + lay["down"] + 5] ^= 1
    ref.set_weights(w["router"], bank, w["stride"], w["shared"], w["bias"])
    m.close()
    ref.close()


def test_verify_refuses_records_without_checksum(torch_dev):
    from quantized_routed_expert_bit_amd import MoEError, MoELayer
    sh = synth.LayerShape(256, 8, 2, 128, 0)
    recs = [synth.make_record(5, 88, 0, e, 256, 128, checksum=(e != 3)) for e in range(8)]
    import torch
    bank = torch.from_numpy(np.concatenate(recs)).to(torch_dev)
    router = torch.from_numpy(synth.make_router(5, 88, 0, 256, 8)).to(torch_dev)
    m = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, 0, 4, verify=True)
    with pytest.raises(MoEError) as ei:
        m.set_weights(router, bank, len(recs[0]))
    assert ei.value.code == -4 and "record 3 carries no payload checksum" in str(ei.value)
    plain = MoELayer(sh.hidden, sh.n_experts, sh.top_k, sh.inter, 0, 4)
    plain.set_weights(router, bank, len(recs[0]))          # without the flag it binds
    m.close()
    plain.close()
