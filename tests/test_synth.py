"""The seeded input generators: determinism, headers, value distributions."""
import numpy as np

import oracle
import synth


def test_same_seed_same_bytes_and_independent_records():
    a = synth.make_record(0, 1, 0, 5, 256, 128)
    b = synth.make_record(0, 1, 0, 5, 256, 128)
    c = synth.make_record(0, 1, 0, 6, 256, 128)
    assert np.array_equal(a, b)
    assert not np.array_equal(a[256:], c[256:])
    li = synth.layer_inputs(synth.WORKLOADS[0])
    bank = li.bank()
    st = li.stride
    assert np.array_equal(bank[3 * st:4 * st], li.record(3))


def test_record_header_fields():
    rec = synth.make_record(0, 1, 0, 7, 2816, 704)
    h = oracle.read_record_header(rec)
    assert h["magic"] == 0x58455251 and h["version"] == 1 and h["expert_id"] == 7
    assert (h["hidden"], h["inter"], h["group"], h["bits"], h["tile_rows"]) == (2816, 704, 64, 4, 64)
    sec = 11 * 44 * 2304
    assert (h["gate_off"], h["up_off"], h["down_off"], h["end_off"]) == (256, 256 + sec, 256 + 2 * sec, 256 + 3 * sec)
    assert len(rec) % 4096 == 0 and len(rec) >= h["end_off"]
    assert len(rec) == 3346432          # 3 * 2816 * 704 * 4.5 bits + header, 4 KiB padded
    sh = oracle.read_record_header(synth.make_record(0, 1, 0, 0, 2816, 2112, shared=True))
    assert sh["expert_id"] == -1 and sh["inter"] == 2112


def test_value_distributions():
    rec = synth.make_record(0, 1, 0, 0, 2816, 704)
    lay = synth.record_layout(2816, 704)
    t = rec[lay["gate"]:lay["end"]].reshape(-1, 2304)
    codes = t[:, :2048].reshape(-1)
    nib = np.concatenate([codes & 15, codes >> 4])
    hist = np.bincount(nib, minlength=16) / nib.size
    assert np.all(np.abs(hist - 1 / 16) < 0.002)
    sb = np.ascontiguousarray(t[:, 2048:]).view(np.float16).reshape(-1, 2)
    s, b = sb[:, 0].astype(np.float64), sb[:, 1].astype(np.float64)
    assert np.all(b == -8 * s)                                  # exact
    sub = np.mean(s < 2.0 ** -14)
    assert 0.015 < sub < 0.025                                  # ~2 % fp16 subnormal scales
    assert abs(np.median(s) - 0.6745 * 0.02 / 8) < 2e-4
    r = synth.make_router(0, 1, 0, 2816, 128).reshape(-1, 4352)
    rsb = np.ascontiguousarray(r[:, 4096:]).view(np.float16).reshape(-1, 2).astype(np.float64)
    assert np.all(rsb[:, 1] == -128 * rsb[:, 0])
    assert 0.27 < np.mean(rsb[:, 0] < 2.0 ** -14) < 0.33        # ~30 % subnormal router scales


def test_hidden_states_are_bf16_normal():
    x = synth.make_hidden(0, 1, 64, 2816)
    v = oracle.bf16_bits_to_f64(x)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    # bf16: the low 16 bits of the fp32 pattern are zero
    assert np.array_equal(v.astype(np.float32).view(np.uint32) & 0xFFFF, np.zeros(v.shape, np.uint32))


def test_router_bias_kinds():
    assert synth.make_router_bias(0, 2, 0, 128, None) is None
    nb = synth.make_router_bias(0, 2, 0, 128, "normal0.5")
    assert nb.dtype == np.float32 and 0.35 < nb.std() < 0.65
    zb = synth.make_router_bias(0, 4, 3, 512, "zipf1.1").astype(np.float64)
    ranks = np.exp(-zb / 1.1)
    assert np.allclose(np.sort(ranks), np.arange(1, 513), rtol=1e-5)
