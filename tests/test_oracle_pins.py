"""Pins of the CPU oracle against things other than itself: hand-built bytes
with closed-form values, a scalar brute force written from the format text,
an independent library (torch, CPU, float64) on the special cases where the
layer reduces to a dense formula, exhaustive subset search for top-k, and
invariants.  CPU only."""
import itertools
import json
import math
import os
import struct

import numpy as np
import pytest

import oracle
import synth
from tests import tilebytes as tb

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- dequant ----

def test_q4_tile_closed_form():
    """q = (r + 3c) % 16, s = 0.5, b = -4  =>  W = 0.5 q - 4 (exact)."""
    r, c = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    q = (r + 3 * c) % 16
    s = tb.f16bits(np.full((64, 1), 0.5))
    b = tb.f16bits(np.full((64, 1), -4.0))
    buf = np.frombuffer(bytes(tb.q4_tiles(q, s, b)), dtype=np.uint8)
    w = oracle.dequant_tiled(buf, 0, 64, 64, 4)
    assert np.array_equal(w, 0.5 * q - 4.0)


def test_q4_nibble_order_golden():
    """Golden fixture: one byte 0x1F at the start of a tile."""
    with open(os.path.join(GOLDEN, "q4_nibble_order.json")) as f:
        fx = json.load(f)
    buf = np.zeros(2304, dtype=np.uint8)
    for off, val in fx["bytes"]:
        buf[off] = val
    w = oracle.dequant_tiled(buf, 0, 64, 64, 4)
    for (rr, cc), val in fx["expect_nonzero"]:
        assert w[rr, cc] == val
    assert np.count_nonzero(w) == len(fx["expect_nonzero"])


def test_subnormal_scale_is_kept():
    """s = smallest fp16 subnormal (2^-24), b = -3 * 2^-24: W = (q - 3) 2^-24."""
    q = np.tile(np.arange(64) % 16, (64, 1))
    s = np.full((64, 1), 0x0001, dtype=np.uint16)
    b = np.full((64, 1), 0x8003, dtype=np.uint16)         # -3 * 2^-24
    buf = np.frombuffer(bytes(tb.q4_tiles(q, s, b)), dtype=np.uint8)
    w = oracle.dequant_tiled(buf, 0, 64, 64, 4)
    assert np.array_equal(w, (q - 3.0) * 2.0 ** -24)
    assert np.all(w[:, 4] != 0)


def test_q8_tile_closed_form():
    r, c = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    q = (3 * r + 5 * c) % 256
    s = tb.f16bits(np.full((64, 1), 2.0 ** -7))
    b = tb.f16bits(np.full((64, 1), -1.0))
    buf = np.frombuffer(bytes(tb.q8_tiles(q, s, b)), dtype=np.uint8)
    w = oracle.dequant_tiled(buf, 0, 64, 64, 8)
    assert np.array_equal(w, q * 2.0 ** -7 - 1.0)


@pytest.mark.parametrize("bits", [4, 8])
def test_tile_order_row_block_major(bits):
    """128 x 192 matrix: tile (rb, g) gets scale rb*3+g+1 and code 1, so
    W[r, c] = (r//64)*3 + c//64 + 1 identifies which tile each element came from."""
    R, C = 128, 192
    q = np.ones((R, C), dtype=np.int64)
    rb, g = np.meshgrid(np.arange(R // 64), np.arange(C // 64), indexing="ij")
    sv = (rb * 3 + g + 1).astype(np.float64)
    s = tb.f16bits(np.repeat(sv, 64, axis=0))
    b = tb.f16bits(np.zeros((R, C // 64)))
    fn = tb.q4_tiles if bits == 4 else tb.q8_tiles
    buf = np.frombuffer(bytes(fn(q, s, b)), dtype=np.uint8)
    w = oracle.dequant_tiled(buf, 0, R, C, bits)
    rr, cc = np.meshgrid(np.arange(R), np.arange(C), indexing="ij")
    assert np.array_equal(w, (rr // 64) * 3 + cc // 64 + 1.0)


# ------------------------------------------------------- scalar brute force --

def _scalar_w(buf, off, cols, bits, r, c):
    tile = 2304 if bits == 4 else 4352
    rb, rr = divmod(r, 64)
    g, cc = divmod(c, 64)
    base = off + (rb * (cols // 64) + g) * tile
    if bits == 4:
        h, w = divmod(cc, 32)
        j, nib = divmod(w, 2)
        byte = int(buf[base + h * 1024 + rr * 16 + j])
        q = byte >> 4 if nib else byte & 15
    else:
        c4, j = divmod(cc, 16)
        q = int(buf[base + c4 * 1024 + rr * 16 + j])
    s, bb = struct.unpack_from("<ee", bytes(buf[base + tile - 256 + 4 * rr: base + tile - 256 + 4 * rr + 4]))
    return s * q + bb


def _scalar_ffn(rec, xv, H, I):
    gate_off, up_off, down_off = struct.unpack_from("<3Q", bytes(rec[32:56]))
    hv = []
    for i in range(I):
        g = sum(_scalar_w(rec, gate_off, H, 4, i, k) * xv[k] for k in range(H))
        u = sum(_scalar_w(rec, up_off, H, 4, i, k) * xv[k] for k in range(H))
        hv.append(g / (1.0 + math.exp(-g)) * u)
    return [sum(_scalar_w(rec, down_off, I, 4, r, i) * hv[i] for i in range(I)) for r in range(H)]


def _scalar_layer(x, router, beta, recs, shared, H, E, k, I, Is):
    ys, sels, ps = [], [], []
    for xv in x:
        lg = [sum(_scalar_w(router, 0, H, 8, e, h) * xv[h] for h in range(H)) + beta[e] for e in range(E)]
        remaining, sel = list(range(E)), []
        for _ in range(k):
            best = remaining[0]
            for e in remaining[1:]:
                if lg[e] > lg[best]:
                    best = e
            sel.append(best)
            remaining.remove(best)
        m = max(lg[e] for e in sel)
        z = [math.exp(lg[e] - m) for e in sel]
        p = [v / sum(z) for v in z]
        y = [0.0] * H
        for j, e in enumerate(sel):
            out = _scalar_ffn(recs[e], xv, H, I)
            y = [a + p[j] * o for a, o in zip(y, out)]
        if shared is not None:
            out = _scalar_ffn(shared, xv, H, Is)
            y = [a + o for a, o in zip(y, out)]
        ys.append(y)
        sels.append(sel)
        ps.append(p)
    return np.array(ys), np.array(sels), np.array(ps)


def test_scalar_brute_force_tiny_layer():
    H, E, k, I, Is, T = 64, 4, 2, 64, 64, 3
    router = synth.make_router(7, 99, 0, H, E)
    recs = [synth.make_record(7, 99, 0, e, H, I) for e in range(E)]
    shared = synth.make_record(7, 99, 0, 0, H, Is, shared=True)
    rng = np.random.default_rng(3)
    beta = rng.standard_normal(E) * 0.01
    x = oracle.bf16_bits_to_f64(synth.make_hidden(7, 99, T, H))
    ys, sels, ps = _scalar_layer(x.tolist(), router, beta, recs, shared, H, E, k, I, Is)
    layer = oracle.OracleLayer(H, E, k, I, Is, router, beta, lambda e: recs[e], shared)
    res = layer.forward(x)
    assert np.array_equal(res["ids"], sels)
    assert np.allclose(res["p"], ps, rtol=1e-13, atol=0)
    assert np.allclose(res["y"], ys, rtol=1e-11, atol=1e-13 * np.abs(ys).max())


# ---------------------------------------------------------------- router ----

def test_zero_router_gives_bias_and_lowest_ids():
    """All codes 128 with b = -128 s: W = 0, logits = beta exactly; with beta = 0
    every logit ties, so the ids are 0..k-1 and p = 1/k."""
    H, E, k = 128, 16, 4
    q = np.full((64, H), 128)
    s = tb.f16bits(np.full((64, H // 64), 2.0 ** -10))
    b = tb.f16bits(np.full((64, H // 64), -128 * 2.0 ** -10))
    router = np.frombuffer(bytes(tb.q8_tiles(q, s, b)), dtype=np.uint8)
    x = np.random.default_rng(0).standard_normal((5, H))
    wr = oracle.router_matrix(router, H, E)
    assert np.array_equal(wr, np.zeros((E, H)))
    beta = np.linspace(-1, 1, E)
    assert np.array_equal(oracle.router_logits(x, wr, beta), np.tile(beta, (5, 1)))
    lg = oracle.router_logits(x, wr, None)
    ids, gap = oracle.select_topk(lg, k)
    assert np.array_equal(ids, np.tile(np.arange(k), (5, 1)))
    assert np.all(gap == 0)
    assert np.allclose(oracle.softmax_selected(lg, ids), 1.0 / k, rtol=0, atol=1e-16)


def test_router_basis_vector_reads_a_column():
    """x = e_i gives logits[:, e] = W[e, i], with W from a hand-built tile."""
    H, E = 64, 64
    r, c = np.meshgrid(np.arange(64), np.arange(64), indexing="ij")
    q = (7 * r + c) % 256
    s = tb.f16bits(np.full((64, 1), 2.0 ** -8))
    b = tb.f16bits(np.full((64, 1), 0.25))
    router = np.frombuffer(bytes(tb.q8_tiles(q, s, b)), dtype=np.uint8)
    wr = oracle.router_matrix(router, H, E)
    for i in (0, 17, 63):
        x = np.zeros((1, H))
        x[0, i] = 1.0
        assert np.array_equal(oracle.router_logits(x, wr)[0], q[:, i] * 2.0 ** -8 + 0.25)


def test_topk_matches_exhaustive_subset_search():
    """For E <= 8: the selected set has the largest logit sum, and among ties the
    lexicographically smallest index set (lowest index wins)."""
    rng = np.random.default_rng(1)
    for trial in range(300):
        E = int(rng.integers(1, 9))
        k = int(rng.integers(1, E + 1))
        lg = rng.integers(0, 4, size=(1, E)).astype(np.float64)   # many ties
        ids, gap = oracle.select_topk(lg, k)
        best = max(itertools.combinations(range(E), k),
                   key=lambda s: (sum(lg[0, list(s)]), [-i for i in s]))
        assert sorted(ids[0].tolist()) == list(best)
        # ordered by (logit desc, index asc)
        seq = [(-lg[0, i], i) for i in ids[0]]
        assert seq == sorted(seq)
        if k < E:
            rest = sorted(set(range(E)) - set(best), key=lambda i: (-lg[0, i], i))
            assert gap[0] == lg[0, ids[0, -1]] - lg[0, rest[0]]
        else:
            assert gap[0] == np.inf


def test_softmax_selected_properties():
    rng = np.random.default_rng(2)
    lg = rng.standard_normal((6, 10))
    ids1, _ = oracle.select_topk(lg, 1)
    assert np.array_equal(oracle.softmax_selected(lg, ids1), np.ones((6, 1)))
    ids, _ = oracle.select_topk(lg, 4)
    p = oracle.softmax_selected(lg, ids)
    assert np.allclose(p.sum(1), 1.0, rtol=0, atol=1e-15)
    assert np.all(np.diff(p, axis=1) <= 0)          # ordered by logit => p non-increasing
    # shift invariance: same ids, same p
    ids2, _ = oracle.select_topk(lg + 3.25, 4)
    assert np.array_equal(ids, ids2)
    assert np.allclose(oracle.softmax_selected(lg + 3.25, ids2), p, rtol=1e-14, atol=0)
    # k = E is a dense softmax (scipy as the independent routine)
    from scipy.special import softmax
    idsE, _ = oracle.select_topk(lg, 10)
    dense = softmax(lg, axis=1)
    assert np.allclose(oracle.softmax_selected(lg, idsE), np.take_along_axis(dense, idsE, 1),
                       rtol=1e-14, atol=0)


# ----------------------------------------------------- layer special cases --

def _tiny_layer(H=128, E=6, k=2, I=64, Is=128, seed=5, beta=None):
    router = synth.make_router(seed, 98, 0, H, E)
    recs = [synth.make_record(seed, 98, 0, e, H, I) for e in range(E)]
    shared = synth.make_record(seed, 98, 0, 0, H, Is, shared=True) if Is else None
    layer = oracle.OracleLayer(H, E, k, I, Is, router, beta, lambda e: recs[e], shared)
    return layer, recs, shared


def _torch_ffn(x, wg, wu, wd):
    import torch
    import torch.nn.functional as F
    xt = torch.from_numpy(x)
    h = F.silu(F.linear(xt, torch.from_numpy(wg))) * F.linear(xt, torch.from_numpy(wu))
    return F.linear(h, torch.from_numpy(wd)).numpy()


def test_top_k_equal_E_is_dense_softmax_moe():
    """k = E: y = sum_e softmax(l)_e FFN_e(x) + FFN_s(x), by torch (float64, CPU)."""
    import torch
    H, E, I, Is = 128, 6, 64, 128
    layer, recs, shared = _tiny_layer(H, E, E, I, Is)
    x = np.random.default_rng(4).standard_normal((5, H))
    res = layer.forward(x)
    pt = torch.softmax(torch.from_numpy(x) @ torch.from_numpy(layer.wr).T, dim=-1).numpy()
    y = _torch_ffn(x, *oracle.expert_matrices(shared, H, Is))
    for e in range(E):
        y = y + pt[:, e:e + 1] * _torch_ffn(x, *oracle.expert_matrices(recs[e], H, I))
    assert np.allclose(res["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_one_hot_router_is_a_single_ffn():
    """beta one-hot at +100 with k = 1: p = 1 and y = FFN_e*(x) (+ shared)."""
    H, E, I, Is = 128, 6, 64, 128
    for e_star in (0, 3, 5):
        beta = np.zeros(E)
        beta[e_star] = 100.0
        layer, recs, shared = _tiny_layer(H, E, 1, I, Is, beta=beta)
        x = np.random.default_rng(e_star).standard_normal((4, H))
        res = layer.forward(x)
        assert np.all(res["ids"] == e_star)
        assert np.all(res["p"] == 1.0)
        y = _torch_ffn(x, *oracle.expert_matrices(recs[e_star], H, I)) + \
            _torch_ffn(x, *oracle.expert_matrices(shared, H, Is))
        assert np.allclose(res["y"], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_zero_input_gives_zero_output():
    layer, _, _ = _tiny_layer(beta=np.arange(6) * 0.1)
    res = layer.forward(np.zeros((3, 128)))
    assert np.array_equal(res["y"], np.zeros((3, 128)))
    assert np.array_equal(res["ids"], np.tile([5, 4], (3, 1)))


def test_constant_weights_closed_form():
    """Every weight of gate, up, down = a, c, d (codes 0, bias = value):
    g = a sum(x), u = c sum(x), h_i = SiLU(g) u for all i, y_r = d * I * h."""
    H, I = 128, 64
    a, c, d = 2.0 ** -6, -2.0 ** -5, 2.0 ** -7
    def const(rows, cols, v):
        return bytes(tb.q4_tiles(np.zeros((rows, cols), dtype=np.int64),
                                 tb.f16bits(np.ones((rows, cols // 64))),
                                 tb.f16bits(np.full((rows, cols // 64), v))))
    rec = tb.record(0, H, I, const(I, H, a), const(I, H, c), const(H, I, d))
    x = np.random.default_rng(9).standard_normal((3, H))
    sx = x.sum(1)
    g, u = a * sx, c * sx
    h = g / (1 + np.exp(-g)) * u
    expect = np.repeat((d * I * h)[:, None], H, axis=1)
    got = oracle.expert_ffn(x, *oracle.expert_matrices(rec, H, I))
    assert np.allclose(got, expect, rtol=1e-13, atol=0)


def test_token_permutation_equivariance():
    layer, _, _ = _tiny_layer(beta=np.zeros(6))
    x = np.random.default_rng(11).standard_normal((7, 128))
    perm = np.random.default_rng(12).permutation(7)
    a = layer.forward(x)
    b = layer.forward(x[perm])
    assert np.array_equal(a["ids"][perm], b["ids"])
    assert np.allclose(a["y"][perm], b["y"], rtol=1e-14, atol=1e-15)


def test_stack_lookahead_does_not_change_result():
    layers = []
    for l in range(3):
        router = synth.make_router(1, 97, l, 128, 8)
        recs = [synth.make_record(1, 97, l, e, 128, 64) for e in range(8)]
        layers.append(oracle.OracleLayer(128, 8, 2, 64, 0, router, None,
                                         (lambda rs: (lambda e: rs[e]))(recs)))
    x = np.random.default_rng(5).standard_normal((4, 128))
    a = oracle.oracle_stack(layers, x)
    b = oracle.oracle_stack(layers, x, lookahead_k=2)
    assert np.array_equal(a["out"], b["out"])
    assert "lookahead_ids" in b["layers"][0] and "lookahead_ids" not in a["layers"][0]
    # residual identity: out = x + y_0 + y_1 + y_2
    assert np.allclose(a["out"], x + sum(r["y"] for r in a["layers"]), rtol=1e-15, atol=1e-15)


def test_rms_normalize_closed_forms():
    """c * 1 -> sign(c) / sqrt(1 + eps/c^2); rows scale-invariant; unit RMS."""
    x = np.full((1, 64), 3.0)
    assert np.allclose(oracle.rms_normalize(x), 1.0 / np.sqrt(1 + 1e-6 / 9), rtol=1e-15, atol=0)
    r = np.random.default_rng(3).standard_normal((4, 256)) * np.array([[0.1], [1], [10], [1e3]])
    n = oracle.rms_normalize(r)
    assert np.allclose(np.sqrt(np.mean(n * n, axis=1)), 1.0, rtol=1e-4, atol=0)
    assert np.allclose(oracle.rms_normalize(r * 7.0)[1:], n[1:], rtol=1e-6, atol=0)
    e = np.zeros((1, 64))
    e[0, 5] = 2.0
    assert np.isclose(oracle.rms_normalize(e)[0, 5], 2.0 / np.sqrt(4 / 64 + 1e-6), rtol=1e-15)


def test_stack_without_norm_grows_quadratically():
    """Random-weight SwiGLU layers roughly square the activation scale, so an
    un-normalized residual stack blows up: the reason the stack normalizes."""
    H, I = 128, 64
    rec = synth.make_record(2, 96, 0, 0, H, I)
    mats = oracle.expert_matrices(rec, H, I)
    x = np.random.default_rng(0).standard_normal((1, H))
    small = oracle.expert_ffn(10 * x, *mats)
    big = oracle.expert_ffn(100 * x, *mats)
    assert 50 < np.abs(big).max() / np.abs(small).max() < 200      # ~ 10^2


# ------------------------------------------- stack with the RMS pre-norm ----

def _scalar_rms(v, eps=1e-6):
    ms = sum(a * a for a in v) / len(v)
    return [a / math.sqrt(ms + eps) for a in v]


def test_stack_with_norm_matches_scalar_loops():
    """Two tiny layers, r_{l+1} = r_l + layer_l(r_l / rms(r_l)), every step as
    pure-Python scalar loops (norm, router, top-k, softmax, FFNs, residual)
    against oracle_stack(norm=True).  The input is scaled by 5 so the norm
    changes the layer input and the residual differs from the normalized rows
    (a residual taken from the normalized rows, a norm left out, or a norm
    applied to the output would each fail)."""
    H, E, k, I, Is, T = 64, 4, 2, 64, 64, 2
    layers, scal = [], []
    for l in range(2):
        router = synth.make_router(8, 95, l, H, E)
        recs = [synth.make_record(8, 95, l, e, H, I) for e in range(E)]
        shared = synth.make_record(8, 95, l, 0, H, Is, shared=True)
        beta = np.random.default_rng(30 + l).standard_normal(E) * 0.01
        layers.append(oracle.OracleLayer(H, E, k, I, Is, router, beta,
                                         (lambda rs: (lambda e: rs[e]))(recs), shared))
        scal.append((router, beta, recs, shared))
    x = 5.0 * oracle.bf16_bits_to_f64(synth.make_hidden(8, 95, T, H))
    r = x.tolist()
    for router, beta, recs, shared in scal:
        xin = [_scalar_rms(row) for row in r]
        ys, _, _ = _scalar_layer(xin, router, beta, recs, shared, H, E, k, I, Is)
        r = [[a + b for a, b in zip(rr, yy)] for rr, yy in zip(r, ys.tolist())]
    res = oracle.oracle_stack(layers, x, norm=True)
    want = np.array(r)
    assert np.allclose(res["out"], want, rtol=1e-11, atol=1e-13 * np.abs(want).max())
    # each layer's "input" is the un-normalized residual it was fed
    assert np.array_equal(res["layers"][0]["input"], x)


def test_stack_with_norm_residual_identity():
    """With the norm on: out = x + sum_l y_l, and y_l = layer_l(rms(r_l)) for
    the residual r_l that layer saw."""
    layers = []
    for l in range(3):
        router = synth.make_router(1, 94, l, 128, 8)
        recs = [synth.make_record(1, 94, l, e, 128, 64) for e in range(8)]
        layers.append(oracle.OracleLayer(128, 8, 2, 64, 0, router, None,
                                         (lambda rs: (lambda e: rs[e]))(recs)))
    x = np.random.default_rng(6).standard_normal((4, 128)) * 3.0
    res = oracle.oracle_stack(layers, x, norm=True)
    ys = [lr["y"] for lr in res["layers"]]
    assert np.allclose(res["out"], x + sum(ys), rtol=1e-15, atol=1e-14)
    r = x
    for layer, lr in zip(layers, res["layers"]):
        assert np.array_equal(lr["input"], r)
        again = layer.forward(r / np.sqrt(np.mean(r * r, axis=1, keepdims=True) + 1e-6))
        assert np.allclose(again["y"], lr["y"], rtol=1e-14, atol=1e-15)
        r = r + lr["y"]


def test_forced_selection_is_hand_assembled_sum():
    """forward(force_ids=S): y = sum_j softmax(l[S])_j FFN_{S_j}(x) + FFN_s(x),
    assembled here with torch (float64, CPU) and scipy's softmax, on a forced
    selection that differs from the top-k (the lowest-logit experts), so an
    ignored force_ids fails."""
    from scipy.special import softmax
    H, E, k, I, Is = 128, 6, 2, 64, 128
    layer, recs, shared = _tiny_layer(H, E, k, I, Is, beta=np.linspace(0, 0.5, E))
    x = np.random.default_rng(13).standard_normal((3, H))
    lg = layer.logits(x)
    top, _ = oracle.select_topk(lg, k)
    forced = np.argsort(lg, axis=1)[:, :k]           # the k lowest logits
    assert not any(set(a) == set(b) for a, b in zip(top.tolist(), forced.tolist()))
    res = layer.forward(x, force_ids=forced)
    assert np.array_equal(res["ids"], forced)
    for t in range(3):
        p = softmax(lg[t, forced[t]])
        assert np.allclose(res["p"][t], p, rtol=1e-14, atol=0)
        y = _torch_ffn(x[t:t + 1], *oracle.expert_matrices(shared, H, Is))[0]
        for j in range(k):
            y = y + p[j] * _torch_ffn(x[t:t + 1], *oracle.expert_matrices(recs[forced[t, j]], H, I))[0]
        assert np.allclose(res["y"][t], y, rtol=1e-12, atol=1e-12 * np.abs(y).max())


def test_concurrent_expert_evaluation_is_identical():
    """forward(pool=executor) gives bitwise the same result as the serial loop."""
    from concurrent.futures import ThreadPoolExecutor
    layer, _, _ = _tiny_layer(beta=np.zeros(6))
    x = np.random.default_rng(14).standard_normal((9, 128))
    a = layer.forward(x)
    with ThreadPoolExecutor(4) as ex:
        b = layer.forward(x, pool=ex)
    for key in ("y", "ids", "p", "gap", "logits"):
        assert np.array_equal(a[key], b[key]), key


def test_stack_forced_selections():
    """oracle_stack(force_ids=...) with each layer's own selection is bitwise
    the unforced stack; with another selection at one layer it is the
    hand-composed stack of forward(force_ids) calls and residual adds."""
    layers = []
    for l in range(3):
        router = synth.make_router(3, 92, l, 128, 8)
        recs = [synth.make_record(3, 92, l, e, 128, 64) for e in range(8)]
        layers.append(oracle.OracleLayer(128, 8, 2, 64, 0, router, None,
                                         (lambda rs: (lambda e: rs[e]))(recs)))
    x = np.random.default_rng(7).standard_normal((5, 128)) * 2.0
    base = oracle.oracle_stack(layers, x, norm=True)
    own = [lr["ids"] for lr in base["layers"]]
    again = oracle.oracle_stack(layers, x, norm=True, force_ids=own)
    assert np.array_equal(again["out"], base["out"])
    other = [own[0], np.array([[6, 7]] * 5), own[2]]
    forced = oracle.oracle_stack(layers, x, norm=True, force_ids=other)
    r = x
    for layer, sel in zip(layers, other):
        r = r + layer.forward(oracle.rms_normalize(r), force_ids=sel)["y"]
    assert np.array_equal(forced["out"], r)
    assert not np.allclose(forced["out"], base["out"])
