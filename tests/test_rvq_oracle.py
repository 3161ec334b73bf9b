"""Pins of the residual-VQ oracle (oracle/rvq_ref.py): the byte layout read
by a scalar loop written from the format text, closed-form codebooks, the
3.00 bits per weight the pages state, stage linearity, a basis vector reading
a column, and the partial inner-product table method the pages describe (3
lookups and 2 additions per run) giving the same product as reconstructing."""
import numpy as np

import oracle
import synth


def test_three_bits_per_weight():
    for r, k in ((64, 64), (4096, 7168), (1408, 2816)):
        assert synth.rvq_bytes(r, k) * 8 == 3 * r * k


def test_layout_against_a_scalar_reading():
    R, K = 128, 192
    buf = synth.make_rvq_matrix(3, R, K)
    cb = oracle.rvq_codebooks_f64(synth.make_rvq_codebooks(3))
    w = oracle.rvq_reconstruct(buf, 0, R, K, synth.make_rvq_codebooks(3))
    for r in (0, 5, 63, 64, 127):
        for c in (0, 7, 8, 63, 64, 100, 191):
            rb, rr = divmod(r, 64)
            g, cc = divmod(c, 64)
            j, d = divmod(cc, 8)
            base = (rb * (K // 64) + g) * 1536
            want = sum(cb[s][int(buf[base + s * 512 + rr * 8 + j])][d] for s in range(3))
            assert w[r, c] == want


def test_closed_form_codebooks():
    """C_0[c] = (c, 0, ..., 0), C_1 = C_2 = 0: W[r, 8j] = i_0(r, j), zero elsewhere."""
    R, K = 64, 128
    buf = synth.make_rvq_matrix(4, R, K)
    cb = np.zeros((3, 256, 8), dtype=np.float16)
    cb[0, :, 0] = np.arange(256)
    w = oracle.rvq_reconstruct(buf, 0, R, K, cb.view(np.uint16))
    idx = oracle.rvq_indices(buf, 0, R, K)
    assert np.array_equal(w[:, 0::8], idx[0].astype(np.float64))
    mask = np.ones(K, bool)
    mask[0::8] = False
    assert not w[:, mask].any()


def test_stages_add_up():
    R, K = 64, 128
    buf = synth.make_rvq_matrix(5, R, K)
    cb = synth.make_rvq_codebooks(5).view(np.float16).reshape(3, 256, 8)
    total = oracle.rvq_reconstruct(buf, 0, R, K, cb.view(np.uint16))
    parts = 0
    for s in range(3):
        one = np.zeros_like(cb)
        one[s] = cb[s]
        parts = parts + oracle.rvq_reconstruct(buf, 0, R, K, one.view(np.uint16))
    assert np.array_equal(total, parts)


def test_basis_vector_reads_a_column():
    R, K = 128, 128
    buf = synth.make_rvq_matrix(6, R, K)
    cbb = synth.make_rvq_codebooks(6)
    w = oracle.rvq_reconstruct(buf, 0, R, K, cbb)
    for k in (0, 9, 127):
        x = np.zeros((1, K))
        x[0, k] = 1.0
        assert np.array_equal(oracle.rvq_gemv(buf, 0, R, K, cbb, x)[0], w[:, k])


def test_table_method_equals_reconstruct_then_multiply():
    """T_s[t, j, c] = <C_s[c], x_t[8j:8j+8]>; y[t, r] = sum_j sum_s T_s[t, j, i_s(r, j)]."""
    R, K, T = 128, 256, 3
    buf = synth.make_rvq_matrix(7, R, K)
    cbb = synth.make_rvq_codebooks(7)
    cb = oracle.rvq_codebooks_f64(cbb)
    x = np.random.default_rng(7).standard_normal((T, K))
    idx = oracle.rvq_indices(buf, 0, R, K)
    xs = x.reshape(T, K // 8, 8)
    y = np.zeros((T, R))
    for s in range(3):
        tab = np.einsum("cd,tjd->tjc", cb[s], xs)                  # [T, K/8, 256]
        y += tab[:, np.arange(K // 8)[None, :], idx[s]].sum(axis=2)
    assert np.allclose(y, oracle.rvq_gemv(buf, 0, R, K, cbb, x), rtol=1e-12, atol=1e-14)
