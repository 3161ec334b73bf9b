"""The GPU parity harness's own acceptance rules, on the CPU: an expert set
inside the 1e-3 logit band must still be a top-k of the oracle's logits up to
that band, and outside it must equal the oracle's."""
import numpy as np
import pytest

from tests import parity as P


def _ref(lg, k):
    import oracle
    lg = np.asarray(lg, dtype=np.float64)
    ids, gap = oracle.select_topk(lg, k)
    return dict(ids=ids, gap=gap, logits=lg)


def test_band_rejects_a_set_that_drops_the_top_expert():
    """Logits [5, 1, 0.9995, -3], k = 2: the k-th/(k+1)-th gap is 5e-4, inside
    the band; {1, 2} is not a valid top-2 (expert 0 beats both by ~4)."""
    ref = _ref([[5.0, 1.0, 0.9995, -3.0]], 2)
    assert ref["gap"][0] < P.GAP
    with pytest.raises(AssertionError):
        P.resolve_ids(ref, np.array([[1, 2]]))
    assert not P.valid_in_band(ref["logits"][0], [1, 2])


def test_band_accepts_either_tied_choice():
    ref = _ref([[5.0, 1.0, 0.9995, -3.0]], 2)
    for sel in ([0, 1], [0, 2], [2, 0]):
        ids, n_tie = P.resolve_ids(ref, np.array([sel]))
        assert n_tie == 1 and set(ids[0].tolist()) == set(sel)


def test_outside_band_ids_must_equal_the_oracle():
    ref = _ref([[5.0, 1.0, 0.5, -3.0]], 2)
    assert ref["gap"][0] > P.GAP
    P.resolve_ids(ref, np.array([[1, 0]]))               # same set, any order
    with pytest.raises(AssertionError):
        P.resolve_ids(ref, np.array([[0, 2]]))


def test_duplicate_or_out_of_range_ids_are_rejected():
    ref = _ref([[5.0, 1.0, 0.9995, -3.0]], 2)
    with pytest.raises(AssertionError):
        P.resolve_ids(ref, np.array([[0, 0]]))
    assert not P.valid_in_band(ref["logits"][0], [0, 7])


def test_valid_in_band_brute_force():
    """valid_in_band agrees with its definition on random small cases: every
    selected logit >= every unselected logit - GAP."""
    import itertools
    rng = np.random.default_rng(0)
    for _ in range(200):
        E = int(rng.integers(2, 7))
        k = int(rng.integers(1, E))
        lg = rng.integers(0, 6, E) * 4e-4                   # steps below and above GAP
        for sel in itertools.combinations(range(E), k):
            rest = [e for e in range(E) if e not in sel]
            want = all(lg[s] >= lg[r] - P.GAP for s in sel for r in rest)
            assert P.valid_in_band(lg, sel) == want


def _zero_router_layer(beta, k=2, H=128, I=64):
    import oracle
    import synth
    from tests import tilebytes as tb
    E = len(beta)
    q = np.full((64, H), 128)
    s = tb.f16bits(np.full((64, H // 64), 2.0 ** -10))
    b = tb.f16bits(np.full((64, H // 64), -128 * 2.0 ** -10))
    router = np.frombuffer(bytes(tb.q8_tiles(q, s, b)), dtype=np.uint8)
    recs = [synth.make_record(4, 93, 0, e, H, I) for e in range(E)]
    return oracle.OracleLayer(H, E, k, I, 0, router, np.asarray(beta, np.float64),
                              lambda e: recs[e])


def test_check_forward_evaluates_the_gpu_choice_inside_the_band():
    """beta = [1, 0.5, 0.5, 0.2] with a zero router: experts 1 and 2 tie for
    the second place.  A GPU result that picks {0, 2} and carries the output
    of {0, 2} passes; one that picks {0, 2} but carries the output of {0, 1}
    fails; so does {0, 3}, outside the band."""
    layer = _zero_router_layer([1.0, 0.5, 0.5, 0.2])
    x = np.random.default_rng(2).standard_normal((3, 128))
    pick = np.array([[0, 2]] * 3)
    good = layer.forward(x, force_ids=pick)
    P.check_forward(layer, x, good["y"], pick, good["p"], "tie, gpu took {0,2}")
    plain = layer.forward(x)
    assert np.array_equal(plain["ids"], [[0, 1]] * 3)
    with pytest.raises(AssertionError):
        P.check_forward(layer, x, plain["y"], pick, good["p"], "tie, wrong output")
    with pytest.raises(AssertionError):
        P.check_forward(layer, x, good["y"], np.array([[0, 3]] * 3), good["p"], "outside band")
