"""Pins of the expert-cache model (oracle/cache_ref.py) on hand-worked
sequences and on properties any bounded cache must have."""
import itertools

import numpy as np
import pytest

from oracle import OracleExpertCache


def test_lfu_then_lru_then_lowest_slot():
    c = OracleExpertCache(8, 2, 100)
    assert c.demand([0]) == [(0, 0)]            # free slots first, lowest first
    assert c.demand([1]) == [(1, 1)]
    # both used once: the least recently used (expert 0, slot 0) goes
    assert c.demand([2]) == [(2, 0)]
    c.demand([1])                               # expert 1: two uses
    # expert 2 (one use) goes before expert 1 (two), although 1 was used earlier
    assert c.demand([3]) == [(3, 0)]
    assert c.resident() == {1: 1, 3: 0}
    assert c.stats["demand_hits"] == 1 and c.stats["demand_misses"] == 4
    assert c.stats["demand_bytes"] == 400


def test_current_set_is_never_evicted():
    c = OracleExpertCache(6, 3, 1)
    c.demand([0, 1, 2])
    for _ in range(5):
        c.demand([0])                           # 0 very frequent
    # 0 is selected again together with two new experts: 1 and 2 go, 0 stays
    copies = c.demand([0, 4, 5])
    assert sorted(e for e, _ in copies) == [4, 5]
    assert c.slot_of[0] >= 0


def test_missing_experts_take_slots_in_expert_order():
    c = OracleExpertCache(10, 4, 1)
    assert c.demand([7, 3, 9, 1]) == [(1, 0), (3, 1), (7, 2), (9, 3)]


def test_capacity_equal_to_experts_misses_only_once():
    rng = np.random.default_rng(0)
    c = OracleExpertCache(16, 16, 1)
    seen = set()
    for _ in range(50):
        sel = set(rng.choice(16, 4, replace=False).tolist())
        copies = c.demand(sel)
        assert set(e for e, _ in copies) == sel - seen
        seen |= sel
    assert c.stats["demand_misses"] == len(seen)


def test_working_set_capacity_always_places_and_keeps_invariants():
    """With as many slots as one forward can select, every forward places all
    its experts; slot_of and owner stay inverse, and the counters add up."""
    rng = np.random.default_rng(1)
    E, k, T = 32, 4, 2
    c = OracleExpertCache(E, k * T, 7)
    for _ in range(200):
        sel = set(rng.choice(E, (T, k)).reshape(-1).tolist())
        if rng.random() < 0.5:
            c.prefetch(rng.choice(E, k, replace=False))
        c.demand(sel)
        for e in sel:
            assert c.owner[c.slot_of[e]] == e
        for s, o in enumerate(c.owner):
            assert o < 0 or c.slot_of[o] == s
        assert sum(1 for v in c.slot_of if v >= 0) == sum(1 for o in c.owner if o >= 0)
    st = c.stats
    assert st["demand_hits"] + st["demand_misses"] == st["selected"]
    assert st["prefetch_used"] + st["prefetch_evicted_unused"] <= st["prefetched"]
    with pytest.raises(RuntimeError):
        c.demand(range(k * T + 1))              # more than the slots: refused


def test_prefetch_is_not_a_use_and_is_evicted_first():
    c = OracleExpertCache(8, 3, 1)
    c.demand([0, 1])
    c.demand([0, 1])
    assert c.prefetch([5]) == [(5, 2)]          # the free slot
    assert c.freq[5] == 0
    # a demand for 6: 5 (prefetched, unused, no uses) goes, not 0 or 1
    assert c.demand([6]) == [(6, 2)]
    assert c.stats["prefetch_evicted_unused"] == 1 and c.stats["prefetch_used"] == 0
    c.prefetch([4])                             # evicts the least used: 6 (one use)
    c.demand([4])
    assert c.stats["prefetch_used"] == 1 and c.stats["demand_hits"] == 3


def test_lfu_brute_force_small():
    """Against a direct restatement on tiny cases: after each forward the
    resident set is the current set plus, of the rest, the survivors chosen by
    the key order; checked over all short sequences of single demands."""
    E, S = 4, 2
    for seq in itertools.product(range(E), repeat=5):
        c = OracleExpertCache(E, S, 1)
        freq = [0] * E
        last = {}
        res = {}
        for t, e in enumerate(seq, 1):
            freq[e] += 1
            if e not in res:
                if len(res) == S:
                    victim = min(res, key=lambda x: (freq[x], last[x], res[x]))
                    slot = res.pop(victim)
                else:
                    slot = min(set(range(S)) - set(res.values()))
                res[e] = slot
            last[e] = t
            c.demand([e])
            assert c.resident() == res, (seq, t)
