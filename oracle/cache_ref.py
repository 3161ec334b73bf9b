"""Plain model of the per-layer expert cache, for checking the GPU's.

TEST INFRASTRUCTURE ONLY: imported by tests/, never by the GPU library.

What it models, and where it comes from:

* a bounded set of slots per layer, filled with the records the router
  selects, least frequently used evicted first -- TurboFieldfare page, section
  "Token üretim süreci" (the top-8 expert ids are compared with a 16-slot LFU
  cache per layer, misses are read in before the experts run); WASTE page,
  section "RAM bütçesi ve dar performans aralığı" (a bounded expert cache; a
  budget below one token's working set is refused);
* prefetch of the next layer's predicted experts -- WASTE page, section
  "Önceden okuma ve router tahmini" (the next layer's router, run one residual
  ahead, prefetches experts; the real router still decides).

Where the pages leave it open (readings of this design): frequency counts the
forwards that selected an expert; among equal counts the least recently used
slot goes first, then the lowest slot; free slots go before any occupied one;
a slot whose expert the current forward (or prediction) selects is never
taken; the missing experts take the chosen slots in ascending expert order; a
prefetch does not count as a use, and a prefetched record not used yet is
marked so that its later use or eviction is counted.
"""
from __future__ import annotations

__all__ = ["OracleExpertCache"]


class OracleExpertCache:
    def __init__(self, n_experts: int, n_slots: int, rec_bytes: int):
        self.E, self.S, self.rec_bytes = n_experts, n_slots, rec_bytes
        self.slot_of = [-1] * n_experts
        self.owner = [-1] * n_slots
        self.freq = [0] * n_experts
        self.stamp = [0] * n_slots
        self.prefetched = [False] * n_slots
        self.clock = 0
        self.stats = dict(forwards=0, selected=0, demand_hits=0, demand_misses=0, demand_bytes=0,
                          prefetched=0, prefetch_bytes=0, prefetch_used=0,
                          prefetch_evicted_unused=0)

    def _victims(self, current: set, n: int) -> list:
        """The first n slots by (occupied, frequency of the occupant, last use,
        slot), leaving out slots whose expert is in `current`."""
        cand = []
        for s in range(self.S):
            o = self.owner[s]
            if o >= 0 and o in current:
                continue
            cand.append(((0, 0, 0, s) if o < 0 else (1, self.freq[o], self.stamp[s], s)))
        cand.sort()
        if len(cand) < n:
            raise RuntimeError("more missing experts than free or evictable slots")
        return [c[3] for c in cand[:n]]

    def _place(self, missing: list, current: set, prefetch: bool) -> list:
        copies = []
        for e, s in zip(missing, self._victims(current, len(missing))):
            o = self.owner[s]
            if o >= 0:
                self.slot_of[o] = -1
            if self.prefetched[s]:
                self.stats["prefetch_evicted_unused"] += 1
            self.owner[s], self.slot_of[e] = e, s
            self.stamp[s] = self.clock
            self.prefetched[s] = prefetch
            copies.append((e, s))
        return copies

    def demand(self, experts) -> list:
        """One forward selecting `experts`: returns the (expert, slot) copies."""
        sel = sorted(set(int(e) for e in experts))
        self.clock += 1
        missing = []
        for e in sel:
            s = self.slot_of[e]
            if s < 0:
                missing.append(e)
            else:
                self.stats["demand_hits"] += 1
                self.stamp[s] = self.clock
                if self.prefetched[s]:
                    self.prefetched[s] = False
                    self.stats["prefetch_used"] += 1
            self.freq[e] += 1
        copies = self._place(missing, set(sel), prefetch=False)
        self.stats["forwards"] += 1
        self.stats["selected"] += len(sel)
        self.stats["demand_misses"] += len(copies)
        self.stats["demand_bytes"] += len(copies) * self.rec_bytes
        return copies

    def prefetch(self, experts) -> list:
        """Prefetch the predicted `experts`: returns the (expert, slot) copies."""
        pred = sorted(set(int(e) for e in experts))
        missing = [e for e in pred if self.slot_of[e] < 0]
        copies = self._place(missing, set(pred), prefetch=True)
        self.stats["prefetched"] += len(copies)
        self.stats["prefetch_bytes"] += len(copies) * self.rec_bytes
        return copies

    def resident(self) -> dict:
        return {e: s for e, s in enumerate(self.slot_of) if s >= 0}
