"""Plain model of the expert residency tier's policy (which expert sits in which slot).

TEST INFRASTRUCTURE ONLY: used by the tests to check the device tier's state exactly;
never imported by the product path.  Pure Python on small integers.

It follows the cache of "MoE 路由与专家流式加载":
  §1.3 cache resolution: per union expert, the pinned hot store, then the LRU cache,
       else a working slot is allocated and the expert loaded; used experts go into the
       cache, evicting the least recently used;
  §1.2 heat/usage counters updated by the routing (eheat, eusage);
  §3   the pinned hot store (never evicted) filled from a usage histogram;
  §4   tier_pick_swap: coldest pinned fc against the hottest unpinned fh, swap only if
       heat[fh] > heat[fc] + heat[fc]/4 + 4, at most a few swaps per pass, then every
       heat shifted right by one (tier_decay);
  §5   router-lookahead prefetch of predicted experts.
Readings where the page is silent (the same as the library's header states): union
experts are resolved in ascending id order; a miss takes the free-or-least-recently-used
slot that is neither pinned nor holding an expert of the same union, empty slots first,
then the smallest use stamp, then the lower slot index; heat and usage grow by the
expert's row count in the batch; the coldest pinned expert is the one with the lowest
heat (ties: lower id), the hottest unpinned one the highest heat (ties: lower id); an fh
already cached takes over the pinned flag, otherwise it is loaded into fc's slot.
"""
from __future__ import annotations


class TierRef:
    def __init__(self, n_experts: int, n_slots: int, pins=()):
        E, S = n_experts, n_slots
        self.E, self.S = E, S
        self.slot_expert = [-1] * S
        self.slot_pinned = [0] * S
        self.slot_used = [-1] * S
        self.expert_slot = [-1] * E
        self.heat = [0] * E
        self.usage = [0] * E
        self.step = 0
        self.hits = self.misses = self.swaps = self.prefetched = 0
        self.last_copies = []
        for s, e in enumerate(pins):
            self.slot_expert[s] = e
            self.slot_pinned[s] = 1
            self.slot_used[s] = 0
            self.expert_slot[e] = s
        self.last_copies = [(e, s) for s, e in enumerate(pins)]

    # ------------------------------------------------------------ resolution
    def _resolve(self, union, counts, stamp, count):
        hits, misses = [], []
        for e in union:
            if count:
                self.heat[e] += counts[e]
                self.usage[e] += counts[e]
            (hits if self.expert_slot[e] >= 0 else misses).append(e)
        busy = set()
        for e in hits:
            s = self.expert_slot[e]
            busy.add(s)
            self.slot_used[s] = stamp
        victims = sorted((self.slot_used[s], s) for s in range(self.S)
                         if not self.slot_pinned[s] and s not in busy)
        copies = []
        for (used, s), e in zip(victims, misses):
            old = self.slot_expert[s]
            if old >= 0:
                self.expert_slot[old] = -1
            self.expert_slot[e] = s
            self.slot_expert[s] = e
            self.slot_used[s] = stamp
            copies.append((e, s))
        self.last_copies = copies
        return hits, misses

    def forward(self, counts: dict):
        """One batch: counts maps each union expert to its row count."""
        self.step += 1
        hits, misses = self._resolve(sorted(counts), counts, self.step, True)
        self.hits += len(hits)
        self.misses += len(misses)

    def prefetch(self, experts):
        """Make the predicted experts resident; no counters, no new step."""
        self._resolve(sorted(set(experts)), None, self.step, False)
        self.prefetched += len(self.last_copies)

    # ------------------------------------------------------------ repin
    def repin(self, max_swaps: int):
        copies = []
        for _ in range(max_swaps):
            pinned = [self.slot_expert[s] for s in range(self.S) if self.slot_pinned[s]]
            free = [e for e in range(self.E)
                    if self.expert_slot[e] < 0 or not self.slot_pinned[self.expert_slot[e]]]
            if not pinned or not free:
                break
            fc = min(pinned, key=lambda e: (self.heat[e], e))
            fh = min(free, key=lambda e: (-self.heat[e], e))
            hc, hh = self.heat[fc], self.heat[fh]
            if not hh > hc + hc // 4 + 4:
                break
            sc, s2 = self.expert_slot[fc], self.expert_slot[fh]
            if s2 >= 0:
                self.slot_pinned[s2] = 1
                self.slot_pinned[sc] = 0
            else:
                self.expert_slot[fc] = -1
                self.expert_slot[fh] = sc
                self.slot_expert[sc] = fh
                self.slot_used[sc] = self.step
                copies.append((fh, sc))
            self.swaps += 1
        self.heat = [h >> 1 for h in self.heat]
        self.last_copies = copies

    def state(self):
        return dict(step=self.step, hits=self.hits, misses=self.misses, swaps=self.swaps,
                    prefetched=self.prefetched, slot_expert=list(self.slot_expert),
                    slot_pinned=list(self.slot_pinned), slot_used=list(self.slot_used),
                    expert_slot=list(self.expert_slot), heat=list(self.heat),
                    usage=list(self.usage), copies=list(self.last_copies))
