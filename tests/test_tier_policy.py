"""Pins of the residency-tier policy model (oracle/tier_ref.py), worked by hand from the
cache rules of "MoE 路由与专家流式加载" §1.3 (pin, then LRU, else a working slot; evict
the least recently used), §3 (pinned experts never evicted) and §4 (swap only when
heat[fh] > heat[fc] + heat[fc]/4 + 4, then every heat halved).  CPU only."""
from oracle.tier_ref import TierRef


def test_lru_worked_example():
    # 6 experts, 3 slots, nothing pinned
    t = TierRef(6, 3)
    t.forward({0: 1, 1: 2})          # empty slots in order: 0 -> s0, 1 -> s1
    assert t.slot_expert == [0, 1, -1] and t.last_copies == [(0, 0), (1, 1)]
    t.forward({2: 1})                # the empty slot s2 before any used one
    assert t.slot_expert == [0, 1, 2] and t.slot_used == [1, 1, 2]
    t.forward({0: 1, 3: 1})          # 0 hits (stamp 3); 3 evicts the oldest free slot, s1
    assert t.slot_expert == [0, 3, 2] and t.expert_slot[1] == -1 and t.slot_used == [3, 3, 2]
    t.forward({1: 1, 2: 1})          # 2 hits; s0 and s1 both stamped 3: the lower slot, s0
    assert t.slot_expert == [1, 3, 2] and t.last_copies == [(1, 0)]
    assert (t.hits, t.misses) == (2, 5)
    assert t.heat == [2, 3, 2, 1, 0, 0] and t.usage == t.heat


def test_union_slots_are_never_victims():
    # a union's own resident experts keep their slots even when they are the oldest
    t = TierRef(8, 3)
    t.forward({0: 1, 1: 1, 2: 1})
    t.forward({0: 1, 1: 1, 5: 1})    # victims exclude s0, s1 (in this union): 5 -> s2
    assert t.slot_expert == [0, 1, 5]


def test_pinned_slots_are_never_evicted():
    t = TierRef(8, 3, pins=[4])
    assert t.slot_expert == [4, -1, -1] and t.slot_pinned == [1, 0, 0]
    for e in range(8):
        if e != 4:
            t.forward({e: 1})
        assert t.slot_expert[0] == 4
    t.forward({4: 5, 6: 1})
    assert t.expert_slot[4] == 0 and t.heat[4] == 5


def test_repin_hysteresis_threshold():
    # pinned expert 0 with heat 8: the bar is 8 + 8 // 4 + 4 = 14, which must be exceeded
    t = TierRef(4, 3, pins=[0])
    t.heat = [8, 14, 3, 0]
    t.repin(4)
    assert t.slot_pinned == [1, 0, 0] and t.swaps == 0 and t.heat == [4, 7, 1, 0]
    t.heat = [8, 15, 3, 0]
    t.repin(4)                       # 15 > 14: expert 1 (not resident) replaces 0 in slot 0
    assert t.slot_expert[0] == 1 and t.expert_slot[0] == -1 and t.last_copies == [(1, 0)]
    assert t.swaps == 1 and t.heat == [4, 7, 1, 0]


def test_repin_cached_expert_takes_the_pin():
    t = TierRef(4, 3, pins=[0])
    t.forward({2: 1})                # expert 2 cached in s1
    t.heat = [1, 0, 30, 0]
    t.repin(4)                       # 30 > 1 + 0 + 4: the flag moves, no copy; 0 stays cached
    assert t.slot_pinned == [0, 1, 0] and t.slot_expert == [0, 2, -1] and t.last_copies == []
    assert t.swaps == 1


def test_repin_at_most_max_swaps_and_ties():
    t = TierRef(8, 4, pins=[0, 1, 2])
    t.heat = [0, 0, 0, 0, 50, 50, 50, 0]
    t.repin(2)                       # two swaps: coldest pinned by id (0, then 1) get the
    assert t.slot_expert[:3] == [4, 5, 2]   # hottest unpinned by id (4, then 5)
    assert t.swaps == 2 and t.heat == [0, 0, 0, 0, 25, 25, 25, 0]


def test_prefetch_counts_nothing_and_keeps_the_step():
    t = TierRef(8, 3)
    t.forward({0: 1})
    t.prefetch([5, 6, 5])
    assert t.slot_expert == [0, 5, 6] and t.step == 1 and t.slot_used == [1, 1, 1]
    assert t.heat[5] == 0 and t.prefetched == 2 and (t.hits, t.misses) == (0, 1)
    t.forward({5: 2})                # now a hit
    assert (t.hits, t.misses) == (1, 1)
