"""Pins of the oracle's expert-cache policy (oracle.cache.LRUCache) against
sequences worked by hand and its invariants (no GPU)."""
import numpy as np
import pytest

from oracle.cache import LRUCache


def test_worked_sequence():
    # 3 slots.  Call 1 {5, 2}: both miss, keys in increasing order take the empty
    # slots 0, 1 -> [2, 5, -].  Call 2 {5, 9}: 5 hits (slot 1, stamp 2); 9 misses and
    # takes the empty slot 2 -> [2, 5, 9].  Call 3 {7}: misses; the slots not used by
    # call 3 by (stamp, index): slot 0 (stamp 1), slot 1 (2), slot 2 (2) -> 7 evicts 2
    # in slot 0.  Call 4 {2, 9, 5}: 9 and 5 hit (slots 2, 1); 2 misses and takes the
    # only slot not used by call 4, slot 0, evicting 7.
    c = LRUCache(3)
    assert c.call([5, 2]) == ({2: 0, 5: 1}, 0, [2, 5], [])
    assert c.call([5, 9]) == ({5: 1, 9: 2}, 1, [9], [])
    assert c.call([7]) == ({7: 0}, 0, [7], [2])
    assert c.key == [7, 5, 9] and c.stamp == [3, 2, 2]
    assert c.call([2, 9, 5]) == ({9: 2, 5: 1, 2: 0}, 2, [2], [7])
    assert (c.hits, c.misses) == (3, 5)


def test_least_recently_used_is_evicted_first():
    c = LRUCache(4)
    c.call([0, 1, 2, 3])                 # slots 0..3, stamp 1
    c.call([3])                          # slot 3 stamp 2
    c.call([1])                          # slot 1 stamp 3
    _, _, _, ev = c.call([10, 11])       # victims: slot 0 (stamp 1), slot 2 (stamp 1)
    assert ev == [0, 2] and c.key == [10, 1, 11, 3]
    _, _, _, ev = c.call([12])           # oldest now: slot 3 (stamp 2)
    assert ev == [3]


def test_invariants_random_calls():
    rng = np.random.default_rng(0)
    c = LRUCache(16)
    for _ in range(200):
        keys = rng.choice(40, size=rng.integers(1, 17), replace=False)
        before = {k for k in c.key if k >= 0}
        slot_of, hits, missing, evicted = c.call(keys)
        assert hits == len(set(keys) & before) and len(missing) == len(set(keys) - before)
        assert set(evicted) <= before - set(keys)
        held = [k for k in c.key if k >= 0]
        assert len(held) == len(set(held))                      # a key in one slot at most
        assert all(c.key[slot_of[k]] == k for k in keys)        # every touched key resident
        assert all(c.stamp[slot_of[k]] == c.clock for k in keys)


def test_more_keys_than_free_slots_stay_uncached():
    # 3 slots hold 1, 2, 3; call {2, 4, 5, 6}: 2 hits (slot 1), the two free slots
    # (0 then 2, both stamp 1) take 4 and 5 in key order, 6 stays uncached.
    c = LRUCache(3)
    c.call([1, 2, 3])
    slot_of, hits, missing, evicted = c.call([2, 4, 5, 6])
    assert slot_of == {2: 1, 4: 0, 5: 2} and hits == 1 and missing == [4, 5, 6]
    assert evicted == [1, 3] and c.key == [4, 2, 5] and (c.uncached, c.last_uncached) == (1, 1)
    c.call([7, 8, 9, 10, 11])                        # all miss: 3 placed, 2 uncached
    assert c.key == [7, 8, 9] and c.uncached == 3
