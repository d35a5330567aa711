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


def test_frequency_admission_worked_sequence():
    # 2 slots, admission by touch counts.  Call 1 {0, 1}: empty slots take both ->
    # [0, 1], counts 0:1 1:1.  Call 2 {0}: hit (count 0:2).  Call 3 {2}: miss; the slots
    # not used by call 3 by (stamp, index): slot 1 (key 1, stamp 1), slot 0 (stamp 2);
    # 2 is paired with slot 1, whose key was touched as often (1 >= 1): not admitted,
    # 2 read from its home, nothing evicted.  Call 4 {2}: 2 now touched twice > 1: it
    # evicts 1.  Plain LRU evicts 1 already in call 3.
    c = LRUCache(2, admit=True)
    c.call([0, 1])
    c.call([0])
    slot_of, hits, missing, evicted = c.call([2])
    assert slot_of == {} and missing == [2] and evicted == [] and c.key == [0, 1]
    assert (c.uncached, c.last_uncached) == (1, 1) and c.stamp == [2, 1]
    slot_of, _, _, evicted = c.call([2])
    assert slot_of == {2: 1} and evicted == [1] and c.key == [0, 2] and c.last_uncached == 0
    assert c.count == {0: 2, 1: 1, 2: 2}
    lru = LRUCache(2)
    lru.call([0, 1])
    lru.call([0])
    assert lru.call([2])[3] == [1]


def test_frequency_admission_invariants_random_calls():
    rng = np.random.default_rng(1)
    c = LRUCache(12, admit=True)
    touches = {}
    p = 1.0 / np.arange(1, 41) ** 1.1                  # skewed popularity over 40 keys
    p /= p.sum()
    for _ in range(300):
        keys = rng.choice(40, size=rng.integers(1, 13), replace=False, p=p)
        for k in keys:
            touches[int(k)] = touches.get(int(k), 0) + 1
        before = {k for k in c.key if k >= 0}
        old_keys = list(c.key)
        slot_of, hits, missing, evicted = c.call(keys)
        assert hits == len(set(keys) & before) and len(missing) == len(set(keys) - before)
        assert c.last_uncached == len(missing) - len(set(missing) & set(slot_of))
        for s in range(c.n):                               # a key is replaced only by a more touched one
            if old_keys[s] >= 0 and c.key[s] != old_keys[s]:
                assert c.count[old_keys[s]] < c.count[c.key[s]]
                assert old_keys[s] in evicted
        held = [k for k in c.key if k >= 0]
        assert len(held) == len(set(held))
        assert c.count == touches
    plain = LRUCache(12)
    rng = np.random.default_rng(1)
    for _ in range(300):
        plain.call(rng.choice(40, size=rng.integers(1, 13), replace=False, p=p))
    assert c.hits > plain.hits                           # the point of the admission rule
