"""Budgeted expert cache, oracle side: the replacement policy as a plain simulation.

TEST INFRASTRUCTURE: only tests/ may import this module.  It shares no code with
the HIP library.

The pages stream routed experts from slower storage into an in-memory expert
cache on misses, with configurable cache budgets ("DwarfStar (ds4)"
(opensourcealternatives.to), section FAQ; "DwarfStar 4" (aiany.app), section
"What Sets It Apart"), and name no replacement policy.  The reading taken here is
least-recently-used over a fixed number of slots, with every tie broken by index:

  state: slot -> key or empty, and slot -> stamp (the number of the call that last
  used the slot, 0 for an empty slot).  Call c (c = 1, 2, ...) touches a set of keys:
    1. every touched key already in a slot is a hit: that slot's stamp becomes c;
    2. the missing keys, in increasing key order, take the slots not used by call c
       in increasing (stamp, slot index) order -- empty slots first (stamp 0), then
       the least recently used; a slot's previous key is evicted, the new key and
       stamp c written;
    3. missing keys beyond those slots (a call touching more keys than the budget
       holds) stay uncached: read from their home for this call only.

With frequency admission (admit=True) every key also carries the number of calls
that touched it (counted at the start of each call, saturating at 2^31 - 1), and in
step 2 a missing key takes its slot only when the key the slot holds was touched by
fewer calls than the missing key; otherwise the slot keeps its key and stamp and the
missing key is read from its home for this call (as in step 3).  Empty slots always
take their key.  Under a skewed, stationary popularity this keeps the frequently
used keys resident instead of letting one-off keys evict them.
"""

COUNT_MAX = 2 ** 31 - 1


class LRUCache:
    def __init__(self, n_slots, admit=False):
        self.n = n_slots
        self.admit = admit
        self.count = {}                    # key -> calls that touched it
        self.key = [-1] * n_slots          # slot -> key (-1: empty)
        self.stamp = [0] * n_slots         # slot -> last call that used it
        self.clock = 0
        self.hits = 0
        self.misses = 0
        self.uncached = 0

    def where(self, k):
        for s in range(self.n):
            if self.key[s] == k:
                return s
        return -1

    def call(self, keys):
        """One call touching `keys`; returns (slot of each cached key as a dict, hits,
        missed keys in increasing order (placed first, then the uncached), evicted keys)."""
        keys = sorted(set(int(k) for k in keys))
        self.clock += 1
        c = self.clock
        for k in keys:
            self.count[k] = min(self.count.get(k, 0) + 1, COUNT_MAX)
        slot_of, missing = {}, []
        for k in keys:
            s = self.where(k)
            if s >= 0:
                self.stamp[s] = c
                slot_of[k] = s
            else:
                missing.append(k)
        free = sorted((self.stamp[s], s) for s in range(self.n) if self.stamp[s] < c)
        evicted = []
        placed = 0
        for k, (_, s) in zip(missing, free):
            old = self.key[s]
            if self.admit and old >= 0 and self.count.get(old, 0) >= self.count[k]:
                continue                   # not admitted: read from its home this call
            if old >= 0:
                evicted.append(old)
            self.key[s] = k
            self.stamp[s] = c
            slot_of[k] = s
            placed += 1
        self.hits += len(keys) - len(missing)
        self.misses += len(missing)
        self.uncached += len(missing) - placed
        self.last_uncached = len(missing) - placed
        return slot_of, len(keys) - len(missing), missing, evicted
