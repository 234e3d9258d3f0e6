"""CPU model of the routed-expert cache's policy.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it; the library never does,
and it shares no code with the library's C++ cache.

What it models (QuarkStar README, "Running Models Larger Than Available
Memory"): the routed experts that do not fit device memory go through a
bounded cache of expert slots, a prefix of layers can stay fully resident,
and a warm start preloads a bounded popularity hotlist.  The page does not
name the replacement policy; the reading taken here is plain
least-recently-used over all slots:

* A decode call uses, in order, the distinct experts of each of its paged
  layers (layers at or after ``resident_layers``): layers ascending, within a
  layer the order of first appearance over tokens, then ranks.  Several
  tokens picking one expert are one use.
* A use of a cached expert is a hit and makes it the most recent.  A use of
  an uncached one is a miss: it is admitted into the free slot of lowest
  index, or, with no slot free, into the slot of the least recently used
  expert, which is evicted.
* Preloading takes (layer, expert) pairs hottest first into free slots only
  (nothing is evicted, a cached pair is skipped) and places each at the
  least-recent end, so the coldest preloaded expert is the first evicted.

Keys are (layer, expert) pairs.  The model has no notion of bytes or time:
the library's outputs do not depend on where an expert is read from, so the
policy is all there is to check.
"""
from __future__ import annotations

import numpy as np

STATS = ("hits", "misses", "admissions", "evictions", "preloaded")


class ExpertCacheModel:
    """Slot table and LRU order of a cache with ``slots`` slots."""

    def __init__(self, slots: int):
        self.slots = int(slots)
        self.owner = [None] * self.slots      # slot -> key
        self.where = {}                       # key -> slot
        self.recency = []                     # occupied slots, least recent first
        self.stats = {n: 0 for n in STATS}

    def _free(self):
        return [v for v in range(self.slots) if self.owner[v] is None]

    def use(self, key) -> bool:
        """One use; True on a hit."""
        key = tuple(key)
        if key in self.where:
            v = self.where[key]
            self.recency.remove(v)
            self.recency.append(v)
            self.stats["hits"] += 1
            return True
        self.stats["misses"] += 1
        free = self._free()
        if free:
            v = free[0]
        elif self.recency:
            v = self.recency.pop(0)
            del self.where[self.owner[v]]
            self.stats["evictions"] += 1
        else:
            return False                      # no slots at all
        self.owner[v] = key
        self.where[key] = v
        self.recency.append(v)
        self.stats["admissions"] += 1
        return False

    def preload(self, keys) -> None:
        for key in keys:
            key = tuple(int(x) for x in key)
            free = self._free()
            if not free:
                break
            if key in self.where:
                continue
            v = free[0]
            self.owner[v] = key
            self.where[key] = v
            self.recency.insert(0, v)
            self.stats["preloaded"] += 1

    @staticmethod
    def call_uses(ids, layer0: int, resident_layers: int):
        """The ordered uses of one decode call; ids [n_layers][T][k]."""
        ids = np.asarray(ids)
        uses = []
        for i in range(ids.shape[0]):
            layer = layer0 + i
            if layer < resident_layers:
                continue
            seen = set()
            for e in ids[i].reshape(-1):
                e = int(e)
                if e not in seen:
                    seen.add(e)
                    uses.append((layer, e))
        return uses

    def call(self, ids, layer0: int, resident_layers: int):
        """Apply one decode call; returns the hit flag of each use."""
        return [self.use(u) for u in self.call_uses(ids, layer0, resident_layers)]

    def table(self) -> np.ndarray:
        """(layer, expert) per slot, (-1, -1) for a free one: int32 [slots][2]."""
        t = np.full((self.slots, 2), -1, dtype=np.int32)
        for v, key in enumerate(self.owner):
            if key is not None:
                t[v] = key
        return t
