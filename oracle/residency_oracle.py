"""Plain reference of the delta cache policy — TEST INFRASTRUCTURE ONLY (nothing in the product
library imports or calls it; the library's C++ manager is checked against it by the tests).

What it follows (BitDelta post, "Infrastructure details"):
* cache eviction policy: LRU weighted by request rate; the variants with the most traffic stay
  pinned (in practice the top 6 by volume are always resident) and the rest share the remaining
  space with least-recently-used eviction;
* cold start: a request for a variant that is not resident pays for loading its delta, after
  which it stays cached until evicted;
* request routing: while a variant's delta is being loaded, further requests for it wait for that
  load instead of each starting its own.

Readings where the post is silent (listed in the design notes):
* request rate = the number of requests seen so far; the pinned set is the num_pinned variants
  with the highest counts (ties to the smaller id), among variants requested at least once;
* a variant that is loading is neither evictable nor loaded twice; pinned variants are never
  evicted; a request that cannot be made to fit (everything else resident is pinned or loading)
  changes nothing but the counts and is answered "no room";
* a variant still in use is not "least recently used" in any sense the eviction could mean: a
  request may hold its variant (answers hit / load / queued), and a held variant is not evicted
  until every holder has released it;
* eviction takes the least recently requested evictable variant first (ties to the smaller id),
  one at a time, until the new delta fits in the capacity.

Parity status: pinned by tests/test_residency.py (hand-derived traces, one of them with holds,
and invariants over random traces).
"""
from __future__ import annotations

ABSENT, LOADING, RESIDENT = 0, 1, 2
HIT, LOAD, QUEUED, NO_ROOM = 0, 1, 2, 3


class ResidencyRef:
    def __init__(self, variant_bytes, capacity_bytes: int, num_pinned: int = 6):
        self.size = [int(b) for b in variant_bytes]
        if any(b <= 0 for b in self.size) or capacity_bytes <= 0 or num_pinned < 0:
            raise ValueError("sizes and capacity must be positive, num_pinned >= 0")
        self.cap = int(capacity_bytes)
        self.k = int(num_pinned)
        n = len(self.size)
        self.count = [0] * n
        self.last = [0] * n   # time of the latest request (0 = never)
        self.state = [ABSENT] * n
        self.holds = [0] * n  # requests holding the variant, not yet released
        self.clock = 0

    def pinned(self):
        order = sorted(range(len(self.size)), key=lambda v: (-self.count[v], v))
        return {v for v in order[: self.k] if self.count[v] > 0}

    def used(self) -> int:
        return sum(s for s, st in zip(self.size, self.state) if st != ABSENT)

    def request(self, v: int, hold: bool = False):
        """One request for variant v: (action, evicted ids in eviction order).  With hold, any
        answer but "no room" also makes the request a holder of v."""
        self.clock += 1
        self.count[v] += 1
        self.last[v] = self.clock
        if self.state[v] == RESIDENT:
            self.holds[v] += int(hold)
            return HIT, []
        if self.state[v] == LOADING:
            self.holds[v] += int(hold)
            return QUEUED, []
        pins = self.pinned()
        evictable = [u for u in range(len(self.size))
                     if self.state[u] == RESIDENT and u not in pins and u != v
                     and self.holds[u] == 0]
        evictable.sort(key=lambda u: (self.last[u], u))
        need = self.used() + self.size[v] - self.cap
        if need > sum(self.size[u] for u in evictable):
            return NO_ROOM, []
        evicted = []
        for u in evictable:
            if need <= 0:
                break
            self.state[u] = ABSENT
            need -= self.size[u]
            evicted.append(u)
        self.state[v] = LOADING
        self.holds[v] += int(hold)
        return LOAD, evicted

    def release(self, v: int):
        if self.holds[v] == 0:
            raise ValueError("variant has no holder")
        self.holds[v] -= 1

    def load_done(self, v: int):
        if self.state[v] != LOADING:
            raise ValueError("variant is not loading")
        self.state[v] = RESIDENT
