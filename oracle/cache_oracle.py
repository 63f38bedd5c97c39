"""Reference document-cache simulation -- TEST INFRASTRUCTURE ONLY.

Plain Python replay of an access trace against a position-agnostic cache
(key = document) or a position-aware cache (key = (document, position)), as
in the hit-ratio model of "LazyAttention" §2 (Eqs. 1-3): LRU eviction with an
OrderedDict, or a static cache of the most popular entries (documents are
numbered by popularity rank).  Small traces only.

Pins (tests/test_cache_sim.py): a static cache's hit ratio converges to
Eq. 1 (agnostic) and Eq. 2 (aware) on long Zipf traces; hand-worked LRU
sequences; a capacity that holds every key misses only on first touches.
"""
from __future__ import annotations

from collections import OrderedDict

__all__ = ["simulate_cache"]


def simulate_cache(docs, pos, num_positions, capacity, policy="agnostic", eviction="lru"):
    aware = policy == "aware"
    if eviction == "static_top":
        top = capacity // num_positions if aware else capacity
        return sum(1 for d in docs if int(d) < top)
    cache = OrderedDict()
    hits = 0
    for i, d in enumerate(docs):
        key = (int(d), int(pos[i])) if aware else int(d)
        if key in cache:
            hits += 1
            cache.move_to_end(key)
            continue
        if capacity == 0:
            continue
        if len(cache) == capacity:
            cache.popitem(last=False)
        cache[key] = True
    return hits
