"""Textbook LRU cache -- test infrastructure only (CPU oracle pin).

With one selected position per step there are no ties inside a step, so the
step-LRU of the HiSparse summary article (section 02: LRU metadata drives
replacement in the B-slot device buffer) must reduce to the classic
least-recently-used cache of capacity B.  This is that classic cache, kept
in an ``OrderedDict`` (most recent at the end).
"""

from __future__ import annotations

from collections import OrderedDict


def miss_sequence(accesses, capacity: int) -> list:
    """True/False per access: did it miss in an LRU cache of ``capacity``?"""
    cache: OrderedDict = OrderedDict()
    out = []
    for a in accesses:
        if a in cache:
            cache.move_to_end(a)
            out.append(False)
        else:
            if len(cache) >= capacity:
                cache.popitem(last=False)
            cache[a] = True
            out.append(True)
    return out
