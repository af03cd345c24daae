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


def fifo_miss_sequence(accesses, capacity: int) -> list:
    """True/False per access in a first-in-first-out cache: a hit leaves the
    queue unchanged; a miss on a full cache evicts the oldest insertion."""
    from collections import deque

    queue, present, out = deque(), set(), []
    for a in accesses:
        if a in present:
            out.append(False)
            continue
        if len(queue) >= capacity:
            present.discard(queue.popleft())
        queue.append(a)
        present.add(a)
        out.append(True)
    return out


def min_miss_sequence(accesses, capacity: int) -> list:
    """True/False per access in Belady's MIN cache (L. A. Belady, "A study of
    replacement algorithms for a virtual-storage computer", IBM Systems
    Journal 5(2), 1966): on a miss with a full cache, evict the resident
    item whose next access is furthest away (never again counts as
    furthest).  Quadratic look-ahead; tiny streams only."""
    cache, out = [], []
    for i, a in enumerate(accesses):
        if a in cache:
            out.append(False)
            continue
        if len(cache) >= capacity:
            def next_access(x):
                for k in range(i + 1, len(accesses)):
                    if accesses[k] == x:
                        return k
                return float("inf")
            dist = [next_access(x) for x in cache]
            far = max(range(len(cache)), key=lambda k: (dist[k], -k))
            cache.pop(far)
        cache.append(a)
        out.append(True)
    return out
