"""Replacement policies other than LRU -- test infrastructure only (CPU
oracle).

The HiSparse summary article (section 04) compares LRU with FIFO, random
replacement and the offline optimum (Belady) on the same selection traces.
All four share the rules of ``oracle.resolve``: residency first, the current
selection pinned, the i-th smallest missing position filling the i-th
victim; they differ in the order victims are taken from the unpinned slots:

* LRU: ascending (step of last use, slot);
* FIFO: ascending (step of the fill, slot) -- a hit does not refresh;
* random: empty slots first (by slot), then ascending (priority, slot) with
  a 31-bit priority drawn per call from SplitMix64 (Steele, Lea, Flood,
  "Fast splittable pseudorandom number generators", OOPSLA 2014):
  ``k = sm(sm(sm(seed) ^ t) ^ (l << 32 | r))``, priority of slot s =
  ``sm(k ^ s) >> 33``, where ``sm(x)`` is the generator's output for state
  x (add the golden gamma 0x9E3779B97F4A7C15, then the mixing function);
* Belady: empty slots first (by slot), then the slot whose position is
  next selected furthest in the future (never again first), ties by slot.
  It needs the future selections, so it exists only here.
"""

from __future__ import annotations

MASK64 = (1 << 64) - 1
GAMMA = 0x9E3779B97F4A7C15


def splitmix64(x: int) -> int:
    z = (x + GAMMA) & MASK64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & MASK64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & MASK64
    return z ^ (z >> 31)


def random_priority(seed: int, t: int, l: int, r: int):
    """Slot -> 31-bit priority of the random policy for one call."""
    k = splitmix64(splitmix64(splitmix64(seed & MASK64) ^ (t & MASK64)) ^ (((l & 0xFFFFFFFF) << 32) | (r & 0xFFFFFFFF)))
    return lambda s: splitmix64(k ^ s) >> 33


def next_use_table(selections):
    """selections: list over steps of iterables of positions (one request,
    one layer group).  Returns f(t, p) = the first step > t that selects p,
    or infinity."""
    occ = {}
    for t, sel in enumerate(selections):
        for p in sel:
            p = int(p)
            if p >= 0:
                occ.setdefault(p, []).append(t)
    import bisect

    def f(t: int, p: int) -> float:
        lst = occ.get(p)
        if not lst:
            return float("inf")
        i = bisect.bisect_right(lst, t)
        return lst[i] if i < len(lst) else float("inf")

    return f
