"""Cross-step prefetch of a predicted selection -- test infrastructure only
(CPU oracle).

The HiSparse summary article (sections 03 and 04) reports that precise
prefetch -- fetching the rows a coming step will select before that step
asks for them -- hides most of the host I/O that a synchronous RESOLVE
exposes, and that a selection the model provides beats speculation.  The
pages do not spell out the mechanism.  The plainest reading that keeps
RESOLVE's rules, used here:

* a prefetch is issued during step t with a predicted selection S' for a
  later step; it runs against the same per-(request, layer) state as
  RESOLVE and never returns row ids;
* it must not disturb step t: every slot already stamped t (the current
  selection, which step t's attention may still be reading, and anything an
  earlier prefetch of step t filled) is pinned, as is every slot that holds
  a position of S' (a hit: pinned, its stamp left alone, so a wrong guess
  does not refresh it);
* resident positions are skipped (they are read in place), repeats and
  out-of-range positions are errors treated as padding, as in RESOLVE;
* the positions of S' that are neither resident nor in the buffer are filled
  in ascending position order into the unpinned slots taken in RESOLVE's
  victim order (ascending (stamp, slot) under LRU and FIFO); when there are
  fewer such slots than misses, the largest positions are dropped (the coming
  step will miss them);
* a filled slot gets owner p and stamp t: the row is as recent as the step
  it was fetched in, so the coming step's RESOLVE finds it as a hit (and,
  under LRU, refreshes it) and a wrong guess ages like the rest of step t.

With the exact next selection and room for all of its misses, the next
step's RESOLVE then has no miss, and its rows and the state after it are
those of the path without prefetch: the victims are the same slots in the
same order, only fetched one step earlier (pinned in
``tests/test_oracle_prefetch.py``).
"""

from __future__ import annotations

from dataclasses import dataclass

from .resolve import ERR_DUP, ERR_RANGE, ERR_STEP


@dataclass
class PrefetchResult:
    n_resident: int
    n_hit: int
    n_filled: int
    n_dropped: int
    fetches: list  # [(position, slot)] in fill order
    errors: int


def prefetch(state, sel, t: int, ctx: int, block_table, page_size: int, policy: str = "lru",
             priority=None) -> PrefetchResult:
    """Prefetch the predicted selection ``sel`` (K positions, -1 = padding,
    any order) into one (request, layer)'s buffer during step t; mutates
    ``state`` (an ``oracle.resolve.LruState``)."""
    B = state.hot_slots
    if t < 0 or t < state.last_t:
        return PrefetchResult(0, 0, 0, 0, [], ERR_STEP)
    state.last_t = t
    errors = 0
    pinned = [state.stamp[s] == t for s in range(B)]
    seen = set()
    misses = []
    n_res = n_hit = 0
    for p in sel:
        p = int(p)
        if p == -1:
            continue
        if p < -1 or p >= ctx:
            errors |= ERR_RANGE
            continue
        if p in seen:
            errors |= ERR_DUP
            continue
        seen.add(p)
        if int(block_table[p // page_size]) >= 0:
            n_res += 1
        elif p in state.slot_of:
            pinned[state.slot_of[p]] = True
            n_hit += 1
        else:
            misses.append(p)
    misses.sort()
    free = [s for s in range(B) if not pinned[s]]
    if policy in ("lru", "fifo"):
        order = sorted((state.stamp[s], s) for s in free)
    elif policy == "random":
        order = sorted(((0, s) if state.owner[s] < 0 else (1 + priority(s), s)) for s in free)
    else:
        raise ValueError(f"prefetch does not support policy {policy}")
    victims = [o[-1] for o in order]
    n = min(len(misses), len(victims))
    fetches = []
    for p, v in zip(misses[:n], victims[:n]):
        old = state.owner[v]
        if old >= 0:
            del state.slot_of[old]
        state.owner[v] = p
        state.slot_of[p] = v
        state.stamp[v] = t
        fetches.append((p, v))
    return PrefetchResult(n_res, n_hit, n, len(misses) - n, fetches, errors)
