"""Exact step-LRU RESOLVE -- test infrastructure only (CPU oracle).

Follows the HiSparse summary article ("显存占用直降30倍！…HiSparse夯爆了"),
section 02, and the vLLM Hybrid HiSparse blog, section "工作原理":

* per (request, layer) a device buffer of B slots caches KV rows; a page
  table maps each logical position to a slot or to "host only"; LRU
  metadata chooses what to replace;
* one RESOLVE per sparse layer does hit detection, LRU replacement,
  metadata update and the fetch of every miss from pinned host memory;
* with mixed residency, a token on a GPU-resident page is read in place
  (the block table entry names its block, the LRU state is untouched), a
  token already in the hot buffer is read there and its LRU entry
  refreshed, and a miss copies one row from host memory into an LRU slot.

Readings where the pages are silent (each also listed in the design notes):

* every slot starts empty: owner -1, stamp -1;
* the LRU clock is the caller's step index t; every slot touched by a call
  gets stamp t, so ties within one step are broken by slot index;
* "the current selection is pinned": a slot hit by this call, or filled by
  this call, cannot be chosen as a victim in the same call;
* the victims are the unpinned slots with the smallest (stamp, slot); the
  i-th smallest missing position goes to the i-th victim;
* residency is checked before the hot buffer; a resident token counts as
  resident, never as a hit;
* -1 in the selection is padding; a position outside [0, ctx) or a repeat of
  an earlier entry of the same list is a caller error: it is reported and
  treated as padding (the earliest occurrence of a repeated position is the
  one kept);
* t must be >= 0 and not below the last t seen by this (request, layer);
  otherwise the call is an error and resolves nothing (all rows -1, state
  unchanged);
* B < K is rejected.
"""

from __future__ import annotations

from dataclasses import dataclass, field

ERR_RANGE = 1  # a position outside [-1, ctx)
ERR_DUP = 2  # a position repeated within one selection
ERR_STEP = 4  # t negative or below the previous t


@dataclass
class LruState:
    """RESOLVE state of one (request, layer)."""

    hot_slots: int
    owner: list = field(default_factory=list)  # slot -> logical position, -1 = empty
    stamp: list = field(default_factory=list)  # slot -> step of last use, -1 = never
    slot_of: dict = field(default_factory=dict)  # logical position -> slot (inverse of owner)
    last_t: int = -1

    def __post_init__(self):
        if not self.owner:
            self.owner = [-1] * self.hot_slots
            self.stamp = [-1] * self.hot_slots


@dataclass
class ResolveResult:
    rows: list  # per input entry: KV row id, or -1
    n_resident: int
    n_hit: int
    n_miss: int
    fetches: list  # [(position, slot)] in fill order
    errors: int


def resolve(state: LruState, sel, t: int, ctx: int, block_table, page_size: int,
            hot_base: int, policy: str = "lru", priority=None, next_use=None) -> ResolveResult:
    """One RESOLVE call for one (request, layer); mutates ``state``.

    ``sel``: the K selected logical positions (-1 = padding), in the
    indexer's order.  ``block_table[page]``: block id of a GPU-resident page,
    or -1 for a page that lives only on the host.  Resident row ids are
    ``block * page_size + offset``; hot row ids are ``hot_base + slot``.

    ``policy`` picks the victim order (``oracle.policy``): "lru" (default),
    "fifo", "random" (``priority(slot)`` gives this call's priorities) or
    "belady" (``next_use(p)`` gives the next step that selects p).  Stamps
    hold the step of last use, except under FIFO the step of the fill.
    """
    B = state.hot_slots
    K = len(sel)
    if B < K:
        raise ValueError("hot_slots must be >= top_k")
    if t < 0 or t < state.last_t:
        return ResolveResult([-1] * K, 0, 0, 0, [], ERR_STEP)
    state.last_t = t

    errors = 0
    rows = [-1] * K
    pinned = [False] * B
    seen = set()
    misses = []  # (position, input index)
    n_res = n_hit = 0

    # Classify every entry in input order.
    for j in range(K):
        p = int(sel[j])
        if p == -1:
            continue
        if p < -1 or p >= ctx:
            errors |= ERR_RANGE
            continue
        if p in seen:
            errors |= ERR_DUP
            continue
        seen.add(p)
        blk = int(block_table[p // page_size])
        if blk >= 0:
            rows[j] = blk * page_size + p % page_size
            n_res += 1
        elif p in state.slot_of:
            s = state.slot_of[p]
            if policy != "fifo":
                state.stamp[s] = t
            pinned[s] = True
            rows[j] = hot_base + s
            n_hit += 1
        else:
            misses.append((p, j))

    # Misses are filled in ascending logical order; victims are the unpinned
    # slots in ascending (stamp, slot) order.
    misses.sort()
    free = [s for s in range(B) if not pinned[s]]
    if policy in ("lru", "fifo"):
        candidates = sorted((state.stamp[s], s) for s in free)
    elif policy == "random":
        candidates = sorted(((0, s) if state.owner[s] < 0 else (1 + priority(s), s)) for s in free)
    elif policy == "belady":
        candidates = sorted(((0, 0.0, s) if state.owner[s] < 0 else (1, -next_use(state.owner[s]), s))
                            for s in free)
    else:
        raise ValueError(f"unknown policy {policy}")
    victims = [c[-1] for c in candidates[: len(misses)]]
    fetches = []
    for (p, j), v in zip(misses, victims):
        old = state.owner[v]
        if old >= 0:
            del state.slot_of[old]
        state.owner[v] = p
        state.slot_of[p] = v
        state.stamp[v] = t
        pinned[v] = True
        rows[j] = hot_base + v
        fetches.append((p, v))
    return ResolveResult(rows, n_res, n_hit, len(misses), fetches, errors)
