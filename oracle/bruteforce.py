"""Brute-force replay of RESOLVE -- test infrastructure only (CPU oracle pin).

A second, deliberately naive rendering of the same rules as
``oracle.resolve`` (HiSparse summary article, section 02; vLLM Hybrid
HiSparse blog, "工作原理"), with no shared code: it keeps only the owner and
stamp arrays, finds a hit by scanning every slot, and picks each victim by a
full scan for the smallest (stamp, slot) among slots not yet used by this
call, one miss at a time in ascending position order.  Intended for tiny
traces, where it pins the state machine of ``oracle.resolve`` step by step.
"""

from __future__ import annotations


def replay(owner, stamp, sel, t, ctx, block_table, page_size, hot_base):
    """Return (rows, (n_res, n_hit, n_miss), new_owner, new_stamp).

    Inputs are not modified.  Assumes a valid call (t not decreasing,
    positions distinct and in range), which the caller guarantees.
    """
    owner = list(owner)
    stamp = list(stamp)
    B = len(owner)
    used = [False] * B
    rows = [-1] * len(sel)
    n_res = n_hit = 0
    pending = []
    for j, p in enumerate(sel):
        p = int(p)
        if p < 0:
            continue
        b = block_table[p // page_size]
        if b >= 0:
            rows[j] = int(b) * page_size + (p - (p // page_size) * page_size)
            n_res += 1
            continue
        found = -1
        for s in range(B):
            if owner[s] == p:
                found = s
        if found >= 0:
            stamp[found] = t
            used[found] = True
            rows[j] = hot_base + found
            n_hit += 1
        else:
            pending.append(j)
    pending.sort(key=lambda jj: int(sel[jj]))
    for j in pending:
        best = -1
        for s in range(B):
            if used[s]:
                continue
            if best < 0 or stamp[s] < stamp[best] or (stamp[s] == stamp[best] and s < best):
                best = s
        owner[best] = int(sel[j])
        stamp[best] = t
        used[best] = True
        rows[j] = hot_base + best
    return rows, (n_res, n_hit, len(pending)), owner, stamp


def replay_prefetch(owner, stamp, sel, t, block_table, page_size):
    """Brute-force prefetch (same reading as ``oracle.prefetch``): slots
    stamped t and slots holding a selected position are off limits; each
    missing position, smallest first, takes the slot of smallest (stamp,
    slot) among the rest, found by a full scan, until none is left.
    Returns (filled [(position, slot)], new_owner, new_stamp).  Assumes a
    valid call (distinct in-range positions, t not decreasing)."""
    owner = list(owner)
    stamp = list(stamp)
    B = len(owner)
    off = [stamp[s] == t for s in range(B)]
    missing = []
    for p in sel:
        p = int(p)
        if p < 0 or block_table[p // page_size] >= 0:
            continue
        hit = False
        for s in range(B):
            if owner[s] == p:
                off[s] = True
                hit = True
        if not hit:
            missing.append(p)
    filled = []
    for p in sorted(missing):
        best = -1
        for s in range(B):
            if off[s]:
                continue
            if best < 0 or stamp[s] < stamp[best] or (stamp[s] == stamp[best] and s < best):
                best = s
        if best < 0:
            break
        owner[best] = p
        stamp[best] = t
        off[best] = True
        filled.append((p, best))
    return filled, owner, stamp
