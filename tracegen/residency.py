"""Block-table schedule of growing contexts (input generation only).

A serving engine decides which pages of a request keep a GPU block; the
decode path only follows the block table.  This module fixes one such
engine policy, deterministically, so that a device run and the CPU oracle
see the same residency over a trace in which every request appends one
token per step (vLLM Hybrid HiSparse blog, section "工作原理": the tail
page stays on the GPU, older pages become host-only placeholders once
their copy in host memory exists):

* before the append of step t (position ctx0_r + t), if that position starts
  a new page, the page leases the smallest free block;
* after step t's write-back, the host pool holds every position below
  ``held = max(ctx0_r, floor((ctx0_r + t + 1) / page) * page)``; the oldest
  resident pages beyond the newest ``keep`` are dropped if they end at or
  below ``held``, and their blocks return to the free list.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class Schedule:
    page_size: int
    ctx0: list
    capacity: list
    initial_bt: list                       # [R] block table at creation (capacity pages each)
    pre: list = field(default_factory=list)   # [steps] list of (r, page, block) before the append
    post: list = field(default_factory=list)  # [steps] list of (r, page, -1) after the write-back
    bt_at: list = field(default_factory=list)  # [steps][R] block table in force during step t

    def ctx_at(self, t: int, r: int) -> int:
        """Context length during step t (after its append)."""
        return self.ctx0[r] + t + 1


def growing_schedule(ctx0, steps: int, page_size: int, total_blocks: int, keep: int = 2) -> Schedule:
    """Initial residency: the page of position ctx0_r (the next append's
    page) holds a block, request r taking block r; blocks R.. are free."""
    R = len(ctx0)
    cap = [c + steps for c in ctx0]
    if total_blocks < R:
        raise ValueError("need at least one block per request")
    bt = []
    for r in range(R):
        pages = -(-cap[r] // page_size)
        row = [-1] * pages
        row[ctx0[r] // page_size] = r
        bt.append(row)
    sch = Schedule(page_size, list(ctx0), cap, [list(b) for b in bt])
    free = list(range(R, total_blocks))
    for t in range(steps):
        pre = []
        for r in range(R):
            pos = ctx0[r] + t
            pg = pos // page_size
            if bt[r][pg] < 0:
                if not free:
                    raise ValueError("block pool exhausted")
                blk = free.pop(0)
                bt[r][pg] = blk
                pre.append((r, pg, blk))
        sch.pre.append(pre)
        sch.bt_at.append([list(b) for b in bt])
        post = []
        for r in range(R):
            held = max(ctx0[r], ((ctx0[r] + t + 1) // page_size) * page_size)
            resident = [pg for pg, b in enumerate(bt[r]) if b >= 0]
            for pg in resident[:-keep] if len(resident) > keep else []:
                if (pg + 1) * page_size <= held:
                    free.append(bt[r][pg])
                    bt[r][pg] = -1
                    post.append((r, pg, -1))
        free.sort()
        sch.post.append(post)
    return sch
