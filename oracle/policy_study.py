"""Miss rates of the four replacement policies against the hot-buffer size
-- test infrastructure only (CPU oracle).

The HiSparse summary article (section 04) reports, on real selection
traces, LRU at 13.4% misses against FIFO 17.2%, random 16.1% and the
offline optimum (Belady) 8.2% for B = 4096, and LRU at 6.7% for B = 8192.
Those traces are not available; this runs the same comparison on the
seeded synthetic traces (``tracegen``) of the 128K workload's shape and
prints a markdown table.  Miss rate = misses / selected non-resident
positions over steps 1.. (step 0 is cold).

    python -m oracle.policy_study [--steps 48] [--requests 4] [--retain 0.85]
"""

from __future__ import annotations

import argparse
import time

from tracegen import SelectionStream

from .policy import next_use_table, random_priority
from .resolve import LruState, resolve

POLICIES = ("lru", "fifo", "random", "belady")


def study(ctx=131072, k=2048, retain=0.85, alpha=0.8, steps=48, requests=4, buffers=(2048, 4096, 8192),
          seed=3, policy_seed=1):
    rows = {}
    for r in range(requests):
        s = SelectionStream(seed, 0, r, ctx, k, retain, alpha)
        sels = [s.next() for _ in range(steps)]
        nu = next_use_table(sels)
        for b in buffers:
            for pol in POLICIES:
                st = LruState(b)
                miss = sel_n = 0
                for t, sel in enumerate(sels):
                    res = resolve(st, sel, t, ctx, [-1] * (ctx // 64), 64, 0, policy=pol,
                                  priority=random_priority(policy_seed, t, 0, r),
                                  next_use=lambda q, t=t: nu(t, q))
                    if t >= 1:
                        miss += res.n_miss
                        sel_n += res.n_hit + res.n_miss
                m, n = rows.get((b, pol), (0, 0))
                rows[(b, pol)] = (m + miss, n + sel_n)
    return rows


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=48)
    ap.add_argument("--requests", type=int, default=4)
    ap.add_argument("--retain", type=float, default=0.85)
    args = ap.parse_args()
    t0 = time.time()
    rows = study(steps=args.steps, requests=args.requests, retain=args.retain)
    bufs = sorted({b for b, _ in rows})
    print(f"| B | " + " | ".join(POLICIES) + " |")
    print("|---|" + "---|" * len(POLICIES))
    for b in bufs:
        cells = []
        for pol in POLICIES:
            m, n = rows[(b, pol)]
            cells.append(f"{100.0 * m / n:.2f}%")
        print(f"| {b} | " + " | ".join(cells) + " |")
    print(f"\n({args.requests} requests x {args.steps} steps, ctx 131072, K 2048, retain {args.retain}, recency 0.8; "
          f"{time.time() - t0:.0f} s)")


if __name__ == "__main__":
    main()
