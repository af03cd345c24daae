"""Pins of the cross-step prefetch oracle (``oracle.prefetch``) -- CPU only.

The pages give prefetch's effect (HiSparse summary article, sections 03-04),
not its mechanism; ``oracle.prefetch`` states the reading.  These tests fix
it against things that do not depend on that code: an independent
brute-force scan replay, the closed form that an exact prediction with room
removes the next step's misses without changing that step's rows or the
state after it, and the guarantees a prefetch must keep for the step that
is still running (its selection is never evicted).
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle.bruteforce import replay_prefetch
from oracle.prefetch import prefetch
from oracle.resolve import ERR_DUP, ERR_RANGE, ERR_STEP, LruState, resolve
from tracegen.trace import selection_trace


def _bt(ctx, page, rng, frac):
    n = (ctx + page - 1) // page
    bt = np.full(n, -1, np.int64)
    if frac > 0:
        pick = rng.random(n) < frac
        bt[pick] = np.arange(int(pick.sum()))
    return bt


def _trace(seed, ctx, K, steps, retain):
    return selection_trace(seed, [ctx], K, steps, 1, retain, 0.8)[:, 0, 0]


@pytest.mark.parametrize("ctx,K,B", [(64, 4, 4), (64, 4, 6), (64, 8, 16), (200, 16, 24), (300, 16, 64)])
@pytest.mark.parametrize("resident", [0.0, 0.3])
def test_prefetch_matches_bruteforce(ctx, K, B, resident):
    """Against the brute-force scan replay, after every RESOLVE, with
    predictions that are exact, partly wrong, or the current selection."""
    for seed in range(12):
        rng = np.random.default_rng(seed)
        page = 4
        bt = _bt(ctx, page, rng, resident)
        tr = _trace(seed, ctx, K, 10, 0.6)
        st = LruState(B)
        for t in range(9):
            resolve(st, list(tr[t]), t, ctx, bt, page, 0)
            kind = seed % 3
            if kind == 0:
                pred = list(tr[t + 1])
            elif kind == 1:
                pred = list(tr[t + 1][: K // 2]) + [int(x) for x in rng.choice(ctx, K - K // 2, replace=False)]
                pred = list(dict.fromkeys(pred))
            else:
                pred = list(tr[t])
            rng.shuffle(pred)
            filled, owner, stamp = replay_prefetch(st.owner, st.stamp, pred, t, bt, page)
            res = prefetch(st, pred, t, ctx, bt, page)
            assert res.fetches == filled, (seed, t)
            assert st.owner == owner and st.stamp == stamp, (seed, t)
            assert res.errors == 0
            assert {p: s for s, p in enumerate(st.owner) if p >= 0} == st.slot_of


@pytest.mark.parametrize("retain", [0.0, 0.5, 0.85])
@pytest.mark.parametrize("resident", [0.0, 0.25])
def test_exact_prediction_removes_next_misses_and_keeps_the_path(retain, resident):
    """B = 2K leaves room for every miss of the next selection, so prefetching
    it exactly during step t gives step t+1 no miss, the same row ids and the
    same state as the path without prefetch, and the same host rows in total
    (each missing row is fetched once, one step earlier)."""
    ctx, K, page = 500, 32, 8
    for seed in range(6):
        rng = np.random.default_rng(50 + seed)
        bt = _bt(ctx, page, rng, resident)
        tr = _trace(100 + seed, ctx, K, 12, retain)
        a, b = LruState(2 * K), LruState(2 * K)
        fetched_a = fetched_b = 0
        for t in range(12):
            ra = resolve(a, list(tr[t]), t, ctx, bt, page, 1000)
            rb = resolve(b, list(tr[t]), t, ctx, bt, page, 1000)
            assert rb.rows == ra.rows, (seed, t)
            assert (b.owner, b.stamp) == (a.owner, a.stamp), (seed, t)
            assert rb.n_miss == (ra.n_miss if t == 0 else 0), (seed, t)
            fetched_a += ra.n_miss
            fetched_b += rb.n_miss
            if t + 1 < 12:
                pf = prefetch(b, list(tr[t + 1]), t, ctx, bt, page)
                assert pf.n_dropped == 0
                fetched_b += pf.n_filled
        assert fetched_a == fetched_b


def test_reusing_the_current_selection_fetches_nothing():
    """Speculation that the selection will not move (S' = S_t) finds every
    position resident or in the buffer: nothing is filled, nothing changes."""
    ctx, K, B, page = 400, 16, 40, 8
    rng = np.random.default_rng(3)
    bt = _bt(ctx, page, rng, 0.2)
    tr = _trace(7, ctx, K, 8, 0.5)
    st = LruState(B)
    for t in range(8):
        resolve(st, list(tr[t]), t, ctx, bt, page, 0)
        before = (list(st.owner), list(st.stamp))
        res = prefetch(st, list(tr[t]), t, ctx, bt, page)
        assert res.n_filled == 0 and res.n_dropped == 0 and res.fetches == []
        assert (st.owner, st.stamp) == before


def test_current_selection_is_never_evicted():
    """Whatever the prediction, the slots that step t's RESOLVE handed out
    keep their positions, so step t's attention reads the right rows."""
    ctx, K, B, page = 300, 16, 24, 4
    for seed in range(10):
        rng = np.random.default_rng(seed)
        bt = _bt(ctx, page, rng, 0.1)
        tr = _trace(seed, ctx, K, 6, 0.4)
        st = LruState(B)
        for t in range(6):
            res = resolve(st, list(tr[t]), t, ctx, bt, page, 10000)  # hot rows from 10000, resident below
            held = {r - 10000: st.owner[r - 10000] for r in res.rows if r >= 10000}
            assert len(held) == res.n_hit + res.n_miss
            pred = [int(x) for x in rng.choice(ctx, K, replace=False)]
            prefetch(st, pred, t, ctx, bt, page)
            for s, p in held.items():
                assert st.owner[s] == p


def test_full_buffer_drops_the_largest_positions():
    """B = K: after RESOLVE every slot belongs to the current selection, so a
    prefetch can fill nothing; with two free slots, the two smallest missing
    positions are the ones filled."""
    ctx, K, page = 100, 4, 4
    bt = np.full(25, -1)
    st = LruState(K)
    resolve(st, [10, 20, 30, 40], 0, ctx, bt, page, 0)
    res = prefetch(st, [50, 60, 70, 10], 0, ctx, bt, page)
    assert (res.n_hit, res.n_filled, res.n_dropped) == (1, 0, 3)
    st = LruState(K + 2)
    resolve(st, [10, 20, 30, 40], 0, ctx, bt, page, 0)
    res = prefetch(st, [70, 50, 60, 10], 0, ctx, bt, page)
    assert res.fetches == [(50, 4), (60, 5)] and res.n_dropped == 1
    assert st.stamp == [0] * 6


def test_worked_example():
    """Hand-worked: B = 6, no residency.  Step 0 resolves (5, 9, 2) into
    slots 0, 1, 2 (ascending fill: 2->0, 5->1, 9->2).  A prefetch during step
    0 of (9, 7, 1) pins slot 2 (hit), slots 0-2 are stamped 0 anyway, and
    fills 1 -> slot 3, 7 -> slot 4 with stamp 0.  Step 1 resolves (1, 7, 9)
    with no miss: rows slot 3, slot 4, slot 2, all stamped 1."""
    bt = np.full(4, -1)
    st = LruState(6)
    r0 = resolve(st, [5, 9, 2], 0, 16, bt, 4, 0)
    assert r0.rows == [1, 2, 0]
    pf = prefetch(st, [9, 7, 1], 0, 16, bt, 4)
    assert pf.fetches == [(1, 3), (7, 4)] and (pf.n_hit, pf.n_dropped) == (1, 0)
    assert st.owner == [2, 5, 9, 1, 7, -1] and st.stamp == [0, 0, 0, 0, 0, -1]
    r1 = resolve(st, [1, 7, 9], 1, 16, bt, 4, 0)
    assert r1.rows == [3, 4, 2] and (r1.n_hit, r1.n_miss) == (3, 0)
    assert st.stamp == [0, 0, 1, 1, 1, -1]


def test_errors():
    bt = np.full(4, -1)
    st = LruState(4)
    resolve(st, [1, 2], 3, 16, bt, 4, 0)
    res = prefetch(st, [3, 4], 2, 16, bt, 4)  # step going backwards
    assert res.errors == ERR_STEP and res.fetches == [] and st.owner == [1, 2, -1, -1]
    res = prefetch(st, [3, 3, 99, -1], 3, 16, bt, 4)
    assert res.errors == ERR_DUP | ERR_RANGE and res.fetches == [(3, 2)]
