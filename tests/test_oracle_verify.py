"""Pins of the multi-token verification RESOLVE (CPU only).

* T = 1 is the single-token RESOLVE.
* T identical selections give, per token, the single-token rows.
* Against a brute-force replay of the distinct positions (the union), built
  with plain sets and the per-miss scan replay: rows of every entry, counts
  and the full state, step by step, on overlapping multi-token traces with
  residency, padding and repeats inside one token's list.
* With B = T x K and disjoint, never-seen selections every slot is filled.
"""

import numpy as np
import pytest

from oracle.bruteforce import replay
from oracle.resolve import ERR_DUP, LruState, resolve
from oracle.verify import resolve_verify


def _trace(rng, ctx, K, T, steps):
    """Token selections that overlap (each token keeps ~60% of the previous)."""
    out = []
    prev = rng.choice(ctx, K, replace=False)
    for _ in range(steps):
        toks = []
        for _ in range(T):
            keep = prev[rng.random(K) < 0.6]
            pool = np.setdiff1d(np.arange(ctx), keep)
            new = rng.choice(pool, K - keep.shape[0], replace=False)
            cur = rng.permutation(np.concatenate([keep, new]))
            toks.append(cur)
            prev = cur
        out.append(toks)
    return out


def test_single_token_is_resolve():
    rng = np.random.default_rng(1)
    bt = [-1] * 20
    s1, s2 = LruState(48), LruState(48)
    for t, toks in enumerate(_trace(rng, 300, 16, 1, 30)):
        a = resolve_verify(s1, toks, t, 300, bt, 16, 7)
        b = resolve(s2, toks[0], t, 300, bt, 16, 7)
        assert a.rows == b.rows and (a.n_resident, a.n_hit, a.n_miss) == (b.n_resident, b.n_hit, b.n_miss)
        assert s1.owner == s2.owner and s1.stamp == s2.stamp


def test_identical_tokens_share_rows():
    rng = np.random.default_rng(2)
    bt = [-1] * 20
    s1, s2 = LruState(64), LruState(64)
    for t, toks in enumerate(_trace(rng, 300, 16, 1, 20)):
        a = resolve_verify(s1, [toks[0]] * 4, t, 300, bt, 16, 0)
        b = resolve(s2, toks[0], t, 300, bt, 16, 0)
        assert a.rows == b.rows * 4
        assert (a.n_resident, a.n_hit, a.n_miss) == (b.n_resident, b.n_hit, b.n_miss)
        assert s1.owner == s2.owner


@pytest.mark.parametrize("T,K,extra", [(2, 8, 0), (3, 8, 5), (4, 6, 13), (2, 32, 30)])
def test_against_union_bruteforce(T, K, extra):
    rng = np.random.default_rng(10 * T + K)
    ctx, page = 400, 16
    B = T * K + extra
    bt = [-1] * (ctx // page)
    for pg in rng.choice(ctx // page, 5, replace=False):
        bt[pg] = int(rng.integers(0, 50))
    st = LruState(B)
    owner, stamp = [-1] * B, [-1] * B
    for t, toks in enumerate(_trace(rng, ctx, K, T, 25)):
        toks = [np.array(x) for x in toks]
        if t % 3 == 1:
            toks[0][rng.random(K) < 0.2] = -1  # padding
        dup_tok = None
        if t % 4 == 2 and K > 2:
            dup_tok = T - 1
            toks[dup_tok][1] = toks[dup_tok][0]  # a repeat inside one token's list
        res = resolve_verify(st, toks, t, ctx, bt, page, 1000)
        # brute force on the union, then each entry takes its position's row
        union = sorted({int(p) for x in toks for p in x if p >= 0})
        rows_u, counts_u, owner, stamp = replay(owner, stamp, union, t, ctx, bt, page, 1000)
        row_of = dict(zip(union, rows_u))
        want = []
        for b, x in enumerate(toks):
            seen = set()
            for p in x:
                p = int(p)
                if p < 0 or p in seen:
                    want.append(-1)
                else:
                    want.append(row_of[p])
                    seen.add(p)
        assert res.rows == want, t
        assert (res.n_resident, res.n_hit, res.n_miss) == counts_u
        assert st.owner == owner and st.stamp == stamp
        assert bool(res.errors & ERR_DUP) == (dup_tok is not None)


def test_full_buffer_when_disjoint():
    T, K = 3, 10
    st = LruState(T * K)
    toks = [list(range(b * K, (b + 1) * K)) for b in range(T)]
    res = resolve_verify(st, toks, 0, 100, [-1] * 10, 16, 0)
    assert res.n_miss == T * K and sorted(st.owner) == list(range(T * K))
    assert sorted(res.rows) == list(range(T * K))
    with pytest.raises(ValueError):
        resolve_verify(LruState(T * K - 1), toks, 0, 100, [-1] * 10, 16, 0)
