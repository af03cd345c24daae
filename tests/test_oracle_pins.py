"""Pins of the CPU oracle against facts fixed outside the oracle itself.

Each test fixes a part of the oracle with something other than its own
code: a hand-worked example, an independent brute-force replay, the
textbook LRU cache, closed forms that the pages' statements imply, and
special cases of softmax attention with known answers.
"""

import json
import math
import os

import numpy as np
import pytest

from oracle import bruteforce, footprint, textbook
from oracle.attention import attend, bf16_bits_to_f64
from oracle.resolve import ERR_DUP, ERR_RANGE, ERR_STEP, LruState, resolve
from oracle.step import OracleDecoder, SimulatedKV
from tracegen import make_workload
from tracegen.values import f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# --------------------------------------------------------------------------
# P1: the hand-worked examples (tie-break, fill order, resident precedence)
# --------------------------------------------------------------------------
def test_worked_examples():
    with open(os.path.join(GOLDEN, "lru_worked_example.json")) as f:
        ex = json.load(f)
    for e in ex["examples"]:
        st = LruState(e["hot_slots"])
        for s in e["steps"]:
            res = resolve(st, s["sel"], s["t"], e["ctx"], e["block_table"], e["page_size"], e["hot_base"])
            want_rows = [
                (e["hot_base"] + sl) if sl is not None else rr
                for sl, rr in zip(s["slots"], s["resident_rows"])
            ]
            assert res.rows == want_rows, (e["name"], s["t"])
            assert st.owner == s["owner"], (e["name"], s["t"])
            assert st.stamp == s["stamp"], (e["name"], s["t"])
            assert [res.n_resident, res.n_hit, res.n_miss] == s["counts"]
            assert res.errors == 0


# --------------------------------------------------------------------------
# P2: brute-force replay on many tiny traces
# --------------------------------------------------------------------------
def _tiny_trace(rng, ctx, k, steps, retain):
    sel = rng.choice(ctx, size=k, replace=False)
    out = []
    for _ in range(steps):
        out.append(list(rng.permutation(sel)))  # unsorted input order on purpose
        keep = rng.choice(sel, size=int(round(retain * k)), replace=False)
        rest = np.setdiff1d(np.arange(ctx), keep)
        sel = np.concatenate([keep, rng.choice(rest, size=k - len(keep), replace=False)])
    return out


@pytest.mark.parametrize("ctx,k,b", [(64, 4, 4), (64, 4, 5), (64, 4, 8), (64, 8, 64), (200, 16, 32)])
@pytest.mark.parametrize("retain", [0.0, 0.5, 0.7, 1.0])
@pytest.mark.parametrize("resident", [False, True])
def test_bruteforce_replay(ctx, k, b, retain, resident):
    page = 8
    for seed in range(20):
        rng = np.random.default_rng(1000 * seed + 7)
        npages = -(-ctx // page)
        bt = [-1] * npages
        if resident:
            for i, pg in enumerate(rng.choice(npages, size=npages // 3, replace=False)):
                bt[int(pg)] = i
        hot_base = 1000
        st = LruState(b)
        owner, stamp = [-1] * b, [-1] * b
        t = 0
        for sel in _tiny_trace(rng, ctx, k, 12, retain):
            t += int(rng.integers(0, 2))  # equal consecutive t is allowed
            res = resolve(st, sel, t, ctx, bt, page, hot_base)
            rows, counts, owner, stamp = bruteforce.replay(owner, stamp, sel, t, ctx, bt, page, hot_base)
            assert res.rows == rows
            assert (res.n_resident, res.n_hit, res.n_miss) == counts
            assert st.owner == owner and st.stamp == stamp


# --------------------------------------------------------------------------
# P3: K = 1 reduces to the textbook LRU cache
# --------------------------------------------------------------------------
@pytest.mark.parametrize("b", [1, 2, 3, 7, 16])
def test_k1_is_textbook_lru(b):
    rng = np.random.default_rng(b)
    acc = [int(x) for x in rng.integers(0, 24, size=400)]
    want = textbook.miss_sequence(acc, b)
    st = LruState(b)
    got = []
    for t, p in enumerate(acc):
        res = resolve(st, [p], t, 24, [-1] * 3, 8, 0)
        got.append(res.n_miss == 1)
    assert got == want


# --------------------------------------------------------------------------
# P4: B = K closed form (the summary article, section 02: with B = k the
# buffer can only hold the previous selection, so what misses is exactly the
# drifted part of the new selection)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("resident", [False, True])
def test_b_equals_k_closed_form(resident):
    w = make_workload("bk", 11, 2, 1, 1, [3000, 1700], 4, 64, 64, 20, 0.6, 0.8,
                      "tail+half" if resident else "none", page_size=16)
    tr = w.trace()
    dec = OracleDecoder(w)
    prev = [set(), set()]
    for t in range(w.steps):
        res = dec.resolve_step(t, tr[t])
        for r in range(2):
            bt = w.block_tables[r]
            cur = {int(p) for p in tr[t][0][r] if p >= 0 and bt[int(p) // w.page_size] < 0}
            if resident:
                # fewer than B host-only picks per step: the buffer also keeps
                # older rows, so the drifted part only bounds the misses
                assert res[(0, r)].n_miss <= len(cur - prev[r])
            else:
                assert res[(0, r)].n_miss == len(cur - prev[r])
            prev[r] = cur


# --------------------------------------------------------------------------
# P5: B >= number of host-only positions => a miss only on first touch
# --------------------------------------------------------------------------
def test_large_buffer_misses_only_first_touch():
    w = make_workload("big", 1, 1, 1, 1, [4096], 16, 256, 4096, 40, 0.7, 0.8, "none")
    tr = w.trace()
    dec = OracleDecoder(w)
    seen = set()
    for t in range(w.steps):
        res = dec.resolve_step(t, tr[t])[(0, 0)]
        cur = {int(p) for p in tr[t][0][0] if p >= 0}
        assert res.n_miss == len(cur - seen)
        seen |= cur
    # once every selected position has been seen, nothing misses
    st = dec.states[(0, 0)]
    again = resolve(st, tr[5][0][0], w.steps, 4096, w.block_tables[0], 64, 0)
    assert again.n_miss == 0


# --------------------------------------------------------------------------
# P6: full residency (the vLLM blog, "工作原理": resident pages are read in
# place) => no hit, no miss, state untouched, in-place row ids
# --------------------------------------------------------------------------
def test_full_residency():
    ctx, page, b = 300, 16, 64
    npages = -(-ctx // page)
    bt = list(np.random.default_rng(3).permutation(npages))
    st = LruState(b)
    rng = np.random.default_rng(4)
    for t in range(10):
        sel = rng.choice(ctx, size=32, replace=False)
        res = resolve(st, list(sel), t, ctx, bt, page, 10_000)
        assert res.n_hit == 0 and res.n_miss == 0 and res.n_resident == 32
        assert res.rows == [int(bt[p // page]) * page + p % page for p in sel]
        assert st.owner == [-1] * b and st.stamp == [-1] * b


# --------------------------------------------------------------------------
# P7: retain = 1 => after step 0 nothing misses
# --------------------------------------------------------------------------
def test_retain_one():
    w = make_workload("r1", 9, 2, 1, 1, [5000, 5000], 4, 128, 256, 10, 1.0, 0.8, "tail")
    tr = w.trace()
    dec = OracleDecoder(w)
    for t in range(w.steps):
        res = dec.resolve_step(t, tr[t])
        for r in range(2):
            if t > 0:
                assert res[(0, r)].n_miss == 0
                assert (tr[t][0][r] == tr[0][0][r]).all()


# --------------------------------------------------------------------------
# P8: invariants after every step
# --------------------------------------------------------------------------
def test_invariants_every_step():
    w = make_workload("inv", 21, 3, 2, 2, [900, 2000, 517], 4, 96, 160, 25, 0.7, 0.8, "tail+half", page_size=32)
    tr = w.trace()
    dec = OracleDecoder(w)
    kv = SimulatedKV(w)
    for t in range(w.steps):
        res = dec.resolve_step(t, tr[t])
        for (l, r), rr in res.items():
            kv.apply_fetches(l, r, rr.fetches, dec.hot_base(r))
            st = dec.states[(l, r)]
            assert {p: s for s, p in enumerate(st.owner) if p >= 0} == st.slot_of
            assert sum(1 for p in st.owner if p >= 0) <= w.hot_slots
            assert max(st.stamp) <= t
            bt = w.block_tables[r]
            for p in tr[t][l // w.index_share][r]:
                if p >= 0 and bt[p // w.page_size] < 0:
                    s = st.slot_of[int(p)]
                    assert st.stamp[s] == t
            # hot rows hold exactly the host rows of their owners
            from tracegen import kv_rows
            owned = [(s, p) for s, p in enumerate(st.owner) if p >= 0]
            host = kv_rows(w.seed, r, l, [p for _, p in owned])
            for i, (s, _) in enumerate(owned):
                assert (kv.rows[(l, dec.hot_base(r) + s)] == host[i]).all()


# --------------------------------------------------------------------------
# Error handling readings
# --------------------------------------------------------------------------
def test_error_paths():
    st = LruState(8)
    res = resolve(st, [3, 99, 3, -1, -5], 0, 50, [-1] * 7, 8, 0)
    assert res.errors == ERR_RANGE | ERR_DUP
    assert res.rows[1] == -1 and res.rows[2] == -1 and res.rows[3] == -1 and res.rows[4] == -1
    assert res.rows[0] >= 0 and res.n_miss == 1
    res = resolve(st, [4], 5, 50, [-1] * 7, 8, 0)
    assert res.errors == 0
    before = (list(st.owner), list(st.stamp))
    res = resolve(st, [6], 4, 50, [-1] * 7, 8, 0)
    assert res.errors == ERR_STEP and res.rows == [-1]
    assert (st.owner, st.stamp) == before
    with pytest.raises(ValueError):
        resolve(LruState(2), [1, 2, 3], 0, 50, [-1] * 7, 8, 0)


# --------------------------------------------------------------------------
# P9: exactness (summary article, section 02): attending through the
# resolved row ids equals attending by logical index, bit for bit
# --------------------------------------------------------------------------
def test_exactness_through_rows():
    w = make_workload("ex", 5, 2, 1, 1, [700, 1500], 8, 64, 96, 8, 0.6, 0.8, "tail+half", page_size=16)
    tr = w.trace()
    dec = OracleDecoder(w)
    kv = SimulatedKV(w)
    for t in range(w.steps):
        res, att = dec.step(t, tr[t])
        for (l, r), rr in res.items():
            kv.apply_fetches(l, r, rr.fetches, dec.hot_base(r))
            from tracegen import q_block
            q = q_block(w.seed, t, l, r, w.num_heads)
            o2, lse2 = attend(q, kv.gather(l, rr.rows), w.scale)
            o1, lse1 = att[(l, r)]
            assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)


# --------------------------------------------------------------------------
# P10: attention special cases with known answers
# --------------------------------------------------------------------------
def _bf(x):
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


def test_attention_single_row():
    rng = np.random.default_rng(0)
    q = _bf(rng.standard_normal((4, 576)))
    x = _bf(rng.standard_normal((1, 576)))
    o, lse = attend(q, x, 0.05)
    xf = bf16_bits_to_f64(x)
    assert np.array_equal(o, np.broadcast_to(xf[0, :512], (4, 512)))
    s = 0.05 * (bf16_bits_to_f64(q) @ xf[0])
    assert np.allclose(lse, s, rtol=0, atol=1e-12)


def test_attention_two_rows_closed_form():
    rng = np.random.default_rng(1)
    q = _bf(rng.standard_normal((3, 576)))
    x = _bf(rng.standard_normal((2, 576)))
    o, lse = attend(q, x, 1 / 24)
    qf, xf = bf16_bits_to_f64(q), bf16_bits_to_f64(x)
    for h in range(3):
        s0 = sum(qf[h, d] * xf[0, d] for d in range(576)) / 24
        s1 = sum(qf[h, d] * xf[1, d] for d in range(576)) / 24
        w0 = 1.0 / (1.0 + math.exp(s1 - s0))
        want = w0 * xf[0, :512] + (1 - w0) * xf[1, :512]
        assert np.allclose(o[h], want, rtol=0, atol=1e-12)
        assert abs(lse[h] - (max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))))) < 1e-12


def test_attention_uniform_and_rope_and_permutation():
    rng = np.random.default_rng(2)
    q = _bf(rng.standard_normal((2, 576)))
    x = _bf(rng.standard_normal((37, 576)))
    # scale 0: uniform weights, O = mean of the value rows, lse = ln n
    o, lse = attend(q, x, 0.0)
    assert np.allclose(o, bf16_bits_to_f64(x)[:, :512].mean(0), rtol=0, atol=1e-12)
    assert np.allclose(lse, math.log(37), rtol=0, atol=1e-12)
    # identical keys: uniform weights whatever the scale
    xi = np.repeat(x[:1], 5, axis=0)
    o, _ = attend(q, xi, 0.3)
    assert np.allclose(o, bf16_bits_to_f64(xi)[0, :512], rtol=0, atol=1e-12)
    # the rope dims (512..575) enter the scores but not the values
    xr = np.zeros((2, 576), np.uint16)
    xr[0, 512:] = _bf(np.ones(64))
    qr = np.zeros((1, 576), np.uint16)
    qr[0, 512:] = _bf(np.ones(64))
    o, lse = attend(qr, xr, 1.0)
    assert np.all(o == 0)  # value dims are all zero
    assert abs(lse[0] - (64 + math.log1p(math.exp(-64)))) < 1e-12
    # permuting the selection leaves the output unchanged
    perm = rng.permutation(37)
    o1, l1 = attend(q, x, 0.1)
    o2, l2 = attend(q, x[perm], 0.1)
    assert np.allclose(o1, o2, rtol=0, atol=1e-13) and np.allclose(l1, l2, rtol=0, atol=1e-13)


def test_attention_empty():
    q = _bf(np.ones((3, 576)))
    o, lse = attend(q, np.zeros((0, 576), np.uint16), 1.0)
    assert np.all(o == 0) and np.all(np.isneginf(lse))


# --------------------------------------------------------------------------
# P11: footprint closed form against the pages' printed numbers
# --------------------------------------------------------------------------
def test_footprint_pages_numbers():
    with open(os.path.join(GOLDEN, "footprint_pages.json")) as f:
        g = json.load(f)
    ratio = footprint.reduction(g["ctx"], g["hot_slots"])
    assert ratio == 32.0
    assert abs(ratio - g["reduction_approx"]) / g["reduction_approx"] < 0.1
    hot_gb = g["full_kv_gb"] / ratio
    assert abs(hot_gb - g["hisparse_kv_gb_approx"]) < 0.05
    assert footprint.hot_buffer_bytes(4096, 4, 1152) * 32 == footprint.full_kv_bytes(131072, 4, 1152)


# --------------------------------------------------------------------------
# P12: growing contexts and block-table transitions (vLLM Hybrid HiSparse
# blog, "工作原理": the tail page stays resident, completed pages become
# host-only once their host copy exists).  The oracle must agree with the
# brute-force replay under a changing block table and context length, every
# miss must be for a position the host pool already holds, and reading the
# rows the oracle names -- with appends written to the tail block and
# fetches to hot rows -- must return exactly the selected positions.
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(8))
def test_growth_transitions(seed):
    from tracegen.residency import growing_schedule

    rng = np.random.default_rng(5000 + seed)
    page, R, steps, k, b = 8, 3, 48, 6, 10
    ctx0 = [int(rng.integers(12, 70)) for _ in range(R)]
    sch = growing_schedule(ctx0, steps, page, total_blocks=4 * R, keep=2)
    hot_base = 10_000
    st = {r: LruState(b) for r in range(R)}
    bf = {r: ([-1] * b, [-1] * b) for r in range(R)}
    # device rows as labels (request, position); resident pages present at creation hold their rows
    dev = {}
    for r in range(R):
        for pg, blk in enumerate(sch.initial_bt[r]):
            if blk >= 0:
                for off in range(page):
                    if pg * page + off < ctx0[r]:
                        dev[blk * page + off] = (r, pg * page + off)
    drops_seen = 0
    for t in range(steps):
        for r in range(R):
            pos = ctx0[r] + t  # this step's append
            bt = sch.bt_at[t][r]
            blk = bt[pos // page]
            assert blk >= 0, "the schedule leases the tail page before the append"
            dev[blk * page + pos % page] = (r, pos)
            ctx = sch.ctx_at(t, r)
            held = max(ctx0[r], ((ctx0[r] + t) // page) * page)  # after the previous step's write-back
            sel = list(rng.choice(ctx, size=k, replace=False))
            if rng.random() < 0.7 and ctx - 1 not in sel:
                sel[0] = ctx - 1
            res = resolve(st[r], sel, t, ctx, bt, page, hot_base + 100 * r)
            rows, counts, o, s = bruteforce.replay(*bf[r], sel, t, ctx, bt, page, hot_base + 100 * r)
            assert res.rows == rows, f"seed {seed} t {t} r {r}"
            assert (res.n_resident, res.n_hit, res.n_miss) == counts
            assert st[r].owner == o and st[r].stamp == s
            bf[r] = (o, s)
            for p, slot in res.fetches:
                assert p < held, f"miss of position {p} the host pool does not hold yet (held {held})"
                dev[hot_base + 100 * r + slot] = (r, p)
            got = [dev[row] for row in res.rows if row >= 0]
            assert got == [(r, int(p)) for p in sel if p >= 0]
        drops_seen += len(sch.post[t])
    assert drops_seen > 0, "the trace exercises pages turning into placeholders"


# --------------------------------------------------------------------------
# P13: replacement policies of the HiSparse summary article's comparison
# (section 04: LRU vs FIFO, random and Belady).
# --------------------------------------------------------------------------
def test_splitmix64_published_outputs():
    from oracle.policy import GAMMA, MASK64, splitmix64

    # first outputs of SplitMix64 from state 0 (reference implementation)
    state, out = 0, []
    for _ in range(3):
        out.append(splitmix64(state))
        state = (state + GAMMA) & MASK64
    assert out == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]


def _k1_policy_misses(stream, b, policy, seed=3):
    from oracle.policy import next_use_table, random_priority

    st = LruState(b)
    nu = next_use_table([[p] for p in stream])
    out = []
    for t, p in enumerate(stream):
        res = resolve(st, [p], t, 10_000, [-1] * 200, 64, 0, policy=policy,
                      priority=random_priority(seed, t, 0, 0), next_use=lambda q, t=t: nu(t, q))
        out.append(res.n_miss == 1)
    return out


@pytest.mark.parametrize("b", [1, 2, 3, 5, 8])
def test_k1_fifo_and_belady_are_textbook(b):
    rng = np.random.default_rng(77 + b)
    for trial in range(6):
        stream = [int(x) for x in rng.integers(0, 3 * b + 2, size=300)]
        assert _k1_policy_misses(stream, b, "fifo") == textbook.fifo_miss_sequence(stream, b)
        bel = _k1_policy_misses(stream, b, "belady")
        assert sum(bel) == sum(textbook.min_miss_sequence(stream, b))
        # MIN is optimal for demand paging: no online policy misses less
        for pol in ("lru", "fifo", "random"):
            assert sum(bel) <= sum(_k1_policy_misses(stream, b, pol))


@pytest.mark.parametrize("policy", ["lru", "fifo", "random", "belady"])
def test_policies_miss_only_on_first_touch_when_buffer_is_large(policy):
    from oracle.policy import next_use_table, random_priority

    rng = np.random.default_rng(11)
    ctx, k = 60, 8
    sels = [list(rng.choice(ctx, size=k, replace=False)) for _ in range(30)]
    nu = next_use_table(sels)
    st = LruState(ctx)
    seen = set()
    for t, sel in enumerate(sels):
        res = resolve(st, sel, t, ctx, [-1] * 1, 64, 0, policy=policy, priority=random_priority(5, t, 0, 0),
                      next_use=lambda q, t=t: nu(t, q))
        assert res.n_miss == len(set(sel) - seen)
        seen |= set(sel)


def test_random_victims_are_uniform():
    # one miss per call into a full buffer with one pinned hit: the victim is
    # one of the B - 1 unpinned slots, each equally likely
    from oracle.policy import random_priority

    b = 8
    counts = np.zeros(b)
    for t in range(4000):
        st = LruState(b)
        for s in range(b):
            st.owner[s] = s
            st.slot_of[s] = s
            st.stamp[s] = 0
        res = resolve(st, [0, 100], t + 1, 1000, [-1] * 20, 64, 0, policy="random",
                      priority=random_priority(9, t, 0, 0))
        assert res.n_hit == 1 and res.n_miss == 1
        counts[res.fetches[0][1]] += 1
    assert counts[0] == 0  # the pinned slot is never the victim
    exp = 4000 / (b - 1)
    chi2 = ((counts[1:] - exp) ** 2 / exp).sum()
    assert chi2 < 24.3  # 99.9th percentile of chi-square with 6 degrees of freedom
