"""The seeded input generator: determinism, trace structure, value stream."""

import numpy as np
import pytest

from tracegen import fill, kv_rows, named_workload, q_block, selection_trace
from tracegen.trace import es_top
from tracegen.values import bf16_values, float_values, kv_key


@pytest.fixture(scope="module", autouse=True)
def _built():
    fill.build(force=False)


def test_fill_c_matches_numpy():
    key = kv_key(7, 3, 1)
    a = np.empty(576 * 257, np.uint16)
    fill.fill_array(a, key, e0=576 * 1000)
    b = bf16_values(key, np.arange(576 * 1000, 576 * 1257, dtype=np.uint64))
    assert np.array_equal(a, b)
    pos = np.array([0, 5, 99999, 3, 5])
    assert np.array_equal(fill.rows(key, pos, 576), kv_rows(7, 3, 1, pos))


def test_value_statistics_and_determinism():
    x = float_values(kv_key(1, 0, 0), np.arange(2_000_000))
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 1) < 3e-3
    assert np.abs(x).max() <= 6
    assert np.array_equal(q_block(1, 2, 0, 0, 4), q_block(1, 2, 0, 0, 4))
    assert not np.array_equal(q_block(1, 2, 0, 0, 4), q_block(1, 3, 0, 0, 4))


def test_trace_structure():
    tr = selection_trace(3, [5000, 200], 256, 12, 2, 0.7, 0.8)
    assert tr.shape == (12, 2, 2, 256)
    n_keep = int(np.floor(0.7 * 256 + 0.5))
    for g in range(2):
        s0 = tr[:, g, 0]
        for t in range(12):
            assert np.all(np.diff(s0[t]) > 0) and s0[t].min() >= 0 and s0[t].max() < 5000
            if t:
                assert len(np.intersect1d(s0[t], s0[t - 1])) >= n_keep
        # ctx < K: whole context, padded with -1
        s1 = tr[:, g, 1]
        assert np.array_equal(s1[0, :200], np.arange(200)) and np.all(s1[:, 200:] == -1)
    assert np.array_equal(tr, selection_trace(3, [5000, 200], 256, 12, 2, 0.7, 0.8))


def test_es_top_ties_and_uniform():
    u = np.array([0.5, 0.5, 0.9, 0.5])
    assert list(np.sort(es_top(u, np.ones(4), 2, None))) == [0, 2]
    rng = np.random.default_rng(0)
    counts = np.zeros(10)
    for _ in range(4000):
        counts[es_top(rng.random(10), np.ones(10), 3, None)] += 1
    assert np.all(np.abs(counts / 4000 - 0.3) < 0.04)


def test_named_workloads_shapes():
    w = named_workload("mixed_r64")
    assert w.num_requests == 64 and min(w.ctx_len) >= 4096 and max(w.ctx_len) <= 163840
    for r in range(64):
        bt = w.block_tables[r]
        assert bt[-1] >= 0  # the tail page is always resident
        assert (bt[:-1] >= 0).sum() == (len(bt) - 1) // 2
    ids = np.concatenate([b[b >= 0] for b in w.block_tables])
    assert np.array_equal(np.sort(ids), np.arange(w.resident_blocks))
    w3 = named_workload("r32_ctx128k_l4")
    assert w3.groups == 1 and w3.resident_rows_per_layer == 32 * 64


def test_growing_trace_structure():
    from tracegen import growing_selection_trace

    ctx0 = [300, 190, 64]
    tr = growing_selection_trace(7, ctx0, 64, 24, 2, 0.7, 0.8)
    again = growing_selection_trace(7, ctx0, 64, 24, 2, 0.7, 0.8)
    assert np.array_equal(tr, again)
    newest = 0
    for t in range(24):
        for g in range(2):
            for r, c0 in enumerate(ctx0):
                s = tr[t, g, r]
                v = s[s >= 0]
                assert v.shape[0] == min(64, c0 + t + 1)
                assert np.all(np.diff(v) > 0) and v.min() >= 0 and v.max() < c0 + t + 1
                newest += int(v.max() == c0 + t)
    assert newest > 24 * 2 * 3 // 2  # recency weighting picks the just-appended token most steps


def test_growing_schedule_invariants():
    from tracegen.residency import growing_schedule

    ctx0, page, steps = [100, 64, 37], 16, 90
    sch = growing_schedule(ctx0, steps, page, total_blocks=12, keep=2)
    for t in range(steps):
        for r in range(3):
            bt = sch.bt_at[t][r]
            pos = ctx0[r] + t
            assert bt[pos // page] >= 0  # tail page resident at its append
            res = [b for b in bt if b >= 0]
            assert len(res) == len(set(res)) and len(res) <= 3
        used = [b for r in range(3) for b in sch.bt_at[t][r] if b >= 0]
        assert len(used) == len(set(used))  # no block shared between requests
