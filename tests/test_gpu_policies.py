"""GPU parity of the replacement policies (HiSparse summary article,
section 04: LRU compared with FIFO and random replacement): the device
RESOLVE under each online policy against the oracle, step by step."""

from __future__ import annotations

import numpy as np
import pytest

from oracle.policy import random_priority
from oracle.resolve import LruState, resolve
from tests.gpu_harness import GpuRun, log, make_pool
from tracegen.workloads import make_workload

pytestmark = pytest.mark.gpu

SEED = 0x5EED_1234_ABCD


def _grouped():
    return make_workload("grouped_l6_g3", 11, 4, 6, 3, [20000, 9000, 33000, 4096], 32, 512, 1024, 8,
                         0.7, 0.8, "tail")


def _check_policy(w, policy, steps):
    hs = make_pool(w)
    hs.set_replacement(policy, SEED)
    run = GpuRun(w, hs)
    tr = w.trace(steps)
    states = {(l, r): LruState(w.hot_slots) for l in range(w.num_layers) for r in range(w.num_requests)}
    misses = 0
    for t in range(steps):
        rows, counts = run.step(t, tr[t])
        for l in range(w.num_layers):
            g = l // w.index_share
            for r in range(w.num_requests):
                res = resolve(states[(l, r)], tr[t][g][r], t, w.ctx_len[r], w.block_tables[r], w.page_size,
                              w.resident_rows_per_layer + r * w.hot_slots, policy=policy,
                              priority=random_priority(SEED, t, l, r))
                assert np.array_equal(rows[l, r], np.asarray(res.rows, np.int32)), \
                    f"{policy} rows t={t} l={l} r={r}"
                assert tuple(int(x) for x in counts[l, r]) == (res.n_resident, res.n_hit, res.n_miss), \
                    f"{policy} counts t={t} l={l} r={r}"
                misses += res.n_miss
    for l in range(w.num_layers):
        for r in range(w.num_requests):
            owner, stamp = hs.export_state(r, l)
            assert np.array_equal(owner, np.asarray(states[(l, r)].owner, np.int32)), f"{policy} owner l={l} r={r}"
            assert np.array_equal(stamp, np.asarray(states[(l, r)].stamp, np.int32)), f"{policy} stamp l={l} r={r}"
    assert hs.check_errors() == 0
    hs.close()
    log(f"{w.name} {policy}: {steps} steps bit-exact, {misses} misses")
    return misses


@pytest.mark.parametrize("policy", ["fifo", "random", "lru"])
def test_policy_parity_grouped(policy):
    _check_policy(_grouped(), policy, 8)


@pytest.mark.parametrize("policy", ["fifo", "random"])
def test_policy_parity_tiny_tight_buffer(policy):
    # B = K: every step evicts most of the buffer; long trace
    w = make_workload("tiny_b_eq_k", 1, 1, 1, 1, [4096], 16, 256, 256, 40, 0.7, 0.8, "none")
    _check_policy(w, policy, 40)
