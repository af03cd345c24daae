"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Bit-exact: row ids, (resident, hit, miss) counts, LRU owner/stamp state and
hot-row bytes.  Attention: max |O_gpu - O_ref| / max |O_ref| <= 2e-3 per
(layer, request, step), |lse_gpu - lse_ref| <= 2e-3.
"""

import json
import os

import numpy as np
import pytest

from tests.gpu_harness import GpuRun, check_attention, check_hot_bytes, check_state, log, make_pool, run_and_compare
from oracle.resolve import ERR_DUP, ERR_RANGE, ERR_STEP, LruState, resolve
from oracle.step import OracleDecoder
from tracegen import fill, make_workload, named_workload
from tracegen.workloads import Workload

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _custom_workload(name, ctx, page, bt, B, K, H=16, L=1):
    w = Workload(name=name, seed=77, num_requests=1, num_layers=L, index_share=1, ctx_len=[ctx],
                 num_heads=H, top_k=K, hot_slots=B, steps=0, retain=0.0, alpha=None, residency="custom",
                 page_size=page)
    w.block_tables = [np.asarray(bt, np.int32)]
    w.resident_blocks = max([b + 1 for b in bt if b >= 0], default=0)
    return w


def test_worked_examples_gpu():
    with open(os.path.join(GOLDEN, "lru_worked_example.json")) as f:
        ex = json.load(f)
    for e in ex["examples"]:
        log(f"worked example {e['name']}")
        w = _custom_workload(e["name"], e["ctx"], e["page_size"], e["block_table"], e["hot_slots"], 3)
        assert w.resident_rows_per_layer == e["hot_base"]
        hs = make_pool(w)
        run = GpuRun(w, hs)
        dec = OracleDecoder(w)
        for s in e["steps"]:
            sel = np.array([[s["sel"]]], np.int32)
            rows, counts = run.step(s["t"], sel)
            want = [(e["hot_base"] + sl) if sl is not None else rr for sl, rr in zip(s["slots"], s["resident_rows"])]
            assert list(rows[0, 0]) == want
            assert list(counts[0, 0]) == s["counts"]
            owner, stamp = hs.export_state(0, 0)
            assert list(owner) == s["owner"] and list(stamp) == s["stamp"]
            dec.resolve_step(s["t"], sel)
            check_hot_bytes(hs, w, dec, [(0, 0)], s["t"])
            check_attention(run, dec, s["t"], sel, [(0, 0)])
        assert hs.check_errors() == 0
        hs.close()


def test_tiny_every_step():
    w = named_workload("tiny")
    hs, _, _ = run_and_compare(w, bytes_pairs=[(0, 0)], label="tiny")
    hs.close()


@pytest.mark.parametrize("case", range(6))
def test_random_small_configs_unsorted(case):
    rng = np.random.default_rng(100 + case)
    page = int(rng.choice([4, 16, 64]))
    K = int(rng.choice([1, 5, 64, 100, 257]))
    B = K + int(rng.integers(0, 3 * K + 1))
    R, L = int(rng.integers(1, 4)), int(rng.choice([1, 2, 4]))
    share = int(rng.choice([s for s in (1, 2, 4) if L % s == 0]))
    ctx = [int(rng.integers(max(K // 2, 1), 6 * K + 50)) for _ in range(R)]
    w = make_workload(f"rand{case}", 200 + case, R, L, share, ctx, 16 * int(rng.integers(1, 3)), K, B, 12,
                      float(rng.choice([0.0, 0.5, 0.9])), 0.8, str(rng.choice(["none", "tail", "tail+half"])),
                      page_size=page)
    log(f"random config {case}: R={R} L={L} g={share} K={K} B={B} page={page} ctx={ctx} res={w.residency}")
    tr = w.trace()
    # scramble the order of every selection and punch some padding holes
    for t in range(w.steps):
        for g in range(w.groups):
            for r in range(R):
                row = tr[t, g, r]
                if case % 2 == 0:
                    row[rng.random(K) < 0.1] = -1
                tr[t, g, r] = rng.permutation(row)
    hs = make_pool(w)
    run = GpuRun(w, hs)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(L) for r in range(R)]
    for t in range(w.steps):
        rows, counts = run.step(t, tr[t])
        res = dec.resolve_step(t, tr[t])
        for (l, r), rr in res.items():
            assert np.array_equal(rows[l, r], np.asarray(rr.rows, np.int32)), (t, l, r)
            assert tuple(int(x) for x in counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), (t, l, r)
        check_state(hs, dec, pairs, t)
        check_hot_bytes(hs, w, dec, pairs, t)
        check_attention(run, dec, t, tr[t], pairs)
    assert hs.check_errors() == 0
    hs.close()


def test_device_error_flags():
    w = _custom_workload("errs", 50, 8, [-1] * 7, 8, 5)
    hs = make_pool(w)
    run = GpuRun(w, hs)
    st = LruState(8)
    cases = [
        (0, [3, 99, 3, -1, -5], ERR_RANGE | ERR_DUP),
        (5, [4, 6, 8, 10, 12], 0),
        (4, [6, 1, 2, 3, 5], ERR_STEP),
        (5, [12, 10, 8, 6, 4], 0),
        (6, [7, 7, 7, 60, 1], ERR_RANGE | ERR_DUP),
    ]
    for t, sel, want_err in cases:
        rows, counts = run.step(t, np.array([[sel]], np.int32))
        res = resolve(st, sel, t, 50, [-1] * 7, 8, 0)
        assert res.errors == want_err
        assert list(rows[0, 0]) == res.rows, (t, sel)
        assert tuple(counts[0, 0]) == (res.n_resident, res.n_hit, res.n_miss)
        owner, stamp = hs.export_state(0, 0)
        assert list(owner) == st.owner and list(stamp) == st.stamp
        assert hs.check_errors() == want_err
    hs.close()


def test_determinism_tiny():
    import torch

    w = named_workload("tiny")
    tr = w.trace(10)
    outs = []
    for _ in range(2):
        hs = make_pool(w)
        run = GpuRun(w, hs)
        acc = []
        for t in range(10):
            rows, counts = run.step(t, tr[t])
            acc.append((rows.copy(), counts.copy(), run.out.cpu().numpy().copy(), run.lse.cpu().numpy().copy()))
        outs.append(acc)
        hs.close()
        torch.cuda.synchronize()
    for a, b in zip(*outs):
        for x, y in zip(a, b):
            assert np.array_equal(x, y)


def test_r8_ctx32k():
    w = named_workload("r8_ctx32k")
    hs, _, _ = run_and_compare(w, attend_every=4, bytes_pairs=[(0, 0), (0, 7)], label="r8_ctx32k")
    hs.close()


def test_mixed_r64():
    w = named_workload("mixed_r64")
    hs, _, _ = run_and_compare(w, attend_every=5, attend_pairs=[(0, r) for r in (0, 13, 40, 63)],
                               bytes_pairs=[(0, 5)], label="mixed_r64")
    hs.close()


def test_miss_1m():
    w = named_workload("miss_1m")
    hs, _, _ = run_and_compare(w, attend_every=4, bytes_pairs=[(0, 0)], label="miss_1m")
    hs.close()


def test_r32_ctx128k_l4():
    w = named_workload("r32_ctx128k_l4")
    pairs = [(0, 0), (1, 9), (2, 21), (3, 31)]
    hs, _, _ = run_and_compare(w, attend_every=5, attend_pairs=pairs, bytes_pairs=[(3, 17)],
                               label="r32_ctx128k_l4")
    hs.close()


def test_indexer_order_misses_in_few_position_buckets():
    """Misses concentrated in a narrow range of a 1M-token context, in
    indexer order: each step's selection of request 0 is a contiguous block
    of 2048 positions (shuffled) that moves on by 1024 per step, so about
    1024 misses per step fall into one or two of the metadata kernel's
    position buckets (1024 positions wide here), whose rank counts are then
    as long as the misses; request 1 draws the usual trace.  Bit-exact
    against the oracle."""
    w = make_workload("few_buckets", 61, 2, 1, 1, [1 << 20, 300000], 16, 2048, 4096, 5, 0.7, 0.8, "none")
    tr = w.trace(w.steps).copy()
    rng = np.random.default_rng(61)
    for t in range(tr.shape[0]):
        tr[t, 0, 0] = rng.permutation(np.arange(500000 + 1024 * t, 500000 + 1024 * t + 2048, dtype=np.int32))
        tr[t, 0, 1] = rng.permutation(tr[t, 0, 1])
    hs, _, _ = run_and_compare(w, bytes_pairs=[(0, 0), (0, 1)], label="misses in few position buckets", trace=tr)
    hs.close()


def test_r8_ctx32k_indexer_order():
    """The r8_ctx32k workload with every selection in a shuffled (indexer)
    order instead of ascending: the metadata kernel's unsorted path at full
    width (K = 2048, one token), bit-exact against the oracle."""
    w = named_workload("r8_ctx32k")
    tr = w.trace(w.steps).copy()
    rng = np.random.default_rng(4242)
    for t in range(tr.shape[0]):
        for g in range(tr.shape[1]):
            for r in range(tr.shape[2]):
                tr[t, g, r] = rng.permutation(tr[t, g, r])
    hs, _, _ = run_and_compare(w, attend_every=4, bytes_pairs=[(0, 3)], label="r8_ctx32k indexer order", trace=tr)
    hs.close()
