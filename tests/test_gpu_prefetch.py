"""GPU parity of the cross-step prefetch (hisparse_prefetch,
hisparse_step_prefetch) against ``oracle.prefetch``: after every prefetch
the LRU state of every (layer, request), the hot-row bytes and the
(resident, hit, filled, dropped) counts are bit-exact; the steps around it
match the oracle as usual (rows, counts, state, attention)."""

from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_harness import check_attention, check_hot_bytes, check_state, log, make_pool
from tests.test_gpu_paths import _Buffers
from oracle.policy import random_priority
from oracle.prefetch import prefetch as oracle_prefetch
from oracle.resolve import resolve
from oracle.step import OracleDecoder
from tracegen import fill, make_workload, named_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _oracle_prefetch(dec, w, t, pred_t, policy="lru", seed=0):
    """oracle.prefetch on every (layer, request); returns {(l, r): result}."""
    out = {}
    for g in range(w.groups):
        for l in range(g * w.index_share, (g + 1) * w.index_share):
            for r in dec.requests:
                pri = random_priority(seed, t, l, r) if policy == "random" else None
                out[(l, r)] = oracle_prefetch(dec.states[(l, r)], list(pred_t[g][r]), t, w.ctx_len[r],
                                              w.block_tables[r], w.page_size, policy=policy, priority=pri)
    return out


def _oracle_resolve(dec, w, t, sel_t, policy, seed):
    """oracle.resolve under `policy` on every (layer, request) of dec."""
    out = {}
    for l in range(w.num_layers):
        g = l // w.index_share
        for r in dec.requests:
            out[(l, r)] = resolve(dec.states[(l, r)], sel_t[g][r], t, w.ctx_len[r], w.block_tables[r], w.page_size,
                                  dec.hot_base(r), policy=policy, priority=random_priority(seed, t, l, r))
    return out


def _check_rows(buf, res, pairs, t, what):
    rows, counts = buf.rows.cpu().numpy(), buf.counts.cpu().numpy()
    for (l, r) in pairs:
        rr = res[(l, r)]
        assert np.array_equal(rows[l, r], np.asarray(rr.rows, np.int32)), f"{what} rows t={t} l={l} r={r}"
        assert tuple(int(x) for x in counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), \
            f"{what} counts t={t} l={l} r={r}"


def _check_pf_counts(pfc, pres, pairs, t):
    for (l, r) in pairs:
        o = pres[(l, r)]
        assert tuple(int(x) for x in pfc[l, r]) == (o.n_resident, o.n_hit, o.n_filled, o.n_dropped), \
            f"prefetch counts t={t} l={l} r={r}: gpu {tuple(pfc[l, r])}"


def _prediction(kind, tr, t, rng, w):
    if kind == "exact":
        return tr[t + 1].copy()
    if kind == "reuse":
        return tr[t].copy()
    # half right, half random positions (distinct), shuffled
    p = tr[t + 1].copy()
    for g in range(p.shape[0]):
        for r in range(p.shape[1]):
            row = list(dict.fromkeys(list(p[g, r][: w.top_k // 2]) +
                                     [int(x) for x in rng.choice(w.ctx_len[r], w.top_k, replace=False)]))
            row = [x for x in row if x >= 0][: w.top_k]
            p[g, r] = rng.permutation(np.asarray(row + [-1] * (w.top_k - len(row)), np.int32))
    return p


@pytest.mark.parametrize("case", range(5))
def test_prefetch_small_configs(case):
    """hisparse_prefetch after each step with an exact, a noisy or a reused
    prediction, on random small configurations (residency, index sharing,
    LRU / FIFO / random replacement, tight and roomy buffers)."""
    import torch

    rng = np.random.default_rng(700 + case)
    K = int(rng.choice([16, 64, 100]))
    B = K + int(rng.choice([0, K // 2, 2 * K]))
    R, L = int(rng.integers(1, 4)), int(rng.choice([1, 2, 4]))
    share = int(rng.choice([s for s in (1, 2, 4) if L % s == 0]))
    ctx = [int(rng.integers(2 * K, 10 * K)) for _ in range(R)]
    w = make_workload(f"pf{case}", 720 + case, R, L, share, ctx, 16, K, B, 10, float(rng.choice([0.3, 0.7])), 0.8,
                      str(rng.choice(["none", "tail", "tail+half"])), page_size=16)
    policy = ["lru", "fifo", "random", "lru", "lru"][case]
    kinds = ["exact", "noisy", "reuse"]
    log(f"prefetch config {case}: R={R} L={L} g={share} K={K} B={B} ctx={ctx} res={w.residency} {policy}")
    tr = w.trace(w.steps + 1)
    hs = make_pool(w)
    if policy != "lru":
        hs.set_replacement(policy, 99)
    buf = _Buffers(w, hs.device)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(L) for r in range(R)]
    pfc = torch.full((L, R, 4), -7, dtype=torch.int32, device=hs.device)
    d_pred = torch.empty_like(buf.topk)
    for t in range(w.steps):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        torch.cuda.synchronize(hs.device)
        res = _oracle_resolve(dec, w, t, tr[t], policy, 99)
        _check_rows(buf, res, pairs, t, "step")
        check_attention(buf_view(w, buf), dec, t, tr[t], pairs)
        pred = _prediction(kinds[t % 3], tr, t, rng, w)
        d_pred.copy_(torch.from_numpy(pred))
        for g in range(w.groups):
            hs.prefetch(g * share, share, buf.d_step, d_pred[g], pfc[g * share:(g + 1) * share])
        torch.cuda.synchronize(hs.device)
        pres = _oracle_prefetch(dec, w, t, pred, policy, 99)
        _check_pf_counts(pfc.cpu().numpy(), pres, pairs, t)
        check_state(hs, dec, pairs, t)
        check_hot_bytes(hs, w, dec, pairs, t)
    assert hs.check_errors() == 0
    hs.close()


class buf_view:
    def __init__(self, w, buf):
        self.w, self.out, self.lse = w, buf.out.cpu(), buf.lse.cpu()


def _grouped():
    return make_workload("pf_grouped_l6_g3", 13, 4, 6, 3, [20000, 9000, 33000, 4096], 32, 512, 1024, 6, 0.7, 0.8,
                         "tail")


@pytest.mark.parametrize("shape,two_part", [("grouped", 0), ("grouped", 1), ("single_layer", 0), ("single_layer", 1),
                                            ("full_size", 0), ("full_size", 1)])
def test_step_prefetch_matches_oracle(shape, two_part):
    """hisparse_step_prefetch with the exact next selection: the step's own
    outputs as in the oracle, the in-step prefetch as oracle.prefetch, and
    (room permitting) no miss in the next step.  two_part = 0 runs the
    default pipeline (the decode reads the filled rows from the host pool,
    the prefetch beside it); two_part = 1 runs separate fetches and decodes
    each group's last layer in two parts (resident_first) where that
    pipeline's default would not (small shapes: both parts split, merged by
    combine_splits); the full size r32_ctx128k_l4 case (requests 0 and 17
    checked) merges in the second part."""
    import torch

    w = {"grouped": _grouped, "single_layer": lambda: named_workload("r8_ctx32k"),
         "full_size": lambda: named_workload("r32_ctx128k_l4")}[shape]()
    steps = 6 if shape != "full_size" else 3
    tr = w.trace(steps + 1)
    hs = make_pool(w)
    if two_part:
        hs.set_pipeline(resident_first=1, fetch_in_decode=-1)
    buf = _Buffers(w, hs.device)
    reqs = list(range(w.num_requests)) if shape != "full_size" else [0, 17]
    dec = OracleDecoder(w, requests=reqs)
    pairs = [(l, r) for l in range(w.num_layers) for r in reqs]
    pfc = torch.full((w.num_layers, w.num_requests, 4), -7, dtype=torch.int32, device=hs.device)
    d_next = torch.empty_like(buf.topk)
    for t in range(steps):
        buf.load(w, t, tr[t])
        d_next.copy_(torch.from_numpy(np.ascontiguousarray(tr[t + 1])))
        hs.step_prefetch(buf.d_step, buf.topk, d_next, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse, pfc)
        torch.cuda.synchronize(hs.device)
        res = dec.resolve_step(t, tr[t])
        _check_rows(buf, res, pairs, t, "step_prefetch")
        if t > 0:
            assert all(res[p].n_miss == 0 for p in pairs), "an exact prediction with room leaves no miss"
        att = {"grouped": pairs, "single_layer": [(0, 0), (0, 5)], "full_size": [(3, 0), (3, 17)]}[shape]
        check_attention(buf_view(w, buf), dec, t, tr[t], att)
        pres = _oracle_prefetch(dec, w, t, tr[t + 1])
        _check_pf_counts(pfc.cpu().numpy(), pres, pairs, t)
        assert all(pres[p].n_dropped == 0 for p in pairs)
        check_state(hs, dec, pairs, t)
        check_hot_bytes(hs, w, dec, pairs[:3], t)
        log(f"{shape} step {t}: misses {sum(res[p].n_miss for p in pairs)}, "
            f"prefetched {sum(pres[p].n_filled for p in pairs)}")
    assert hs.check_errors() == 0
    hs.close()


@pytest.mark.parametrize("fetch_in_decode", [1, -1], ids=["fetch_in_decode", "separate_fetches"])
def test_step_prefetch_full_size_exact_path(fetch_in_decode):
    """r32_ctx128k_l4 with the exact next selection prefetched in every step:
    from step 1 on no miss, and row ids and LRU state bit-identical to the
    plain step path (the same victims, fetched one step earlier); O and lse
    too, since the decode sees the same rows in the same order: whether a
    row is read from the host pool (a fill) or from its hot row (a hit once
    prefetched) changes no arithmetic.  With separate fetches both runs
    decode each group's last layer in one launch (decoded resident rows
    first, its keys would be split by hit or miss, which the prefetch
    changes, and the results would then agree to rounding only)."""
    import torch

    w = named_workload("r32_ctx128k_l4")
    steps = 5
    tr = w.trace(steps + 1)
    hs = make_pool(w)
    hs.set_pipeline(resident_first=-1, fetch_in_decode=fetch_in_decode)
    buf = _Buffers(w, hs.device)
    plain = []
    for t in range(steps):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        torch.cuda.synchronize(hs.device)
        plain.append(buf.snapshot())
    st_plain = [hs.export_state(r, l) for l in range(w.num_layers) for r in range(w.num_requests)]
    hs.reset_state()
    d_next = torch.empty_like(buf.topk)
    pfc = torch.zeros((w.num_layers, w.num_requests, 4), dtype=torch.int32, device=hs.device)
    for t in range(steps):
        buf.load(w, t, tr[t])
        pfc.zero_()
        if t + 1 < steps:
            d_next.copy_(torch.from_numpy(np.ascontiguousarray(tr[t + 1])))
            hs.step_prefetch(buf.d_step, buf.topk, d_next, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse,
                             pfc)
        else:  # no prefetch after the last step, so the final states compare
            hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        torch.cuda.synchronize(hs.device)
        rows, counts, out, lse = buf.snapshot()
        assert np.array_equal(rows, plain[t][0]), f"rows differ at step {t}"
        assert np.array_equal(out.view(np.uint32), plain[t][2].view(np.uint32)), f"O differs at step {t}"
        assert np.array_equal(lse.view(np.uint32), plain[t][3].view(np.uint32)), f"lse differs at step {t}"
        if t > 0:
            # every miss of the plain path became a hit; residents unchanged
            assert counts[..., 2].sum() == 0
            assert np.array_equal(counts[..., 0], plain[t][1][..., 0])
            assert np.array_equal(counts[..., 1], plain[t][1][..., 1] + plain[t][1][..., 2])
        p = pfc.cpu().numpy()
        assert p[..., 3].sum() == 0
        if t + 1 < steps:
            assert p[..., 2].sum() == plain[t + 1][1][..., 2].sum(), "prefetched rows = the next step's misses"
        log(f"full size step {t}: prefetched {int(p[..., 2].sum())} rows")
    st = [hs.export_state(r, l) for l in range(w.num_layers) for r in range(w.num_requests)]
    for (o1, s1), (o2, s2) in zip(st_plain, st):
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2)
    assert hs.check_errors() == 0
    hs.close()
