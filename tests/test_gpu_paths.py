"""GPU tests of the step orchestration: the layer-ahead (overlapped) step
against the synchronous path and the oracle, fetch launch shapes, state
reset, and replay of a captured step graph."""

from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_harness import LSE_TOL, O_TOL, check_attention, check_hot_bytes, check_state, log, make_pool
from oracle.step import OracleDecoder
from tracegen.populate import queries
from tracegen.workloads import make_workload, with_fp8

pytestmark = pytest.mark.gpu


def _grouped_workload():
    # two index-share groups of three layers, ragged contexts, tail pages resident
    return make_workload("grouped_l6_g3", 11, 4, 6, 3, [20000, 9000, 33000, 4096], 32, 512, 1024, 6,
                         0.7, 0.8, "tail")


class _Buffers:
    """Step inputs and outputs; with T verify tokens the request axis of
    rows, queries and outputs carries R*T query sets (token-minor)."""

    def __init__(self, w, dev):
        import torch

        L, R, K, H, T = w.num_layers, w.num_requests, w.top_k, w.num_heads, w.num_verify
        self.rows = torch.full((L, R, T * K), -7, dtype=torch.int32, device=dev)
        self.counts = torch.full((L, R, 3), -7, dtype=torch.int32, device=dev)
        self.out = torch.full((L, R * T, H, 512), float("nan"), dtype=torch.float32, device=dev)
        self.lse = torch.full((L, R * T, H), float("nan"), dtype=torch.float32, device=dev)
        self.d_step = torch.zeros(1, dtype=torch.int32, device=dev)
        G = L // w.index_share
        self.topk = torch.empty((G, R, T * K), dtype=torch.int32, device=dev)
        self.q = torch.empty((L, R * T, H, 576), dtype=torch.int16, device=dev)

    def load(self, w, t, sel_t):
        import torch

        self.d_step.fill_(t)
        self.topk.copy_(torch.from_numpy(np.ascontiguousarray(sel_t, dtype=np.int32)).reshape(self.topk.shape))
        self.q.copy_(torch.from_numpy(queries(w, t).view(np.int16)).reshape(self.q.shape))

    def snapshot(self):
        return tuple(x.cpu().numpy().copy() for x in (self.rows, self.counts, self.out, self.lse))


def _run_step_path(hs, w, tr, buf):
    import torch

    snaps = []
    for t in range(w.steps):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        torch.cuda.synchronize(hs.device)
        snaps.append(buf.snapshot())
    return snaps


def _run_sync_path(hs, w, tr, buf):
    """hisparse_resolve of each group, then hisparse_sparse_mla_decode per layer."""
    import torch

    snaps = []
    g = w.index_share
    for t in range(w.steps):
        buf.load(w, t, tr[t])
        for gi in range(w.num_layers // g):
            l0 = gi * g
            hs.resolve(l0, g, buf.d_step, buf.topk[gi], buf.rows[l0:l0 + g], buf.counts[l0:l0 + g])
            for l in range(l0, l0 + g):
                hs.decode(l, buf.q[l], buf.rows[l], w.scale, buf.out[l], buf.lse[l])
        torch.cuda.synchronize(hs.device)
        snaps.append(buf.snapshot())
    return snaps


def _assert_same(a, b, what, exact_attention=True):
    """rows and counts bit for bit; O and lse bit for bit, or (when the two
    runs split the keys differently) within the oracle tolerances."""
    for t, (x, y) in enumerate(zip(a, b)):
        for name, u, v in zip(("rows", "counts", "out", "lse"), x, y):
            if exact_attention or name in ("rows", "counts"):
                assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"{what}: {name} differs at step {t}"
            elif name == "out":
                for l in range(u.shape[0]):
                    for r in range(u.shape[1]):
                        den = max(np.abs(u[l, r]).max(), 1e-30)
                        err = np.abs(u[l, r].astype(np.float64) - v[l, r]).max() / den
                        assert err <= O_TOL, f"{what}: O l={l} r={r} step {t} rel err {err:.3e}"
            else:
                fin = np.isfinite(u)
                assert np.array_equal(fin, np.isfinite(v)), f"{what}: lse finiteness differs at step {t}"
                assert np.abs(u[fin].astype(np.float64) - v[fin]).max(initial=0.0) <= LSE_TOL, \
                    f"{what}: lse differs at step {t}"


def test_overlapped_step_matches_oracle_and_sync_path():
    w = _grouped_workload()
    tr = w.trace(w.steps)
    hs = make_pool(w)
    buf = _Buffers(w, hs.device)
    log("overlapped step path, default fetch shape")
    step_snaps = _run_step_path(hs, w, tr, buf)

    # oracle: every step, every (layer, request)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(w.num_layers) for r in range(w.num_requests)]

    class _View:
        pass

    for t in range(w.steps):
        res = dec.resolve_step(t, tr[t])
        rows, counts, out, lse = step_snaps[t]
        for (l, r) in pairs:
            rr = res[(l, r)]
            assert np.array_equal(rows[l, r], np.asarray(rr.rows, np.int32)), f"rows t={t} l={l} r={r}"
            assert tuple(int(x) for x in counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), \
                f"counts t={t} l={l} r={r}"
        v = _View()
        v.w = w
        import torch

        v.out = torch.from_numpy(out)
        v.lse = torch.from_numpy(lse)
        worst = check_attention(v, dec, t, tr[t], pairs)
        assert worst <= O_TOL
    check_state(hs, dec, pairs, w.steps - 1)
    check_hot_bytes(hs, w, dec, [(0, 0), (2, 3), (5, 2)], w.steps - 1)

    log("synchronous path after reset, odd whole-group fetch grid")
    hs.reset_state()
    hs.set_pipeline(group_fetch_workgroups=7)
    sync_snaps = _run_sync_path(hs, w, tr, buf)
    _assert_same(step_snaps, sync_snaps, "sync path vs overlapped step", exact_attention=False)
    check_state(hs, dec, pairs, w.steps - 1)

    log("overlapped step path after reset, one workgroup per fetch, last layer unchunked")
    hs.reset_state()
    hs.set_pipeline(unit_fetch_workgroups=1, tail_chunks=1)
    again = _run_step_path(hs, w, tr, buf)
    _assert_same(step_snaps, again, "fetch grid 1, no tail chunks vs default", exact_attention=False)

    log("overlapped step path after reset, one request per tail chunk")
    hs.reset_state()
    hs.set_pipeline(unit_fetch_workgroups=5, tail_chunks=16)
    again = _run_step_path(hs, w, tr, buf)
    _assert_same(step_snaps, again, "4 tail chunks of one request vs default", exact_attention=False)
    assert hs.check_errors() == 0
    hs.close()


@pytest.mark.parametrize("variant", ["bf16", "fp8_verify2", "separate_fetches", "prefetch"])
def test_captured_step_graph_replays(variant):
    """A captured hisparse_step, replayed once per step with fresh inputs
    copied in between, matches eager steps of a second pool bit for bit
    (bf16 rows; FP8 rows with two verify tokens per request; the pipeline
    of separate fetches on two streams; hisparse_step_prefetch of the next
    step's selection, forked onto the side stream and joined)."""
    import torch

    w = _grouped_workload()
    if variant == "fp8_verify2":
        w = with_fp8(w)
        w.num_verify = 2
    tr = w.trace(w.steps + 1)
    pipeline = -1 if variant == "separate_fetches" else 1
    prefetch = variant == "prefetch"

    def run_step(hs, buf, nxt):
        if prefetch:
            hs.step_prefetch(buf.d_step, buf.topk, nxt, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse, None)
        else:
            hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)

    eager = make_pool(w)
    eager.set_pipeline(fetch_in_decode=pipeline)
    ebuf = _Buffers(w, eager.device)
    enext = torch.empty_like(ebuf.topk)
    want = []
    for t in range(w.steps):
        ebuf.load(w, t, tr[t])
        enext.copy_(torch.from_numpy(np.ascontiguousarray(tr[t + 1], dtype=np.int32)).reshape(enext.shape))
        run_step(eager, ebuf, enext)
        torch.cuda.synchronize(eager.device)
        want.append(ebuf.snapshot())
    eager.close()

    hs = make_pool(w)
    hs.set_pipeline(fetch_in_decode=pipeline)
    buf = _Buffers(w, hs.device)
    nxt = torch.empty_like(buf.topk)
    side = torch.cuda.Stream(device=hs.device)
    side.wait_stream(torch.cuda.current_stream(hs.device))
    graph = torch.cuda.CUDAGraph()
    buf.load(w, 0, tr[0])
    torch.cuda.synchronize(hs.device)
    with torch.cuda.graph(graph, stream=side):
        run_step(hs, buf, nxt)
    torch.cuda.synchronize(hs.device)
    # capture enqueues nothing: the state is still empty
    owner, stamp = hs.export_state(0, 0)
    assert np.all(owner == -1) and np.all(stamp == -1)
    for t in range(w.steps):
        buf.load(w, t, tr[t])
        nxt.copy_(torch.from_numpy(np.ascontiguousarray(tr[t + 1], dtype=np.int32)).reshape(nxt.shape))
        torch.cuda.synchronize(hs.device)
        graph.replay()
        torch.cuda.synchronize(hs.device)
        got = buf.snapshot()
        _assert_same([want[t]], [got], f"graph replay {t}")
        log(f"graph replay step {t} ok")
    assert hs.check_errors() == 0
    del graph
    hs.close()


def test_decode_layers_matches_oracle():
    """hisparse_sparse_mla_decode_layers over a whole group, on the rows a
    step resolved, equals the oracle's attention for every (layer, request)."""
    import torch

    w = _grouped_workload()
    tr = w.trace(w.steps)
    hs = make_pool(w)
    buf = _Buffers(w, hs.device)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(w.num_layers) for r in range(w.num_requests)]
    out2 = torch.full_like(buf.out, float("nan"))
    lse2 = torch.full_like(buf.lse, float("nan"))
    for t in range(3):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        dec.resolve_step(t, tr[t])
        g = w.index_share
        for gi in range(w.num_layers // g):
            l0 = gi * g
            hs.decode_layers(l0, g, buf.q[l0:l0 + g], buf.rows[l0:l0 + g], w.scale, out2[l0:l0 + g], lse2[l0:l0 + g])
        torch.cuda.synchronize(hs.device)

        class _View:
            pass

        v = _View()
        v.w, v.out, v.lse = w, out2.cpu(), lse2.cpu()
        worst = check_attention(v, dec, t, tr[t], pairs)
        log(f"decode_layers step {t}: worst O rel err {worst:.3e}")
    assert hs.check_errors() == 0
    hs.close()


def test_decode_layers_part_of_group_then_steps():
    """decode_layers over 1, 2 and 3 layers of a 4-layer index-share group
    (launch shapes whose key splits need more partial rows than a whole-group
    or a one-layer launch), then further steps: attention matches the oracle
    and the LRU state stays exact, so no partial write reached the
    metadata that follows the partial region in the workspace."""
    import torch

    # 64 requests x 64 heads x K 512: a 3-layer launch takes 2 key splits
    # (384 partial sets) where one layer at any request count needs at most 315
    w = make_workload("part_group_r64_g4", 21, 64, 4, 4, [4096] * 64, 64, 512, 1024, 6, 0.7, 0.8, "tail")
    tr = w.trace(w.steps)
    hs = make_pool(w)
    buf = _Buffers(w, hs.device)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(w.num_layers) for r in range(w.num_requests)]
    some = [(l, r) for l in range(w.num_layers) for r in (0, 17, 63)]
    out2 = torch.full_like(buf.out, float("nan"))
    lse2 = torch.full_like(buf.lse, float("nan"))

    class _View:
        pass

    for t in range(w.steps):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        res = dec.resolve_step(t, tr[t])
        torch.cuda.synchronize(hs.device)
        rows, counts = buf.rows.cpu().numpy(), buf.counts.cpu().numpy()
        for (l, r) in pairs:
            rr = res[(l, r)]
            assert np.array_equal(rows[l, r], np.asarray(rr.rows, np.int32)), f"rows t={t} l={l} r={r}"
            assert tuple(int(x) for x in counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), \
                f"counts t={t} l={l} r={r}"
        check_state(hs, dec, pairs, t)
        for (l0, n) in ((0, 3), (1, 3), (1, 2), (3, 1)):
            hs.decode_layers(l0, n, buf.q[l0:l0 + n], buf.rows[l0:l0 + n], w.scale, out2[l0:l0 + n],
                             lse2[l0:l0 + n])
            torch.cuda.synchronize(hs.device)
            v = _View()
            v.w, v.out, v.lse = w, out2.cpu(), lse2.cpu()
            lp = [(l, r) for (l, r) in some if l0 <= l < l0 + n]
            worst = check_attention(v, dec, t, tr[t], lp)
            log(f"step {t}: decode_layers({l0}, {n}) worst O rel err {worst:.3e}")
    assert hs.check_errors() == 0
    hs.close()
