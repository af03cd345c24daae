"""Run-to-run determinism of the whole step at the named workloads' full
sizes: each runs twice from the empty state and once as a captured-graph
replay, and row ids, counts, the LRU state of every (layer, request), O and
lse must agree bit for bit (the vLLM Hybrid HiSparse blog, "与 vLLM 其余部分的
组合": speculative decoding relies on a per-step replayable resolver plan)."""

from __future__ import annotations

import numpy as np
import pytest

from tests.gpu_harness import log, make_pool
from tests.test_gpu_paths import _Buffers
from tracegen import fill, named_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _state(hs, w):
    return [hs.export_state(r, l) for l in range(w.num_layers) for r in range(w.num_requests)]


def _same(a, b, what):
    for t, (x, y) in enumerate(zip(a, b)):
        for name, u, v in zip(("rows", "counts", "out", "lse"), x, y):
            assert np.array_equal(u.view(np.uint8), v.view(np.uint8)), f"{what}: {name} differs at step {t}"


def _eager(hs, w, tr, buf, steps):
    import torch

    snaps = []
    for t in range(steps):
        buf.load(w, t, tr[t])
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
        torch.cuda.synchronize(hs.device)
        snaps.append(buf.snapshot())
    return snaps


@pytest.mark.parametrize("name,steps", [("r32_ctx128k_l4", 6), ("mixed_r64", 8), ("miss_1m", 8)])
def test_full_size_runs_are_bitwise_repeatable(name, steps):
    import torch

    w = named_workload(name)
    tr = w.trace(steps)
    hs = make_pool(w)
    buf = _Buffers(w, hs.device)
    log(f"{name}: first eager run of {steps} steps")
    first = _eager(hs, w, tr, buf, steps)
    st1 = _state(hs, w)
    hs.reset_state()
    log(f"{name}: second eager run")
    second = _eager(hs, w, tr, buf, steps)
    _same(first, second, f"{name} second run")
    st2 = _state(hs, w)
    for (o1, s1), (o2, s2) in zip(st1, st2):
        assert np.array_equal(o1, o2) and np.array_equal(s1, s2), f"{name}: LRU state differs"
    del second

    log(f"{name}: captured-graph replay")
    hs.reset_state()
    side = torch.cuda.Stream(device=hs.device)
    side.wait_stream(torch.cuda.current_stream(hs.device))
    graph = torch.cuda.CUDAGraph()
    buf.load(w, 0, tr[0])
    torch.cuda.synchronize(hs.device)
    with torch.cuda.graph(graph, stream=side):
        hs.step(buf.d_step, buf.topk, buf.q, w.scale, buf.rows, buf.counts, buf.out, buf.lse)
    torch.cuda.synchronize(hs.device)
    for t in range(steps):
        buf.load(w, t, tr[t])
        torch.cuda.synchronize(hs.device)
        graph.replay()
        torch.cuda.synchronize(hs.device)
        _same([first[t]], [buf.snapshot()], f"{name} graph replay {t}")
    st3 = _state(hs, w)
    for (o1, s1), (o3, s3) in zip(st1, st3):
        assert np.array_equal(o1, o3) and np.array_equal(s1, s3), f"{name}: LRU state differs after replays"
    assert hs.check_errors() == 0
    del graph
    hs.close()
    log(f"{name}: two eager runs and the graph replays agree bit for bit")
