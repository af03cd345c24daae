"""The allocation-free decode entry point against the workspace one.

hisparse_sparse_mla_decode_layers_static keeps its key-split partials in a
fixed device array instead of the pool's workspace; on the same rows and
queries it must give the same O and lse as
hisparse_sparse_mla_decode_layers, bit for bit, call after call, also when
a later call is smaller than the one before it or comes from another pool.
"""

from __future__ import annotations

import numpy as np
import pytest

from host_offloaded_kv_amd import hisparse as H
from tests.gpu_harness import log, make_pool
from tracegen import fill, make_workload, named_workload
from tracegen.populate import queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load()
    fill.build(force=False)


def _resolved(w, steps):
    """A pool stepped `steps` times; returns (pool, q, rows) of the last step."""
    import torch

    hs = make_pool(w)
    dev = hs.device
    L, R, K, Hh = w.num_layers, w.num_requests, w.top_k, w.num_heads
    rows = torch.empty((L, R, K), dtype=torch.int32, device=dev)
    counts = torch.empty((L, R, 3), dtype=torch.int32, device=dev)
    out = torch.empty((L, R, Hh, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((L, R, Hh), dtype=torch.float32, device=dev)
    d_step = torch.zeros(1, dtype=torch.int32, device=dev)
    tr = w.trace(steps)
    for t in range(steps):
        d_step.fill_(t)
        topk = torch.from_numpy(tr[t]).to(dev)
        q = torch.from_numpy(queries(w, t).view(np.int16)).to(dev)
        hs.step(d_step, topk, q, w.scale, rows, counts, out, lse)
    torch.cuda.synchronize(dev)
    return hs, q, rows


def _both(hs, w, q, rows, l0, n):
    """(O, lse) of layers [l0, l0 + n) from the workspace entry point and
    from the static one (into buffers pre-filled with NaN)."""
    import torch

    outs = []
    for fn in (H.hisparse_sparse_mla_decode_layers, H.hisparse_sparse_mla_decode_layers_static):
        o = torch.full((n, w.num_requests, w.num_heads, 512), float("nan"), device=hs.device)
        ls = torch.full((n, w.num_requests, w.num_heads), float("nan"), device=hs.device)
        fn(hs.pool, l0, n, q[l0].data_ptr(), rows[l0].data_ptr(), w.scale, o.data_ptr(), ls.data_ptr(), hs.stream)
        torch.cuda.synchronize(hs.device)
        outs.append((o.cpu().numpy(), ls.cpu().numpy()))
    return outs


def _same(a, b, what):
    for x, y, name in zip(a, b, ("O", "lse")):
        assert np.array_equal(x.view(np.uint32), y.view(np.uint32)), f"{what}: {name} differs"
    assert np.isfinite(a[0]).all()


def test_static_scratch_matches_workspace_partials():
    # 8 requests x 64 heads, one 4-layer group: a 3-layer launch takes 11
    # key splits (35 MB of partials), a 1-layer launch 16 (17 MB)
    wa = make_workload("noalloc_g4", 31, 8, 4, 4, [8192] * 8, 64, 1024, 2048, 3, 0.7, 0.8, "tail")
    hs, q, rows = _resolved(wa, 3)
    ref, got = _both(hs, wa, q, rows, 0, 3)
    _same(ref, got, "layers 0..2")
    log("static scratch: 3-layer launch matches")
    ref, got = _both(hs, wa, q, rows, 3, 1)  # a smaller launch right after a larger one
    _same(ref, got, "layer 3 after layers 0..2")
    log("static scratch: a smaller launch after it matches")
    # a different, smaller pool shares the same array
    wt = named_workload("tiny")
    ht, qt, rt = _resolved(wt, 4)
    ref, got = _both(ht, wt, qt, rt, 0, 1)
    _same(ref, got, "tiny after the grouped pool")
    # and the first pool again, after the tiny one
    ref, got = _both(hs, wa, q, rows, 1, 2)
    _same(ref, got, "layers 1..2 after tiny")
    assert hs.check_errors() == 0 and ht.check_errors() == 0
    ht.close()
    hs.close()


def test_static_scratch_rejects_launches_beyond_its_size():
    """255 requests x 64 heads split twice need 510 x 64 partial rows
    (67.4 MB), just above the 64 MiB array: refused before any launch."""
    import torch

    w = make_workload("noalloc_big", 32, 255, 1, 1, [128] * 255, 64, 128, 128, 1, 0.7, 0.8, "none")
    hs = make_pool(w)
    q = torch.zeros((w.num_requests, w.num_heads, 576), dtype=torch.int16, device=hs.device)
    rows = torch.full((w.num_requests, w.top_k), -1, dtype=torch.int32, device=hs.device)
    o = torch.zeros((w.num_requests, w.num_heads, 512), device=hs.device)
    ls = torch.zeros((w.num_requests, w.num_heads), device=hs.device)
    with pytest.raises(H.HiSparseError) as ei:
        H.hisparse_sparse_mla_decode_layers_static(hs.pool, 0, 1, q.data_ptr(), rows.data_ptr(), 1.0, o.data_ptr(),
                                                   ls.data_ptr(), hs.stream)
    assert ei.value.status == H.HISPARSE_EINVAL
    msg = H.hisparse_last_error()
    assert "static scratch" in msg and str(H.HISPARSE_STATIC_SCRATCH_BYTES) in msg and "67368960" in msg
    # the workspace entry point serves the same launch
    H.hisparse_sparse_mla_decode_layers(hs.pool, 0, 1, q.data_ptr(), rows.data_ptr(), 1.0, o.data_ptr(),
                                        ls.data_ptr(), hs.stream)
    torch.cuda.synchronize(hs.device)
    assert (o == 0).all().item() and torch.isneginf(ls).all().item()
    assert hs.check_errors() == 0
    hs.close()
