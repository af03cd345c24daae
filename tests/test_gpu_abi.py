"""Host-side error paths of the C ABI that need a live pool: misaligned
query pointers, and the pinned-pool budget (ENOMEM) on a real device."""

from __future__ import annotations

import ctypes

import pytest

from host_offloaded_kv_amd import hisparse as H
from tracegen import fill, named_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    H.load()
    fill.build(force=False)


def test_misaligned_query_and_rows_rejected():
    import torch

    w = named_workload("tiny")
    hs = H.HiSparse(w.config_dict(), "cuda:0")
    lib = H.load()
    dev = hs.device
    K, Hh = w.top_k, w.num_heads
    q = torch.zeros(Hh * 576 + 8, dtype=torch.int16, device=dev)
    rows = torch.full((K,), -1, dtype=torch.int32, device=dev)
    counts = torch.zeros(3, dtype=torch.int32, device=dev)
    out = torch.zeros(Hh * 512, dtype=torch.float32, device=dev)
    lse = torch.zeros(Hh, dtype=torch.float32, device=dev)
    step = torch.zeros(1, dtype=torch.int32, device=dev)
    topk = torch.full((K,), -1, dtype=torch.int32, device=dev)
    bad_q = q.data_ptr() + 2  # bf16-aligned but not 16-byte aligned
    s = hs.stream
    assert lib.hisparse_sparse_mla_decode(hs.pool, 0, bad_q, rows.data_ptr(), 1.0, out.data_ptr(), lse.data_ptr(),
                                          s) == H.HISPARSE_EINVAL
    assert "d_q" in H.hisparse_last_error()
    assert lib.hisparse_sparse_mla_decode_layers(hs.pool, 0, 1, bad_q, rows.data_ptr(), 1.0, out.data_ptr(),
                                                 lse.data_ptr(), s) == H.HISPARSE_EINVAL
    assert lib.hisparse_step(hs.pool, step.data_ptr(), topk.data_ptr(), bad_q, 1.0, rows.data_ptr(),
                             counts.data_ptr(), out.data_ptr(), lse.data_ptr(), s) == H.HISPARSE_EINVAL
    assert lib.hisparse_append(hs.pool, q.data_ptr() + 4, s) == H.HISPARSE_EINVAL
    assert lib.hisparse_sparse_mla_decode(hs.pool, 0, q.data_ptr(), rows.data_ptr(), float("inf"), out.data_ptr(),
                                          lse.data_ptr(), s) == H.HISPARSE_EINVAL
    assert lib.hisparse_sparse_mla_decode(hs.pool, 1, q.data_ptr(), rows.data_ptr(), 1.0, out.data_ptr(),
                                          lse.data_ptr(), s) == H.HISPARSE_EINVAL  # layer out of range
    # nothing was enqueued: the state is still empty and no error bit is set
    owner, stamp = hs.export_state(0, 0)
    assert (owner == -1).all() and (stamp == -1).all()
    assert hs.check_errors() == 0
    hs.close()


def test_host_pool_limit_on_a_real_device():
    """A pool is created when its pinned pool fits the budget exactly, and
    refused with ENOMEM (nothing allocated, nothing left behind) when the
    budget is one byte short."""
    import torch

    w = named_workload("tiny")
    need = w.num_layers * sum(w.ctx_len) * 1152
    cfg = w.config_dict()
    cfg["host_pool_limit"] = need
    hs = H.HiSparse(cfg, "cuda:0")
    assert hs.pool
    hs.close()
    cfg["host_pool_limit"] = need - 1
    with pytest.raises(H.HiSparseError) as ei:
        H.HiSparse(cfg, "cuda:0")
    assert ei.value.status == H.HISPARSE_ENOMEM
    assert str(need) in H.hisparse_last_error()
    torch.cuda.synchronize()
