"""GPU checks of the measurement helpers: the row gather and the stream copy
move bytes exactly (pinned host source and device source)."""

import ctypes

import numpy as np
import pytest

from tests.gpu_harness import log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()


@pytest.mark.parametrize("row_bytes", [16, 576, 1152])
def test_row_gather_is_exact(row_bytes):
    import torch

    from host_offloaded_kv_amd import hisparse as H

    dev = torch.device("cuda:0")
    n_src, n_rows = 3000, 2500
    nbytes = n_src * row_bytes
    rng = np.random.default_rng(row_bytes)
    src = rng.integers(0, 256, nbytes, dtype=np.uint8)
    rows = rng.integers(0, n_src, n_rows).astype(np.int64)
    want = src.reshape(n_src, row_bytes)[rows]
    h, d = H.hisparse_host_alloc(nbytes, 0)
    try:
        ctypes.memmove(h, src.ctypes.data, nbytes)
        d_rows = torch.from_numpy(rows).to(dev)
        dst = torch.zeros(n_rows * row_bytes, dtype=torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev).cuda_stream
        log(f"row gather: {n_rows} rows of {row_bytes} B from pinned host memory")
        H.hisparse_row_gather(dst.data_ptr(), d, d_rows.data_ptr(), n_rows, row_bytes, stream)
        torch.cuda.synchronize(dev)
        assert np.array_equal(dst.cpu().numpy().reshape(n_rows, row_bytes), want)
        # the same from device memory, and the stream copy of the whole source
        d_src = torch.from_numpy(src).to(dev)
        dst.zero_()
        H.hisparse_row_gather(dst.data_ptr(), d_src.data_ptr(), d_rows.data_ptr(), n_rows, row_bytes, stream)
        copy = torch.zeros(nbytes, dtype=torch.uint8, device=dev)
        H.hisparse_stream_copy(copy.data_ptr(), d, nbytes, stream)
        torch.cuda.synchronize(dev)
        assert np.array_equal(dst.cpu().numpy().reshape(n_rows, row_bytes), want)
        assert np.array_equal(copy.cpu().numpy(), src)
    finally:
        H.hisparse_host_free(h)
