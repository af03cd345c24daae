"""GPU parity with FP8 E4M3 KV rows (host pool, hot rows and resident pages
hold 576 one-byte codes; each layer has a scale).

Bit-exact: row ids, counts, LRU state, hot-row bytes.  Attention within the
same bound as bf16 rows, against the oracle's decoded codes times the scale.
The single-row test checks the kernel's E4M3 widening for every finite code
bit for bit.
"""

import numpy as np
import pytest

from tests.gpu_harness import GpuRun, check_attention, check_hot_bytes, check_state, log, make_pool, run_and_compare
from oracle.fp8 import e4m3_to_f64
from oracle.step import OracleDecoder
from tracegen import fill, make_workload, named_workload, with_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


@pytest.mark.parametrize("kv_scale", [0.0390625, 0.3])
def test_fp8_single_row_widening_exact(kv_scale):
    """One valid row: O = decode(code)[:512] * scale, exactly, for all codes."""
    import torch

    from host_offloaded_kv_amd.hisparse import HiSparse

    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]  # the two NaN codes
    rows = np.stack([np.resize(codes, 576), np.resize(codes[::-1], 576)])  # every finite code in both halves
    cfg = dict(num_requests=2, num_layers=1, top_k=1, hot_slots=1, num_heads=16, ctx_len=[1, 1],
               kv_dtype="fp8", kv_scale=[kv_scale])
    hs = HiSparse(cfg, "cuda:0")
    dev = hs.device
    hs.kv[0][:2] = torch.from_numpy(rows).to(dev)
    q = torch.full((2, 16, 576), 0.001, dtype=torch.bfloat16, device=dev)
    d_rows = torch.tensor([[0], [1]], dtype=torch.int32, device=dev)
    out = torch.empty((2, 16, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((2, 16), dtype=torch.float32, device=dev)
    log(f"fp8 single-row decode, scale {kv_scale}")
    hs.decode(0, q, d_rows, 0.5, out, lse)
    torch.cuda.synchronize()
    want = (e4m3_to_f64(rows[:, :512]).astype(np.float32) * np.float32(kv_scale)).astype(np.float32)
    got = out.cpu().numpy()
    for r in range(2):
        assert np.array_equal(got[r], np.repeat(want[r][None], 16, axis=0)), f"request {r}"
    assert hs.check_errors() == 0
    hs.close()


def test_fp8_tiny_every_step():
    w = with_fp8(named_workload("tiny"))
    hs, _, _ = run_and_compare(w, bytes_pairs=[(0, 0)], label="tiny_fp8")
    hs.close()


def test_fp8_r8_ctx32k():
    w = with_fp8(named_workload("r8_ctx32k"))
    hs, _, _ = run_and_compare(w, steps=12, attend_every=3, bytes_pairs=[(0, 0), (0, 7)], label="r8_ctx32k_fp8")
    hs.close()


@pytest.mark.parametrize("case", range(3))
def test_fp8_random_small_configs(case):
    rng = np.random.default_rng(500 + case)
    page = int(rng.choice([8, 64]))
    K = int(rng.choice([33, 64, 200]))
    B = K + int(rng.integers(0, 2 * K + 1))
    R, L = int(rng.integers(1, 4)), int(rng.choice([2, 4]))
    share = int(rng.choice([s for s in (1, 2, 4) if L % s == 0]))
    ctx = [int(rng.integers(K, 6 * K + 50)) for _ in range(R)]
    w = with_fp8(make_workload(f"rand_fp8_{case}", 600 + case, R, L, share, ctx, 16 * int(rng.integers(1, 5)), K,
                               B, 10, float(rng.choice([0.0, 0.6])), 0.8,
                               str(rng.choice(["none", "tail", "tail+half"])), page_size=page))
    log(f"fp8 random config {case}: R={R} L={L} g={share} K={K} B={B} H={w.num_heads} page={page} ctx={ctx}")
    pairs = [(l, r) for l in range(L) for r in range(R)]
    hs, _, _ = run_and_compare(w, bytes_pairs=pairs, label=w.name)
    hs.close()
