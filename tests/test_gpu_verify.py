"""GPU parity of multi-token verification (num_verify = T > 1): one RESOLVE
over the T verify tokens' selections per (request, layer), then decode of
every (request, token) with its own query.

Bit-exact: row ids of every entry (copies across tokens share a row),
counts over distinct positions, LRU state and hot-row bytes; attention per
token within the usual bound.  The small configurations run both step
pipelines: the decode that reads the filled rows from the host pool (an
entry of a later token that shares a filled row reads it there too) and
separate miss fetches.
"""

import numpy as np
import pytest

from tests.gpu_harness import LSE_TOL, O_TOL, check_hot_bytes, check_state, log, make_pool
from oracle.step import OracleDecoder
from tracegen import fill, make_workload, named_workload, with_fp8
from tracegen.populate import queries

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _run(w, steps, attend_every=1, attend_pairs=None, dup_step=None, fetch_in_decode=1):
    import torch

    T, L, R, K, H = w.num_verify, w.num_layers, w.num_requests, w.top_k, w.num_heads
    tr = w.trace(steps)  # [steps][G][R][T][K]
    if dup_step is not None:
        tr[dup_step, 0, 0, T - 1, 1] = tr[dup_step, 0, 0, T - 1, 0]  # a repeat inside one token's list
    hs = make_pool(w)
    hs.set_pipeline(fetch_in_decode=fetch_in_decode)
    dev = hs.device
    rows = torch.empty((L, R, T, K), dtype=torch.int32, device=dev)
    counts = torch.empty((L, R, 3), dtype=torch.int32, device=dev)
    out = torch.empty((L, R, T, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((L, R, T, H), dtype=torch.float32, device=dev)
    d_step = torch.zeros(1, dtype=torch.int32, device=dev)
    dec = OracleDecoder(w)
    pairs = [(l, r) for l in range(L) for r in range(R)]
    worst = 0.0
    for t in range(steps):
        d_step.fill_(t)
        topk = torch.from_numpy(np.ascontiguousarray(tr[t])).to(dev)
        q = torch.from_numpy(queries(w, t).view(np.int16)).to(dev)
        hs.step(d_step, topk, q, w.scale, rows, counts, out, lse)
        torch.cuda.synchronize(dev)
        g_rows, g_counts = rows.cpu().numpy(), counts.cpu().numpy()
        res = dec.resolve_step(t, tr[t])
        for (l, r), rr in res.items():
            assert np.array_equal(g_rows[l, r].reshape(-1), np.asarray(rr.rows, np.int32)), f"rows t={t} l={l} r={r}"
            assert tuple(int(x) for x in g_counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), \
                f"counts t={t} l={l} r={r}"
        check_state(hs, dec, pairs, t)
        check_hot_bytes(hs, w, dec, pairs, t)
        if t % attend_every == 0 or t == steps - 1:
            g_out, g_lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
            for (l, r) in (attend_pairs or pairs):
                g = l // w.index_share
                for i in range(T):
                    o_ref, lse_ref = dec.attend_one(t, l, r, tr[t][g][r][i], token=i)
                    err = np.abs(g_out[l, r, i] - o_ref).max() / np.abs(o_ref).max()
                    worst = max(worst, err)
                    assert err <= O_TOL, f"O t={t} l={l} r={r} token={i} err {err:.3e}"
                    assert np.abs(g_lse[l, r, i] - lse_ref).max() <= LSE_TOL
    flags = hs.check_errors()
    hs.close()
    log(f"{w.name}: T={T} {steps} steps ok, worst O rel err {worst:.3e}, flags {flags:#x}")
    return flags


@pytest.mark.parametrize("pipeline", [1, -1], ids=["fetch_in_decode", "separate_fetches"])
@pytest.mark.parametrize("case", range(4))
def test_verify_small_configs(case, pipeline):
    rng = np.random.default_rng(900 + case)
    T = int(rng.choice([2, 3, 4]))
    K = int(rng.choice([16, 50, 128]))
    B = T * K + int(rng.integers(0, K + 1))
    R, L = int(rng.integers(1, 4)), int(rng.choice([1, 2, 4]))
    share = int(rng.choice([s for s in (1, 2, 4) if L % s == 0]))
    ctx = [int(rng.integers(T * K, 8 * T * K)) for _ in range(R)]
    w = make_workload(f"verify{case}", 950 + case, R, L, share, ctx, 16 * int(rng.integers(1, 5)), K, B, 8,
                      float(rng.choice([0.5, 0.8])), 0.8, str(rng.choice(["none", "tail", "tail+half"])),
                      page_size=int(rng.choice([16, 64])))
    w.num_verify = T
    if case == 3:
        w = with_fp8(w)
    log(f"verify config {case}: T={T} R={R} L={L} g={share} K={K} B={B} ctx={ctx} res={w.residency} {w.kv_dtype}")
    flags = _run(w, w.steps, dup_step=3 if case == 1 else None, fetch_in_decode=pipeline)
    from host_offloaded_kv_amd.hisparse import HISPARSE_ERR_DUP

    assert flags == (HISPARSE_ERR_DUP if case == 1 else 0)


@pytest.mark.parametrize("pipeline", [1, -1], ids=["fetch_in_decode", "separate_fetches"])
def test_verify_tokens_off_word_boundaries(pipeline):
    """K = 50 with 3 tokens: each token's entries start inside a 64-bit word
    of the fill mask; index sharing over 2 layers, 16 heads, contexts a few
    times the width, resident tail pages."""
    w = make_workload("verify_k50", 977, 2, 2, 2, [700, 1300], 16, 50, 200, 6, 0.6, 0.8, "tail", page_size=16)
    w.num_verify = 3
    assert _run(w, w.steps, fetch_in_decode=pipeline) == 0


def test_verify_mtp1_r8_ctx32k():
    """One speculative token on the 8 x 32K workload: T*K = 4096 = B."""
    w = named_workload("r8_ctx32k")
    w.num_verify = 2
    w.name = "r8_ctx32k_mtp1"
    assert _run(w, 8, attend_every=3, attend_pairs=[(0, 0), (0, 5)]) == 0


def test_verify_mtp3_r8_ctx32k():
    """Three speculative tokens (MTP3, the blog's benchmark setting) on the
    8 x 32K workload at its top-K of 2048: one RESOLVE over T*K = 8192
    entries per (request, layer) into a buffer of (T + 1) * K = 10240 slots,
    the blog's (num_speculative_tokens + 2) x top-K sizing."""
    w = named_workload("r8_ctx32k")
    w.num_verify = 4
    w.hot_slots = (w.num_verify + 1) * w.top_k
    w.name = "r8_ctx32k_mtp3"
    assert _run(w, 6, attend_every=2, attend_pairs=[(0, 0), (0, 6)]) == 0


def test_random_policy_refused_where_its_sort_does_not_fit():
    """Random replacement sorts B keys in LDS beside the miss list; at T*K =
    8192 and B = 10240 that does not fit, and the pool says so."""
    from host_offloaded_kv_amd import hisparse as H

    w = make_workload("mtp3_small", 5, 1, 1, 1, [16384], 16, 2048, 10240, 2, 0.7, 0.8, "none")
    w.num_verify = 4
    hs = make_pool(w)
    with pytest.raises(H.HiSparseError) as ei:
        hs.set_replacement("random", 1)
    assert ei.value.status == H.HISPARSE_EDEVICE and "LDS" in H.hisparse_last_error()
    hs.set_replacement("fifo", 0)  # the order-array policies fit
    hs.close()
