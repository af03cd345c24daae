"""GPU parity of the fetch in the decode (fetch_in_decode of
hisparse_set_pipeline, the default of hisparse_step): one decode launch per
index-share group reads the rows the step fills straight from the pinned
host pool into its tiles, and the workgroups of head group 0 write them to
their hot rows.

Checked against the oracle (rows, counts, LRU state and every hot row's
bytes bit for bit, attention within the bound) and against the same steps
with separate miss fetches, including a request with two head groups (both
read the row from the host pool, one writes it) and FP8 rows.  A value
beyond fp16 planted in a host row sends the workgroup that reads it to the
exact fp32 path, which reads the row from the host pool as well; a step
later the row is a hit and is read from the hot row the decode wrote.  Both
pipelines also run on a host pool in coherent pinned memory.
"""

import ctypes

import numpy as np
import pytest

from oracle.attention import attend
from tests.gpu_harness import LSE_TOL, O_TOL, GpuRun, log, make_pool, run_and_compare
from tracegen import fill
from tracegen.populate import queries
from tracegen.values import f32_to_bf16_bits
from tracegen.workloads import make_workload, with_fp8

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _workload(kind):
    if kind == "two_head_groups":
        # 128 heads: two 64-head workgroups per request read each filled row
        return make_workload("fid_h128", 81, 4, 2, 2, [9000, 20000, 4096, 15000], 128, 256, 512, 6, 0.7, 0.8, "tail")
    w = make_workload("fid_grouped", 82, 4, 6, 3, [20000, 9000, 33000, 4096], 32, 512, 1024, 6, 0.7, 0.8,
                      "tail+half")
    return with_fp8(w) if kind == "fp8" else w


@pytest.mark.parametrize("kind", ["grouped", "two_head_groups", "fp8"])
def test_fetch_in_decode_matches_oracle_and_separate_fetches(kind):
    import torch

    w = _workload(kind)
    pairs = [(l, r) for l in range(w.num_layers) for r in range(w.num_requests)]
    hs, run, _ = run_and_compare(w, label=f"fetch in decode, {kind}", bytes_pairs=pairs)
    fused = (run.rows.cpu().numpy(), run.counts.cpu().numpy(), run.out.cpu().numpy().astype(np.float64),
             run.lse.cpu().numpy().astype(np.float64))
    hot_fused = [hs.kv[l].view(torch.uint8).cpu().numpy() for l in range(w.num_layers)]
    hs.close()

    hs = make_pool(w)
    hs.set_pipeline(fetch_in_decode=-1)
    run = GpuRun(w, hs)
    tr = w.trace(w.steps)
    for t in range(w.steps):
        run.step(t, tr[t])
    sep = (run.rows.cpu().numpy(), run.counts.cpu().numpy(), run.out.cpu().numpy().astype(np.float64),
           run.lse.cpu().numpy().astype(np.float64))
    assert np.array_equal(fused[0], sep[0]) and np.array_equal(fused[1], sep[1])
    for l in range(w.num_layers):
        assert np.array_equal(hot_fused[l], hs.kv[l].view(torch.uint8).cpu().numpy()), f"KV tensor of layer {l}"
        for r in range(w.num_requests):
            den = np.abs(sep[2][l, r]).max()
            assert np.abs(fused[2][l, r] - sep[2][l, r]).max() / den <= O_TOL
            assert np.abs(fused[3][l, r] - sep[3][l, r]).max() <= LSE_TOL
    assert hs.check_errors() == 0
    hs.close()


@pytest.mark.parametrize("pipeline", ["fetch_in_decode", "separate_fetches"])
def test_coherent_host_pool(pipeline):
    """The host pool in coherent pinned memory (host_coherent = 1): reads
    of it are not cached on the device, so both head groups of a request
    read a filled row over the link; the results are the same."""
    w = _workload("two_head_groups")
    setup = None if pipeline == "fetch_in_decode" else (lambda hs: hs.set_pipeline(fetch_in_decode=-1))
    pairs = [(l, r) for l in range(w.num_layers) for r in range(w.num_requests)]
    hs, _, _ = run_and_compare(w, label=f"coherent host pool, {pipeline}", bytes_pairs=pairs, setup=setup,
                               host_coherent=1)
    hs.close()


@pytest.mark.parametrize("heads", [64, 128])
def test_fetch_in_decode_exact_path_reads_host_rows(heads):
    """A V value of 70000 (zero query weight on its dimension) in the host
    row of a position request 0 selects in steps 0 and 1: a miss read from
    the host pool in step 0, a hit read from the hot row the decode wrote in
    step 1; the exact path runs both times.  Reference: fp64 attention over
    the host pool's rows of the selected positions (as planted)."""
    import torch

    R = 4
    w = make_workload(f"fid_fb{heads}", 83, R, 1, 1, [4096] * R, heads, 128, 256, 2, 0.7, 0.8, "none")
    tr = w.trace(2).copy()
    sel0, sel1 = tr[0][0][0], tr[1][0][0]
    pos = next(p for p in range(64, 4000) if p not in sel0 and p not in sel1)
    sel0[0] = pos
    sel1[0] = pos
    hs = make_pool(w)
    dim = 5
    base = hs.host_rows_ptr(0, 0)
    ctypes.c_uint16.from_address(base + pos * 576 * 2 + dim * 2).value = int(
        f32_to_bf16_bits(np.array([70000.0], np.float32))[0])
    run = GpuRun(w, hs)
    dev = hs.device
    for t in range(2):
        q = queries(w, t)
        q[:, :, :, dim] = 0
        run.d_step.fill_(t)
        topk = torch.from_numpy(np.ascontiguousarray(tr[t], dtype=np.int32)).to(dev)
        hs.step(run.d_step, topk, torch.from_numpy(q.view(np.int16)).to(dev), w.scale, run.rows, run.counts, run.out,
                run.lse)
        torch.cuda.synchronize(dev)
        fallbacks = hs.decode_fallback_count()
        assert fallbacks >= 1, f"step {t}: no workgroup took the exact path"
        out, lse = run.out.cpu().numpy().astype(np.float64), run.lse.cpu().numpy().astype(np.float64)
        for r in (0, R - 1):
            sel = np.array([p for p in tr[t][0][r] if p >= 0], np.int64)
            n = 576
            host = np.ctypeslib.as_array(
                (ctypes.c_uint16 * ((int(sel.max()) + 1) * n)).from_address(hs.host_rows_ptr(r, 0)))
            x = host.reshape(-1, n)[sel]
            o_ref, l_ref = attend(q[0, r], x, w.scale)
            err = np.abs(out[0, r] - o_ref).max() / np.abs(o_ref).max()
            assert np.isfinite(err) and err <= O_TOL, f"step {t} r={r}: O rel err {err:.3e}"
            assert np.abs(lse[0, r] - l_ref).max() <= LSE_TOL, f"step {t} r={r}: lse"
        log(f"fetch in decode, H={heads}, step {t}: {fallbacks} exact workgroups, "
            f"request 0 counts {tuple(run.counts.cpu().numpy()[0, 0])}")
    assert hs.check_errors() == 0
    hs.close()
