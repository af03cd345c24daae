"""GPU parity of the two-part decode of an index-share group's last layer
(resident_first of hisparse_set_pipeline, with separate fetches; the
fetch in the decode is switched off here): the entries whose rows were in
place before the layer's fetch are decoded beside the fetches, the entries
the fetch fills after it, and the two parts' partial softmax sums are
merged.  Attention over a set of keys is the same for any partition of the
set (HiSparse summary article, section 02: the outputs are those of
attention over the selected keys wherever their rows live), so the results
are checked against the oracle like every other step.

Two shapes of the merge: with fewer than 32 (request, head group)
workgroups the part after the fetch is split by keys and combine_splits
merges every part's partials; with 32 or more, it runs unsplit and merges
the first part's partials in its own epilogue.  A value beyond fp16 in a V
dimension (with a zero query weight on it, so that the exact result stays
ordinary) sends either part to the exact fp32 path, which merges the same
way.
"""

import ctypes

import numpy as np
import pytest

from oracle.attention import attend
from tests.gpu_harness import LSE_TOL, O_TOL, GpuRun, log, make_pool, run_and_compare
from tracegen import fill
from tracegen.populate import queries
from tracegen.values import f32_to_bf16_bits
from tracegen.workloads import make_workload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()
    fill.build(force=False)


def _force_two_part(hs):
    hs.set_pipeline(resident_first=1, fetch_in_decode=-1)


@pytest.mark.parametrize("variant", ["split_and_combine", "merge_in_second_part"])
def test_two_part_last_layer_matches_oracle(variant):
    if variant == "split_and_combine":
        # 4 requests x 1 head group of 32: the second part is split by keys
        w = make_workload("two_part_small", 71, 4, 4, 2, [20000, 9000, 33000, 4096], 32, 256, 512, 8, 0.7, 0.8,
                          "tail")
    else:
        # 32 requests x 1 head group of 64: one workgroup each, merging in its epilogue
        w = make_workload("two_part_r32", 72, 32, 2, 2, [3000 + 97 * r for r in range(32)], 64, 128, 256, 6, 0.7,
                          0.8, "tail+half")
    run_and_compare(w, label=f"two-part {variant}", setup=_force_two_part, bytes_pairs=[(w.num_layers - 1, 0)])


def test_two_part_off_matches_on():
    """The same steps with the last layer decoded in one launch after its
    fetch: rows and counts bit for bit, O and lse within the oracle bound."""
    w = make_workload("two_part_ab", 73, 32, 1, 1, [2500 + 31 * r for r in range(32)], 64, 128, 256, 5, 0.7, 0.8,
                      "tail")
    tr = w.trace(w.steps)
    snaps = {}
    for mode in (1, -1):
        hs = make_pool(w)
        hs.set_pipeline(resident_first=mode, fetch_in_decode=-1)
        run = GpuRun(w, hs)
        snaps[mode] = []
        for t in range(w.steps):
            rows, counts = run.step(t, tr[t])
            snaps[mode].append((rows, counts, run.out.cpu().numpy().astype(np.float64), run.lse.cpu().numpy()))
        assert hs.check_errors() == 0
        hs.close()
    for t, (a, b) in enumerate(zip(snaps[1], snaps[-1])):
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1]), f"rows/counts differ at step {t}"
        for r in range(w.num_requests):
            den = np.abs(b[2][0, r]).max()
            assert np.abs(a[2][0, r] - b[2][0, r]).max() / den <= O_TOL, f"O differs at step {t} r={r}"
            assert np.abs(a[3][0, r].astype(np.float64) - b[3][0, r]).max() <= LSE_TOL, f"lse step {t} r={r}"


@pytest.mark.parametrize("n_requests", [4, 32])
def test_two_part_fallback_merges(n_requests):
    """A V value of 70000 in the host row of one position of request 0: in
    step 0 the position misses (the part after the fetch meets it), in step 1
    it hits (the part beside the fetches meets it); both take the exact path
    and merge.  Reference: fp64 attention over the rows the device holds
    under the returned row ids, with the queries given."""
    import torch

    from host_offloaded_kv_amd.hisparse import HiSparse  # noqa: F401  (loaded by the fixture)

    w = make_workload(f"two_part_fb{n_requests}", 74, n_requests, 1, 1, [4096] * n_requests, 64, 128, 256, 2, 0.7,
                      0.8, "tail")
    tr = w.trace(2).copy()
    sel0, sel1 = tr[0][0][0], tr[1][0][0]
    pos = next(p for p in range(64, 4000) if p not in sel0 and p not in sel1)
    sel0[0] = pos  # (the lists may lose their ascending order: any order is accepted)
    sel1[0] = pos
    hs = make_pool(w)
    hs.set_pipeline(resident_first=1, fetch_in_decode=-1)
    dim = 5
    host = hs.host_rows_ptr(0, 0) + pos * 576 * 2 + dim * 2
    ctypes.c_uint16.from_address(host).value = int(f32_to_bf16_bits(np.array([70000.0], np.float32))[0])
    run = GpuRun(w, hs)
    for t in range(2):
        q = queries(w, t)
        q[:, :, :, dim] = 0  # the planted dimension does not move the scores
        dev = hs.device
        run.d_step.fill_(t)
        topk = torch.from_numpy(np.ascontiguousarray(tr[t], dtype=np.int32)).to(dev)
        hs.step(run.d_step, topk, torch.from_numpy(q.view(np.int16)).to(dev), w.scale, run.rows, run.counts, run.out,
                run.lse)
        torch.cuda.synchronize(dev)
        fallbacks = hs.decode_fallback_count()
        assert fallbacks >= 1, f"step {t}: no workgroup took the exact path"
        rows = run.rows.cpu().numpy()
        out, lse = run.out.cpu().numpy().astype(np.float64), run.lse.cpu().numpy().astype(np.float64)
        for r in (0, n_requests - 1):
            ids = rows[0, r][rows[0, r] >= 0]
            x = hs.kv[0][torch.from_numpy(ids.astype(np.int64)).to(dev)].view(torch.int16).cpu().numpy()
            o_ref, l_ref = attend(q[0, r], x.view(np.uint16), w.scale)
            err = np.abs(out[0, r] - o_ref).max() / np.abs(o_ref).max()
            assert np.isfinite(err) and err <= O_TOL, f"step {t} r={r}: O rel err {err:.3e}"
            assert np.abs(lse[0, r] - l_ref).max() <= LSE_TOL, f"step {t} r={r}: lse"
        c = run.counts.cpu().numpy()[0, 0]
        log(f"fallback merge R={n_requests} step {t}: {fallbacks} exact workgroups, request 0 counts {tuple(c)}")
    assert hs.check_errors() == 0
    hs.close()
