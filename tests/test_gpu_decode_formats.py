"""GPU parity of the decode's fast path and its exact fp32 fallback
against the fp64 oracle.

The fast path scores the bf16 rows and queries as given and multiplies P
(one fp16 plane) by the rows' V part converted to fp16, which is exact
below 2^16; a workgroup that meets a V value it cannot convert, or an inf
or NaN, computes its result again in fp32 on the values as given.  These
cases plant large values where they leave the exact result finite and of
ordinary size (a zero query weight on the planted dimension), so that a
result that used a converted value shows up as NaN or as a large error:

* row values of 70000 and -1e30 in a rope dimension, and a query value of
  70000: beyond fp16 but exact on the bf16 scores, so the fast path holds;
* a row value of 70000 in a V dimension: the fallback;
* the filler row that padding entries (-1) stage, holding 70000 in a V
  dimension: the fallback (its zero weight times inf would poison O);
* a later tile whose scores exceed the first tile's by more than 2^15
  (log2 units), which the fast path handles with a second pass.

Outputs start as NaN, so a workgroup that wrote nothing fails.  The count
of fallback workgroups is checked through hisparse_decode_fallback_count,
which clears it when read.
"""

import numpy as np
import pytest

from oracle.attention import attend
from tests.gpu_harness import LSE_TOL, O_TOL, log
from tracegen.values import f32_to_bf16_bits, kv_rows, q_block

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from host_offloaded_kv_amd import hisparse

    hisparse.load()


def _bits(x: float) -> np.uint16:
    return f32_to_bf16_bits(np.array([x], np.float32))[0]


def _run(R, H, K, n_rows, rows, q, sel, scale=1 / 24.0, seed=11):
    """Decode one layer on the GPU and compare every request with the oracle.

    rows: uint16 [n_rows, 576] bf16 bits (row ids index it); q: uint16
    [R, H, 576]; sel: int32 [R, K] (-1 = padding).  Returns the count of
    workgroups that took the fp32 fallback."""
    import torch

    from host_offloaded_kv_amd.hisparse import HiSparse

    cfg = dict(num_requests=R, num_layers=1, top_k=K, hot_slots=max(K, n_rows // R + 1), num_heads=H,
               ctx_len=[1] * R)
    hs = HiSparse(cfg, "cuda:0")
    assert hs.kv_rows >= n_rows
    dev = hs.device
    hs.kv[0][:n_rows] = torch.from_numpy(rows.view(np.int16)).to(dev).view(torch.bfloat16)
    d_q = torch.from_numpy(q.view(np.int16)).to(dev)
    d_sel = torch.from_numpy(sel).to(dev)
    out = torch.full((R, H, 512), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=dev)
    hs.decode(0, d_q, d_sel, scale, out, lse)
    torch.cuda.synchronize()
    fallbacks = hs.decode_fallback_count()
    assert hs.decode_fallback_count() == 0  # read and cleared
    assert hs.check_errors() == 0
    got_o, got_l = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    for r in range(R):
        valid = sel[r][sel[r] >= 0]
        o_ref, l_ref = attend(q[r], rows[valid], scale)
        err = np.abs(got_o[r] - o_ref).max() / np.abs(o_ref).max()
        lerr = np.abs(got_l[r] - l_ref).max()
        assert np.isfinite(err) and err <= O_TOL, f"request {r}: O rel err {err:.3e}"
        assert lerr <= LSE_TOL, f"request {r}: lse abs err {lerr:.3e}"
    hs.close()
    return fallbacks


def _inputs(R, H, K, n_rows, seed):
    rows = kv_rows(seed, 0, 0, np.arange(n_rows))
    q = np.stack([q_block(seed, 0, 0, r, H) for r in range(R)])
    rng = np.random.default_rng(seed)
    sel = np.stack([rng.permutation(n_rows)[:K] for _ in range(R)]).astype(np.int32)
    return rows, q, sel


@pytest.mark.parametrize("H", [16, 48, 64, 96, 128])  # head groups of 16, 16 x 3, 64, 32 x 3, 64 x 2
def test_in_range_inputs_stay_on_the_fast_path(H):
    R, K, n = 2, 100, 300
    rows, q, sel = _inputs(R, H, K, n, seed=21)
    log(f"decode formats: in range, H={H}")
    assert _run(R, H, K, n, rows, q, sel) == 0


@pytest.mark.parametrize("H", [64, 128])
def test_rope_values_beyond_fp16_stay_on_the_fast_path(H):
    R, K, n = 2, 100, 300
    rows, q, sel = _inputs(R, H, K, n, seed=22)
    d = 540  # a rope dimension: not part of V
    rows[sel[0][37], d] = _bits(70000.0)
    rows[sel[0][90], d] = _bits(-1.0e30)
    q[:, :, d] = 0  # the exact scores do not see it
    log(f"decode formats: rope values beyond fp16, H={H}")
    assert _run(R, H, K, n, rows, q, sel) == 0


@pytest.mark.parametrize("H", [64, 128])
def test_v_value_beyond_fp16_takes_the_fallback(H):
    R, K, n = 2, 100, 300
    rows, q, sel = _inputs(R, H, K, n, seed=27)
    d = 100  # a V dimension
    rows[sel[1][12], d] = _bits(70000.0)
    q[:, :, d] = 0  # the scores do not see it; O of request 1 does
    log(f"decode formats: V value beyond fp16, H={H}")
    assert _run(R, H, K, n, rows, q, sel) >= 1


def test_query_beyond_fp16_stays_on_the_fast_path():
    R, H, K, n = 2, 64, 96, 300
    rows, q, sel = _inputs(R, H, K, n, seed=23)
    d = 3
    rows[:, d] = 0  # the exact scores do not see the planted query value
    q[1, 5, d] = _bits(70000.0)  # head 5 of request 1
    log("decode formats: query beyond fp16")
    assert _run(R, H, K, n, rows, q, sel) == 0


def test_padding_filler_row_beyond_fp16_takes_the_fallback():
    """Entries of -1 stage row 0 as filler with zero weight; 0 * inf would
    poison O in fp16, so a filler row that does not fit sends the
    workgroup to the fallback too."""
    R, H, K, n = 1, 32, 64, 200
    rows, q, sel = _inputs(R, H, K, n, seed=24)
    sel[0] = np.random.default_rng(24).permutation(np.arange(1, n))[:K]  # row 0 only as filler
    sel[0][40:] = -1
    d = 7  # a V dimension
    rows[0, d] = _bits(70000.0)
    q[:, :, d] = 0
    log("decode formats: filler row beyond fp16")
    assert _run(R, H, K, n, rows, q, sel) >= 1


def test_late_tile_growth_takes_a_second_fp16_pass():
    """A row in the third tile is the sign pattern of head 0's query: head 0
    scores it about 25 log2 units above the first tile's maximum, beyond
    the 2^15 range of an fp16 weight, so the fast path repeats the range
    with the true maximum (no fallback)."""
    R, H, K, n = 1, 64, 128, 400
    rows, q, sel = _inputs(R, H, K, n, seed=25)
    q0 = (q[0, 0].astype(np.uint32) << 16).view(np.float32)
    rows[sel[0][70]] = f32_to_bf16_bits(np.sign(q0).astype(np.float32))
    x = (rows[sel[0]].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s0 = x @ q0.astype(np.float64) / 24.0 * np.log2(np.e)
    assert s0[70] - s0[:32].max() > 20  # the case is what it claims
    log("decode formats: late tile growth")
    assert _run(R, H, K, n, rows, q, sel) == 0


def test_fp8_rows_with_query_beyond_fp16_stay_on_the_fast_path():
    """FP8 rows always fit fp16, and the scores take the bf16 query as
    given, so a query value beyond fp16 stays on the fast path, which
    applies the layer scale to the scores and to O."""
    import torch

    from host_offloaded_kv_amd.hisparse import HiSparse
    from oracle.attention import attend_f64, bf16_bits_to_f64
    from oracle.fp8 import e4m3_to_f64
    from tracegen.values import fp8_values

    R, H, K, n, scale, kvs = 1, 64, 80, 160, 1 / 24.0, 0.25
    e = np.arange(n * 576, dtype=np.uint64).reshape(n, 576)
    codes = fp8_values(91, e, kvs)
    q = q_block(26, 0, 0, 0, H)[None]
    d = 9
    codes[:, d] = 0  # code 0 is +0: the exact scores do not see the planted query value
    q[0, 3, d] = _bits(70000.0)
    sel = np.random.default_rng(26).permutation(n)[:K].astype(np.int32)[None]
    cfg = dict(num_requests=R, num_layers=1, top_k=K, hot_slots=n, num_heads=H, ctx_len=[1],
               kv_dtype="fp8", kv_scale=[kvs])
    hs = HiSparse(cfg, "cuda:0")
    dev = hs.device
    hs.kv[0][:n] = torch.from_numpy(codes).to(dev)
    out = torch.full((R, H, 512), float("nan"), dtype=torch.float32, device=dev)
    lse = torch.full((R, H), float("nan"), dtype=torch.float32, device=dev)
    log("decode formats: fp8 rows, query beyond fp16")
    hs.decode(0, torch.from_numpy(q.view(np.int16)).to(dev), torch.from_numpy(sel).to(dev), scale, out, lse)
    torch.cuda.synchronize()
    assert hs.decode_fallback_count() == 0
    assert hs.check_errors() == 0
    x = e4m3_to_f64(codes[sel[0]]) * kvs
    o_ref, l_ref = attend_f64(bf16_bits_to_f64(q[0]), x, scale)
    got_o, got_l = out.cpu().numpy()[0].astype(np.float64), lse.cpu().numpy()[0].astype(np.float64)
    err = np.abs(got_o - o_ref).max() / np.abs(o_ref).max()
    assert np.isfinite(err) and err <= O_TOL, f"O rel err {err:.3e}"
    assert np.abs(got_l - l_ref).max() <= LSE_TOL
    hs.close()


def test_key_splits_with_empty_and_padded_ranges():
    """One request, 64 heads, K = 300: the launch splits K over many
    workgroups; whole splits hold only padding (-1) and the last tile is
    ragged, so combine_splits meets empty partials."""
    R, H, K, n = 1, 64, 300, 400
    rows, q, sel = _inputs(R, H, K, n, seed=27)
    sel[0][32:128] = -1   # three whole 32-row tiles of padding
    sel[0][290:] = -1
    log("decode formats: key splits with empty ranges")
    assert _run(R, H, K, n, rows, q, sel) == 0
