"""Pins of the FP8 E4M3 row format (CPU only).

* The oracle's E4M3 decoder against an independent implementation
  (PyTorch's float8_e4m3fn) for all 256 codes, and against values the OCP
  definition fixes by hand.
* The input generator's float32 -> E4M3 rounding against PyTorch's cast
  (nearest, ties to even), including every exact midpoint, and its C fill
  against its NumPy definition.
* Oracle exactness and hot-row invariants with FP8 rows (the decode path
  attends to decoded codes times the layer scale).
"""

import numpy as np
import pytest

from oracle.attention import attend_f64, bf16_bits_to_f64
from oracle.fp8 import e4m3_to_f64
from oracle.step import OracleDecoder, SimulatedKV, row_values
from tracegen import fill, make_workload, q_block, with_fp8
from tracegen.values import f32_to_e4m3_codes, kv_key, kv_rows

torch = pytest.importorskip("torch")


def test_e4m3_decoder_all_codes_against_torch():
    codes = np.arange(256, dtype=np.uint8)
    mine = e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert np.array_equal(mine[~nan], ref[~nan])


def test_e4m3_decoder_hand_values():
    # fields s eeee mmm: subnormals m * 2^-9, normals (1 + m/8) * 2^(e - 7)
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x38: 1.0, 0x39: 1.125,
             0x3F: 1.875, 0x40: 2.0, 0x7E: 448.0, 0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0, 0x77: 240.0}
    for c, v in table.items():
        got = e4m3_to_f64(np.array([c], np.uint8))[0]
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)


def test_encoder_matches_torch_cast_including_ties():
    rng = np.random.default_rng(3)
    vals = e4m3_to_f64(np.arange(127, dtype=np.uint8))  # 0 .. 448 ascending
    mids = ((vals[:-1] + vals[1:]) / 2).astype(np.float32)  # exact midpoints (ties)
    x = np.concatenate([rng.standard_normal(50000) * 60, rng.standard_normal(20000) * 1e-2,
                        rng.standard_normal(20000) * 1e-3, mids, -mids, [0.0, -0.0, 448.0, -448.0]])
    x = np.clip(x, -448, 448).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(f32_to_e4m3_codes(x), ref)


def test_encoder_saturates():
    x = np.array([449.0, 1e6, -500.0], np.float32)
    assert list(f32_to_e4m3_codes(x)) == [0x7E, 0x7E, 0xFE]


@pytest.mark.parametrize("scale", [2.0 ** -5, 0.0390625, 0.3])
def test_c_fill_matches_numpy_fp8(scale):
    fill.build(force=False)
    pos = np.arange(0, 9000, 13)
    a = fill.rows_fp8(kv_key(11, 2, 1), pos, 576, scale)
    b = kv_rows(11, 2, 1, pos, 576, fp8_scale=scale)
    assert np.array_equal(a, b)
    # the generated values stay finite and use the format's range
    v = e4m3_to_f64(b)
    assert np.isfinite(v).all() and np.abs(v).max() <= 448


def test_fp8_single_row_gives_scaled_row():
    # one valid row: O = x[:512] exactly, here x = decode(code) * scale
    codes = np.arange(256, dtype=np.uint8)
    codes = codes[(codes != 0x7F) & (codes != 0xFF)]
    row = np.resize(codes, 576).reshape(1, 576)
    scale = 0.0390625
    x = e4m3_to_f64(row) * scale
    q = bf16_bits_to_f64(np.full((4, 576), 0x3F80, np.uint16))  # q = 1
    o, lse = attend_f64(q, x, 0.01)
    assert np.array_equal(o, np.repeat(x[:, :512], 4, axis=0))
    assert np.allclose(lse, 0.01 * x.sum())


def test_fp8_exactness_and_hot_rows():
    w = with_fp8(make_workload("ex8", 6, 2, 2, 2, [700, 1500], 16, 64, 96, 8, 0.6, 0.8, "tail+half",
                               page_size=16))
    tr = w.trace()
    dec = OracleDecoder(w)
    kv = SimulatedKV(w)
    for t in range(w.steps):
        res, att = dec.step(t, tr[t])
        for (l, r), rr in res.items():
            kv.apply_fetches(l, r, rr.fetches, dec.hot_base(r))
            q = bf16_bits_to_f64(q_block(w.seed, t, l, r, w.num_heads))
            o2, lse2 = attend_f64(q, row_values(w, l, kv.gather(l, rr.rows)), w.scale)
            o1, lse1 = att[(l, r)]
            assert np.array_equal(o1, o2) and np.array_equal(lse1, lse2)
            st = dec.states[(l, r)]
            owned = [(s, p) for s, p in enumerate(st.owner) if p >= 0]
            host = kv_rows(w.seed, r, l, [p for _, p in owned], fp8_scale=w.fp8_scale(l))
            for i, (s, _) in enumerate(owned):
                assert (kv.rows[(l, dec.hot_base(r) + s)] == host[i]).all()


def test_fp8_rows_are_close_to_bf16_rows():
    # the FP8 pool stores the same underlying values to E4M3 precision:
    # |decode(code) * scale - v| <= 2^-4 |v| + 2^-10 * scale (half a quantum)
    from tracegen.values import float_values
    e = np.arange(576 * 50, dtype=np.uint64)
    for scale in (2.0 ** -5, 0.3):
        v = float_values(kv_key(3, 0, 0), e).astype(np.float64)
        x = e4m3_to_f64(kv_rows(3, 0, 0, np.arange(50), 576, fp8_scale=scale).reshape(-1)) * scale
        assert np.all(np.abs(x - v) <= 2.0 ** -4 * np.abs(v) + 2.0 ** -10 * scale * 1.0001)
