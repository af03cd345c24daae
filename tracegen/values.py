"""Counter-based synthetic values for KV latent rows and query vectors.

Input generation only: nothing here computes any part of the decode path.
Both the HIP path's tests/bench and the CPU oracle draw their inputs from
here, so any row of the host pool can be regenerated on demand without
holding the pool.

Definition (the same in the NumPy code below and in ``fill.c``):

* ``mix64(z)`` is the output function of the SplitMix64 generator
  (Steele, Lea & Flood, "Fast splittable pseudorandom number generators",
  OOPSLA 2014): ``z ^= z >> 30; z *= 0xBF58476D1CE4E5B9; z ^= z >> 27;
  z *= 0x94D049BB133111EB; z ^= z >> 31`` on 64-bit words.
* A stream key is folded from a tuple of words:
  ``k = 0; for w in words: k = mix64((k ^ w) + GOLDEN)``.
* Element ``e`` of the stream with key ``k`` uses the three words
  ``w_i = mix64(k + (3e + i + 1) * GOLDEN)`` for ``i = 0, 1, 2`` (the
  3e-th..3e+2-th outputs of a SplitMix64 generator seeded with ``k``).
* Their twelve 16-bit fields are summed: ``S = sum(c_j)``, and the value is
  ``(S - 393210) / 65536``: the classic sum-of-twelve-uniforms approximation
  of a standard normal (each ``(c_j + 0.5) / 65536`` is uniform on (0,1), so
  the sum minus 6 has mean 0 and variance ~1).  Every step is integer or
  exact, so the float32 value is identical on any machine and in any
  language.
* That float32 is rounded to bfloat16 with round-to-nearest-even.  For
  FP8 pools the float32 is first divided by the layer's scale (float32
  division) and rounded to an OCP FP8 E4M3 code, nearest with ties to the
  even code.

KV element (seed, request r, layer l, position p, dim d) uses stream words
``(seed, TAG_KV, r, l)`` and element index ``p * dim + d``.  Query element
(seed, step t, layer l, request r, head h, dim d) uses
``(seed, TAG_Q, t, l, r)`` and element index ``h * dim + d``.
"""

from __future__ import annotations

import numpy as np

MASK64 = (1 << 64) - 1
GOLDEN = 0x9E3779B97F4A7C15
MIX_C1 = 0xBF58476D1CE4E5B9
MIX_C2 = 0x94D049BB133111EB
TAG_KV = 0x4B56_524F_5753  # "KVROWS"
TAG_Q = 0x5155_4552_59  # "QUERY"
SUM_OFFSET = 393210  # sum((c+0.5)/65536) - 6 == (S + 6 - 6*65536) / 65536


def mix64_int(z: int) -> int:
    """SplitMix64 output function on a Python int (64-bit wrap)."""
    z &= MASK64
    z = ((z ^ (z >> 30)) * MIX_C1) & MASK64
    z = ((z ^ (z >> 27)) * MIX_C2) & MASK64
    return z ^ (z >> 31)


def stream_key(*words: int) -> int:
    """Fold a tuple of non-negative words into one 64-bit stream key."""
    k = 0
    for w in words:
        if w < 0:
            raise ValueError("stream words must be non-negative")
        k = mix64_int(((k ^ (w & MASK64)) + GOLDEN) & MASK64)
    return k


def kv_key(seed: int, r: int, l: int) -> int:
    return stream_key(seed, TAG_KV, r, l)


def q_key(seed: int, t: int, l: int, r: int) -> int:
    return stream_key(seed, TAG_Q, t, l, r)


def _mix64_np(z: np.ndarray) -> np.ndarray:
    z = (z ^ (z >> np.uint64(30))) * np.uint64(MIX_C1)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(MIX_C2)
    return z ^ (z >> np.uint64(31))


def float_values(key: int, elems: np.ndarray) -> np.ndarray:
    """float32 values (exact, before bf16 rounding) of the given elements."""
    e = np.asarray(elems, dtype=np.uint64)
    k = np.uint64(key)
    s = np.zeros(e.shape, dtype=np.int64)
    with np.errstate(over="ignore"):
        for i in range(3):
            n = e * np.uint64(3) + np.uint64(i + 1)
            w = _mix64_np(k + n * np.uint64(GOLDEN))
            for c in range(4):
                s += ((w >> np.uint64(16 * c)) & np.uint64(0xFFFF)).astype(np.int64)
    return (s - SUM_OFFSET).astype(np.float32) / np.float32(65536.0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest-even); returns uint16 bit patterns.

    Inputs here are always finite, so no NaN handling is needed.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    bias = np.uint64(0x7FFF) + ((b >> np.uint64(16)) & np.uint64(1))
    return ((b + bias) >> np.uint64(16)).astype(np.uint16)


def bf16_values(key: int, elems: np.ndarray) -> np.ndarray:
    return f32_to_bf16_bits(float_values(key, elems))


def f32_to_e4m3_codes(x: np.ndarray) -> np.ndarray:
    """Round float32 to OCP FP8 E4M3 codes (nearest, ties to the even code;
    magnitudes past 448 saturate to 448).  Returns uint8 codes.

    Works on the float32 bit fields: a normal E4M3 keeps the top 3 stored
    mantissa bits of float32 (exponent -6..8, bias 7); below 2^-6 the code
    counts multiples of 2^-9 (subnormals).  Either way the kept bits are the
    float32 significand (with its leading 1) shifted right, and the dropped
    bits decide the rounding.
    """
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.int64)
    sign = ((b >> 31) & 1).astype(np.uint8) << np.uint8(7)
    e32 = (b >> 23) & 0xFF
    sig = np.where(e32 > 0, (b & 0x7FFFFF) | (1 << 23), 0)  # float32 subnormals are far below 2^-10: -> 0
    E = e32 - 127
    # value = sig * 2^(E - 23); in units of the target quantum 2^(max(E, -6) - 3):
    qexp = np.maximum(E, -6) - 3
    shift = np.clip(qexp - (E - 23), 0, 62)  # >= 20 for normals, more for subnormals
    q = sig >> shift
    rem = sig - (q << shift)
    half = np.where(shift > 0, np.int64(1) << np.maximum(shift - 1, 0), 0)
    up = (rem > half) | ((rem == half) & (shift > 0) & ((q & 1) == 1))
    q = q + up.astype(np.int64)
    # assemble: q counts quanta 2^qexp; for E >= -6, q in [8, 16] (16 = carry into the next binade)
    mag = np.where(E >= -6, ((np.maximum(E, -6) + 7) << 3) + (q - 8), q)  # subnormal/min-normal: code = q
    mag = np.where(e32 == 0, 0, mag)
    mag = np.minimum(mag, 0x7E)  # saturate at 448
    return (sign | mag.astype(np.uint8)).astype(np.uint8)


def fp8_values(key: int, elems: np.ndarray, scale: float) -> np.ndarray:
    """FP8 E4M3 codes of the stream's values divided by ``scale`` (float32)."""
    v = float_values(key, elems) / np.float32(scale)
    return f32_to_e4m3_codes(v.astype(np.float32))


def kv_rows(seed: int, r: int, l: int, positions, dim: int = 576, fp8_scale: float | None = None) -> np.ndarray:
    """Host KV rows at ``positions``: bf16 bits uint16 [n, dim], or, with
    ``fp8_scale``, FP8 E4M3 codes uint8 [n, dim] of value / fp8_scale."""
    pos = np.asarray(positions, dtype=np.uint64).reshape(-1)
    e = pos[:, None] * np.uint64(dim) + np.arange(dim, dtype=np.uint64)[None, :]
    if fp8_scale is not None:
        return fp8_values(kv_key(seed, r, l), e, fp8_scale)
    return bf16_values(kv_key(seed, r, l), e)


def q_block(seed: int, t: int, l: int, r: int, heads: int, dim: int = 576) -> np.ndarray:
    """bf16 bits [heads, dim] of the query of request r, layer l, step t."""
    e = np.arange(heads * dim, dtype=np.uint64).reshape(heads, dim)
    return bf16_values(q_key(seed, t, l, r), e)
