"""OCP FP8 E4M3 decoding -- test infrastructure only (CPU oracle).

The vLLM Hybrid HiSparse blog (measurements section) runs with an FP8 KV
cache without describing its layout; the reading used here is one OCP
8-bit floating point E4M3 code per latent value (the "OFP8" format of the
Open Compute Project specification) times a per-layer scale.  A code
``s eeee mmm`` is:

* NaN when ``eeee mmm`` is all ones (no infinities in E4M3);
* ``(-1)^s * 2^(1 - 7) * (m / 8)`` when ``eeee = 0`` (subnormal);
* ``(-1)^s * 2^(e - 7) * (1 + m / 8)`` otherwise (exponent bias 7).

The largest finite magnitude is 2^8 * 1.75 = 448.  The value is computed
directly from those fields in float64, where it is exact.
"""

from __future__ import annotations

import numpy as np


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, np.ldexp(m / 8.0, 1 - 7), np.ldexp(1.0 + m / 8.0, e - 7))
    mag = np.where((e == 0xF) & (m == 0x7), np.nan, mag)
    return np.where(s == 1, -mag, mag)
