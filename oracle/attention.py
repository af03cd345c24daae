"""Dense fp64 sparse-MLA decode attention -- test infrastructure only.

The HiSparse summary article (section 02) states that the method is exact:
it changes only where KV rows live, so the selected positions, the
attention scores and the outputs equal those of attention over the full KV
restricted to the same selection.  The oracle is therefore the plain
definition of softmax attention over the gathered rows, in float64:

    s[h, j]  = scale * sum_{d < 576} q[h, d] * x_j[d]
    w[h, :]  = softmax(s[h, :])            (max subtracted first)
    O[h, c]  = sum_j w[h, j] * x_j[c],     c < 512
    lse[h]   = max_j s[h, j] + ln sum_j exp(s[h, j] - max_j s[h, j])

where x_j is a 576-wide bf16 latent row (512 "nope" dims followed by 64
rope dims) and the value vector of row j is its first 512 dims (the
absorbed-MLA decode form).  With no valid row, O = 0 and lse = -inf.
"""

from __future__ import annotations

import numpy as np


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening: a bf16 value is the upper half of a float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def attend(q_bits: np.ndarray, x_bits: np.ndarray, scale: float, v_dim: int = 512):
    """q_bits: uint16 [H, D]; x_bits: uint16 [n, D] bf16 rows (valid rows only).

    Returns (O float64 [H, v_dim], lse float64 [H]).
    """
    x = bf16_bits_to_f64(x_bits) if x_bits.shape[0] else np.zeros((0, q_bits.shape[1]))
    return attend_f64(bf16_bits_to_f64(q_bits), x, scale, v_dim)


def attend_f64(q: np.ndarray, x: np.ndarray, scale: float, v_dim: int = 512):
    """The same with the query and the rows already widened to float64
    (FP8 rows: their decoded values times the layer scale)."""
    H = q.shape[0]
    if x.shape[0] == 0:
        return np.zeros((H, v_dim)), np.full(H, -np.inf)
    s = float(scale) * (q @ x.T)  # [H, n]
    m = s.max(axis=1, keepdims=True)
    e = np.exp(s - m)
    z = e.sum(axis=1, keepdims=True)
    w = e / z
    out = w @ x[:, :v_dim]
    lse = (m + np.log(z))[:, 0]
    return out, lse
