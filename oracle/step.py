"""One decode step over a workload -- test infrastructure only (CPU oracle).

For each layer group (the layers that share one selection, as with GLM 5.3's
IndexShare in the vLLM Hybrid HiSparse blog, section "在需要时利用稀疏性"),
RESOLVE every layer of the group with the group's selection, then attend
every layer (HiSparse summary article, section 02: one RESOLVE per sparse
layer, then sparse attention over the resolved rows).  State is per
(request, layer); each layer fetches its own host rows.

Attention is computed from the host rows of the selected logical positions
(the method is exact, so this is what the device must reproduce).
``SimulatedKV`` additionally mirrors the device KV tensor (resident pages
plus hot rows written by each fetch) so a test can check that attending
through the resolved row ids gives the same result bit for bit.
"""

from __future__ import annotations

import numpy as np

from tracegen import kv_rows, q_block

from .attention import attend, attend_f64, bf16_bits_to_f64
from .fp8 import e4m3_to_f64
from .resolve import LruState, resolve
from .verify import resolve_verify


class OracleDecoder:
    def __init__(self, w, requests=None):
        self.w = w
        self.requests = list(range(w.num_requests)) if requests is None else list(requests)
        self.states = {(l, r): LruState(w.hot_slots) for l in range(w.num_layers) for r in self.requests}

    def hot_base(self, r: int) -> int:
        return self.w.resident_rows_per_layer + r * self.w.hot_slots

    def resolve_step(self, t: int, sel_t: np.ndarray):
        """sel_t: int32 [groups][R][K] ([groups][R][T][K] with T verify
        tokens).  Returns {(l, r): ResolveResult}."""
        w = self.w
        out = {}
        for g in range(w.groups):
            for l in range(g * w.index_share, (g + 1) * w.index_share):
                for r in self.requests:
                    if w.num_verify > 1:
                        out[(l, r)] = resolve_verify(self.states[(l, r)], sel_t[g][r], t, w.ctx_len[r],
                                                     w.block_tables[r], w.page_size, self.hot_base(r))
                    else:
                        out[(l, r)] = resolve(self.states[(l, r)], sel_t[g][r], t, w.ctx_len[r],
                                              w.block_tables[r], w.page_size, self.hot_base(r))
        return out

    def attend_one(self, t: int, l: int, r: int, sel: np.ndarray, token: int = 0):
        """fp64 (O [H, 512], lse [H]) of (request r, layer l, verify token)
        at step t; ``sel`` is that token's selection."""
        w = self.w
        pos = list(dict.fromkeys(int(p) for p in sel if p >= 0))  # a repeat inside one list is padding
        q = q_block(w.seed, w.query_step(t, token), l, r, w.num_heads, w.latent_dim)
        if w.kv_dtype == "fp8":
            codes = kv_rows(w.seed, r, l, pos, w.latent_dim, fp8_scale=w.fp8_scale(l)) if pos else \
                np.zeros((0, w.latent_dim), np.uint8)
            return attend_f64(bf16_bits_to_f64(q), row_values(w, l, codes), w.scale, w.v_dim)
        x = kv_rows(w.seed, r, l, pos, w.latent_dim) if pos else np.zeros((0, w.latent_dim), np.uint16)
        return attend(q, x, w.scale, w.v_dim)

    def step(self, t: int, sel_t: np.ndarray, attend_pairs=None):
        """Resolve every layer of every group, then attend.

        ``attend_pairs``: iterable of (l, r) to attend (default: all).
        Returns (resolve results, {(l, r): (O, lse)}), keyed (l, r, token)
        with T > 1 verify tokens.
        """
        res = self.resolve_step(t, sel_t)
        w = self.w
        if attend_pairs is None:
            attend_pairs = [(l, r) for l in range(w.num_layers) for r in self.requests]
        att = {}
        for (l, r) in attend_pairs:
            g = l // w.index_share
            if w.num_verify > 1:
                for i in range(w.num_verify):
                    att[(l, r, i)] = self.attend_one(t, l, r, sel_t[g][r][i], token=i)
            else:
                att[(l, r)] = self.attend_one(t, l, r, sel_t[g][r])
        return res, att


def row_values(w, l: int, rows: np.ndarray) -> np.ndarray:
    """float64 values of stored rows of layer l: bf16 bits, or FP8 E4M3 codes
    times the layer's scale."""
    if w.kv_dtype == "fp8":
        return e4m3_to_f64(rows) * w.fp8_scale(l)
    return bf16_bits_to_f64(rows)


class SimulatedKV:
    """Mirror of the device KV tensor of every layer, for small workloads."""

    def __init__(self, w):
        self.w = w
        self.rows = {}  # (layer, row id) -> uint16 [D]
        for r in range(w.num_requests):
            bt = w.block_tables[r]
            for page, blk in enumerate(bt):
                if blk < 0:
                    continue
                lo = page * w.page_size
                hi = min(lo + w.page_size, w.ctx_len[r])
                for l in range(w.num_layers):
                    data = kv_rows(w.seed, r, l, list(range(lo, hi)), w.latent_dim, fp8_scale=w.fp8_scale(l))
                    for i, p in enumerate(range(lo, hi)):
                        self.rows[(l, int(blk) * w.page_size + (p - lo))] = data[i]

    def apply_fetches(self, l: int, r: int, fetches, hot_base: int) -> None:
        if not fetches:
            return
        data = kv_rows(self.w.seed, r, l, [p for p, _ in fetches], self.w.latent_dim, fp8_scale=self.w.fp8_scale(l))
        for i, (_, s) in enumerate(fetches):
            self.rows[(l, hot_base + s)] = data[i]

    def gather(self, l: int, row_ids) -> np.ndarray:
        ids = [int(x) for x in row_ids if x >= 0]
        if not ids:
            return np.zeros((0, self.w.latent_dim), np.uint8 if self.w.kv_dtype == "fp8" else np.uint16)
        return np.stack([self.rows[(l, i)] for i in ids])
