"""Synthetic decode workloads (input generation only).

Each workload fixes the shapes of one decode-path scenario: requests R,
sparse layers L, layers per shared selection (index share g), context
lengths, query heads H, top-K, hot-buffer slots B per (request, layer),
decode steps, the drift of the selection and which 64-token pages of each
request are GPU-resident.  The five named workloads are:

* ``tiny``: 1 request x 1 layer, 4096-token context, 16 heads, K=256, B=512,
  64 steps, retain 0.7 recency-biased, every page host-only.
* ``r8_ctx32k``: 8 x 32768, 1 layer, 64 heads, K=2048, B=4096, 32 steps,
  retain 0.7, the tail page (last 64 tokens) GPU-resident.
* ``r32_ctx128k_l4``: 32 x 131072, 4 layers sharing one selection, 128 heads,
  K=2048, B=4096, 16 steps, retain 0.85, tail page resident.
* ``mixed_r64``: 64 requests with contexts uniform in [4096, 163840], 64
  heads, K=2048, B=4096, 16 steps, retain 0.7, tail page plus half of the
  other pages GPU-resident at random block ids.
* ``miss_1m``: 1 x 1000000, 128 heads, K=B=2048, 32 steps, a fresh uniform
  selection every step (nearly every selected row misses).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .trace import selection_trace

LATENT_DIM = 576
V_DIM = 512


@dataclass
class Workload:
    name: str
    seed: int
    num_requests: int
    num_layers: int
    index_share: int
    ctx_len: list
    num_heads: int
    top_k: int
    hot_slots: int
    steps: int
    retain: float
    alpha: float | None  # None = uniform weights
    residency: str  # "none" | "tail" | "tail+half"
    page_size: int = 64
    latent_dim: int = LATENT_DIM
    v_dim: int = V_DIM
    block_tables: list = field(default_factory=list)  # per request int32 [n_pages]
    resident_blocks: int = 0
    kv_dtype: str = "bf16"  # "bf16" or "fp8" (OCP FP8 E4M3 codes with a per-layer scale)
    kv_scale: list | None = None  # [L] FP8 row scales
    num_verify: int = 1  # T query tokens per request per step (multi-token verification)

    @property
    def groups(self) -> int:
        return self.num_layers // self.index_share

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.latent_dim)

    @property
    def resident_rows_per_layer(self) -> int:
        return self.resident_blocks * self.page_size

    def fp8_scale(self, l: int) -> float | None:
        """Scale of layer l's FP8 rows, or None for bf16 rows."""
        return float(self.kv_scale[l]) if self.kv_dtype == "fp8" else None

    def n_pages(self, r: int) -> int:
        return -(-int(self.ctx_len[r]) // self.page_size)

    def trace(self, steps: int | None = None) -> np.ndarray:
        """int32 [steps][groups][R][K] selections; with T = num_verify > 1,
        [steps][groups][R][T][K], where token i of step t is step t*T + i of
        the single-token drift trace (consecutive tokens overlap)."""
        n = self.steps if steps is None else steps
        T = self.num_verify
        tr = selection_trace(self.seed, self.ctx_len, self.top_k, n * T, self.groups, self.retain, self.alpha)
        if T == 1:
            return tr
        G, R, K = tr.shape[1], tr.shape[2], tr.shape[3]
        return np.ascontiguousarray(tr.reshape(n, T, G, R, K).transpose(0, 2, 3, 1, 4))

    def query_step(self, t: int, token: int = 0) -> int:
        """Counter of the query of verify token ``token`` at step t."""
        return t * self.num_verify + token

    def config_dict(self) -> dict:
        return dict(num_requests=self.num_requests, num_layers=self.num_layers,
                    index_share=self.index_share, latent_dim=self.latent_dim,
                    v_dim=self.v_dim, top_k=self.top_k, hot_slots=self.hot_slots,
                    page_size=self.page_size, num_heads=self.num_heads,
                    resident_rows_per_layer=self.resident_rows_per_layer,
                    ctx_len=[int(c) for c in self.ctx_len], kv_dtype=self.kv_dtype,
                    kv_scale=list(self.kv_scale) if self.kv_dtype == "fp8" else None,
                    num_verify=self.num_verify)


def _assign_residency(w: Workload) -> None:
    R = w.num_requests
    bts = [np.full(w.n_pages(r), -1, dtype=np.int32) for r in range(R)]
    if w.residency == "none":
        w.resident_blocks = 0
    elif w.residency == "tail":
        for r in range(R):
            bts[r][-1] = r
        w.resident_blocks = R
    elif w.residency == "tail+half":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([w.seed, 2 << 20])))
        chosen = []
        for r in range(R):
            others = w.n_pages(r) - 1
            pick = rng.choice(others, size=others // 2, replace=False) if others > 0 else np.zeros(0, np.int64)
            pages = np.sort(np.concatenate([pick.astype(np.int64), [others]]))
            chosen.append(pages)
        nb = sum(len(c) for c in chosen)
        ids = rng.permutation(nb).astype(np.int32)
        k = 0
        for r in range(R):
            for pg in chosen[r]:
                bts[r][pg] = ids[k]
                k += 1
        w.resident_blocks = nb
    else:
        raise ValueError(w.residency)
    w.block_tables = bts


def make_workload(name: str, seed: int, num_requests: int, num_layers: int, index_share: int,
                  ctx_len, num_heads: int, top_k: int, hot_slots: int, steps: int,
                  retain: float, alpha: float | None, residency: str,
                  page_size: int = 64) -> Workload:
    w = Workload(name=name, seed=seed, num_requests=num_requests, num_layers=num_layers,
                 index_share=index_share, ctx_len=[int(c) for c in ctx_len], num_heads=num_heads,
                 top_k=top_k, hot_slots=hot_slots, steps=steps, retain=retain, alpha=alpha,
                 residency=residency, page_size=page_size)
    _assign_residency(w)
    return w


def named_workload(name: str) -> Workload:
    if name == "tiny":
        return make_workload(name, 1, 1, 1, 1, [4096], 16, 256, 512, 64, 0.7, 0.8, "none")
    if name == "r8_ctx32k":
        return make_workload(name, 2, 8, 1, 1, [32768] * 8, 64, 2048, 4096, 32, 0.7, 0.8, "tail")
    if name == "r32_ctx128k_l4":
        return make_workload(name, 3, 32, 4, 4, [131072] * 32, 128, 2048, 4096, 16, 0.85, 0.8, "tail")
    if name == "mixed_r64":
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([4, 1 << 20])))
        ctx = rng.integers(4096, 163840, endpoint=True, size=64)
        return make_workload(name, 4, 64, 1, 1, ctx, 64, 2048, 4096, 16, 0.7, 0.8, "tail+half")
    if name == "miss_1m":
        return make_workload(name, 5, 1, 1, 1, [1_000_000], 128, 2048, 2048, 32, 0.0, None, "none")
    raise KeyError(name)


NAMED = ("tiny", "r8_ctx32k", "r32_ctx128k_l4", "mixed_r64", "miss_1m")


def default_fp8_scales(num_layers: int) -> list:
    """Per-layer FP8 scales of the synthetic pools: 2^-5 * (1 + l/4) (float32).
    The generated values lie in [-6, 6], so value / scale stays inside E4M3's
    +-448; layer 0's scale is a power of two, the others are not."""
    return [float(np.float32(2.0 ** -5 * (1 + l / 4))) for l in range(num_layers)]


def with_fp8(w: Workload, scales=None) -> Workload:
    """The same workload with FP8 E4M3 host and device rows."""
    w.kv_dtype = "fp8"
    w.kv_scale = list(scales) if scales is not None else default_fp8_scales(w.num_layers)
    w.name = w.name + "_fp8"
    return w
