"""Seeded synthetic top-K selection traces (input generation only).

Stand-in for the indexer of a sparse-attention model: every decode step it
names K distinct logical positions per request and layer group.  Two
structural facts from the HiSparse summary article ("显存占用直降30倍！…
HiSparse夯爆了", section 01) shape the generator: consecutive steps reselect
many of the same positions, and the selection drifts.  The drift model is
"keep a fraction of the previous selection, resample the rest":

* weights: ``w(p) = (ctx - p) ** -alpha`` (recency-biased, alpha = 0.8) or
  ``w(p) = 1`` (uniform);
* step 0: K positions by Efraimidis-Spirakis weighted sampling without
  replacement (Information Processing Letters 97(5), 2006): draw
  ``u ~ U[0,1)`` for every candidate, key ``ln(u) / w``, keep the K largest
  keys, equal keys going to the lower position;
* step t > 0: keep ``floor(retain * K + 0.5)`` positions of the previous
  selection, chosen uniformly without replacement, then draw the rest with
  the same weighted method over every position not kept (positions dropped
  earlier may come back);
* each selection is stored sorted ascending as int32; if ctx < K the list is
  the whole context padded with -1 at the end.

Randomness: request r of layer group g uses
``numpy.random.Generator(PCG64(SeedSequence([seed, g, r])))``, drawing per
step in this order: (t > 0 only) ``rng.choice(prev, n_keep, replace=False)``,
then ``rng.random(ctx)``.
"""

from __future__ import annotations

import numpy as np


def recency_weights(ctx: int, alpha: float) -> np.ndarray:
    pos = np.arange(ctx, dtype=np.float64)
    return (ctx - pos) ** (-alpha)


def es_top(u: np.ndarray, w: np.ndarray, k: int, excluded: np.ndarray | None) -> np.ndarray:
    """Indices of the k largest keys ln(u)/w; ties go to the lower index."""
    with np.errstate(divide="ignore"):
        key = np.log(u) / w
    if excluded is not None:
        key[excluded] = -np.inf
    n = key.shape[0]
    if k <= 0:
        return np.zeros(0, dtype=np.int64)
    if k >= n:
        return np.arange(n)
    kth = np.partition(key, n - k)[n - k]
    cand = np.nonzero(key >= kth)[0]
    if cand.shape[0] > k:
        order = np.lexsort((cand, -key[cand]))
        cand = cand[order[:k]]
    return cand


class SelectionStream:
    """Step-by-step selection trace of one (layer group, request)."""

    def __init__(self, seed: int, group: int, request: int, ctx: int, k: int,
                 retain: float, alpha: float | None):
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, group, request])))
        self.ctx = int(ctx)
        self.k = int(k)
        self.retain = float(retain)
        self.w = recency_weights(self.ctx, alpha) if alpha is not None else np.ones(self.ctx)
        self.prev: np.ndarray | None = None

    def next(self) -> np.ndarray:
        kk = min(self.k, self.ctx)
        if self.prev is None:
            u = self.rng.random(self.ctx)
            sel = es_top(u, self.w, kk, None)
        else:
            n_keep = int(np.floor(self.retain * kk + 0.5))
            kept = self.rng.choice(self.prev, size=n_keep, replace=False) if n_keep > 0 else np.zeros(0, np.int64)
            u = self.rng.random(self.ctx)
            excl = np.zeros(self.ctx, dtype=bool)
            excl[kept] = True
            fresh = es_top(u, self.w, kk - n_keep, excl)
            sel = np.concatenate([kept.astype(np.int64), fresh.astype(np.int64)])
        sel = np.sort(sel.astype(np.int64))
        self.prev = sel
        out = np.full(self.k, -1, dtype=np.int32)
        out[: sel.shape[0]] = sel
        return out


def selection_trace(seed: int, ctx_lens, k: int, steps: int, groups: int,
                    retain: float, alpha: float | None) -> np.ndarray:
    """int32 [steps][groups][R][k] selection trace."""
    ctx_lens = list(ctx_lens)
    out = np.empty((steps, groups, len(ctx_lens), k), dtype=np.int32)
    for g in range(groups):
        for r, ctx in enumerate(ctx_lens):
            s = SelectionStream(seed, g, r, ctx, k, retain, alpha)
            for t in range(steps):
                out[t, g, r] = s.next()
    return out


class GrowingSelectionStream:
    """Selection stream of a context that grows by one token per step.

    At step t the candidates are positions [0, ctx0 + t + 1): the token
    appended at step t can already be selected.  Weights are recomputed for
    the current length each step (recency relative to the newest token);
    retain and resample as in ``SelectionStream``.  Randomness:
    ``Generator(PCG64(SeedSequence([seed, group, request, 1])))``, drawing
    per step (t > 0 only) ``rng.choice(prev, n_keep, replace=False)``, then
    ``rng.random(ctx_t)``.
    """

    def __init__(self, seed: int, group: int, request: int, ctx0: int, k: int,
                 retain: float, alpha: float | None):
        self.rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, group, request, 1])))
        self.ctx0 = int(ctx0)
        self.k = int(k)
        self.retain = float(retain)
        self.alpha = alpha
        self.t = 0
        self.prev: np.ndarray | None = None

    def next(self) -> np.ndarray:
        ctx = self.ctx0 + self.t + 1
        self.t += 1
        w = recency_weights(ctx, self.alpha) if self.alpha is not None else np.ones(ctx)
        kk = min(self.k, ctx)
        if self.prev is None:
            sel = es_top(self.rng.random(ctx), w, kk, None)
        else:
            n_keep = int(np.floor(self.retain * min(kk, self.prev.shape[0]) + 0.5))
            kept = self.rng.choice(self.prev, size=n_keep, replace=False) if n_keep > 0 else np.zeros(0, np.int64)
            u = self.rng.random(ctx)
            excl = np.zeros(ctx, dtype=bool)
            excl[kept] = True
            fresh = es_top(u, w, kk - n_keep, excl)
            sel = np.concatenate([kept.astype(np.int64), fresh.astype(np.int64)])
        sel = np.sort(sel.astype(np.int64))
        self.prev = sel
        out = np.full(self.k, -1, dtype=np.int32)
        out[: sel.shape[0]] = sel
        return out


def growing_selection_trace(seed: int, ctx0s, k: int, steps: int, groups: int,
                            retain: float, alpha: float | None) -> np.ndarray:
    """int32 [steps][groups][R][k]; step t selects from [0, ctx0_r + t + 1)."""
    ctx0s = list(ctx0s)
    out = np.empty((steps, groups, len(ctx0s), k), dtype=np.int32)
    for g in range(groups):
        for r, c0 in enumerate(ctx0s):
            s = GrowingSelectionStream(seed, g, r, c0, k, retain, alpha)
            for t in range(steps):
                out[t, g, r] = s.next()
    return out
