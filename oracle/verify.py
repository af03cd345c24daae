"""RESOLVE of a multi-token verification step -- test infrastructure only.

The vLLM Hybrid HiSparse blog (section on composing with the rest of vLLM,
and the note under its concurrency calculator) says that speculative
decoding works through a per-step replayable resolver plan in which the
verification steps share the request's hot state, and that with MTP the hot
buffer must hold all verification tokens at once, so it is sized
(num_speculative_tokens + 2) x top-K.  The plainest reading, used here:

* a step verifies T = num_speculative_tokens + 1 query tokens per request;
  each has its own top-K selection;
* one RESOLVE per (request, layer) covers the T selections together: a
  position selected by several tokens is resolved once (the earliest entry
  of the concatenated lists is the one resolved), and every copy gets that
  entry's row; a position repeated inside one token's own list is a caller
  error, treated as padding, as for a single token;
* the resolved positions are handled by the single-token rules (residency
  first, hits refreshed and pinned, misses in ascending position order into
  the least recent unpinned slots), so the whole union stays in the buffer
  for the step; that needs B >= T x K (the blog's +1 is headroom);
* counts (resident, hit, miss) are over the distinct positions resolved.
"""

from __future__ import annotations

from .resolve import ERR_DUP, ERR_RANGE, ERR_STEP, ResolveResult, resolve


def resolve_verify(state, sels, t: int, ctx: int, block_table, page_size: int, hot_base: int,
                   policy: str = "lru", priority=None) -> ResolveResult:
    """``sels``: T lists of K positions (-1 = padding).  Returns rows for the
    T*K entries in token-major order; mutates ``state``."""
    T = len(sels)
    K = len(sels[0])
    W = T * K
    if state.hot_slots < W:
        raise ValueError("hot_slots must be >= num_verify * top_k")
    if t < 0 or t < state.last_t:
        return ResolveResult([-1] * W, 0, 0, 0, [], ERR_STEP)
    flat = [int(p) for s in sels for p in s]
    errors = 0
    first = {}  # position -> index of the entry that is resolved
    tokens = {}  # position -> tokens that selected it so far
    link = [-1] * W
    kept = [-1] * W  # the selection the single-token rules see
    for j, p in enumerate(flat):
        if p == -1:
            continue
        if p < -1 or p >= ctx:
            errors |= ERR_RANGE
            continue
        b = j // K
        if p in first:
            if b in tokens[p]:
                errors |= ERR_DUP
            else:
                tokens[p].add(b)
                link[j] = first[p]
            continue
        first[p] = j
        tokens[p] = {b}
        kept[j] = p
    res = resolve(state, kept, t, ctx, block_table, page_size, hot_base, policy=policy, priority=priority)
    rows = list(res.rows)
    for j in range(W):
        if link[j] >= 0:
            rows[j] = rows[link[j]]
    return ResolveResult(rows, res.n_resident, res.n_hit, res.n_miss, res.fetches, res.errors | errors)
