"""Shared helpers of the GPU parity tests: run a workload through the C ABI
(``hisparse_step``) and compare every step with the CPU oracle."""

from __future__ import annotations

import sys

import numpy as np

from oracle.step import OracleDecoder
from tracegen import fill
from tracegen.populate import populate, queries

O_TOL = 2e-3  # max |O_gpu - O_ref| / max |O_ref| per (layer, request, step)
LSE_TOL = 2e-3  # absolute, on the natural-log normaliser


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def make_pool(w, device="cuda:0", host_coherent=0):
    from host_offloaded_kv_amd.hisparse import HiSparse

    cfg = w.config_dict()
    cfg["host_coherent"] = host_coherent
    hs = HiSparse(cfg, device)
    populate(hs, w)
    return hs


class GpuRun:
    """Drives ``hisparse_step`` over a trace, one step at a time."""

    def __init__(self, w, hs):
        import torch

        self.torch = torch
        self.w = w
        self.hs = hs
        dev = hs.device
        L, R, K, H = w.num_layers, w.num_requests, w.top_k, w.num_heads
        self.rows = torch.empty((L, R, K), dtype=torch.int32, device=dev)
        self.counts = torch.empty((L, R, 3), dtype=torch.int32, device=dev)
        self.out = torch.empty((L, R, H, 512), dtype=torch.float32, device=dev)
        self.lse = torch.empty((L, R, H), dtype=torch.float32, device=dev)
        self.d_step = torch.zeros(1, dtype=torch.int32, device=dev)

    def step(self, t: int, sel_t: np.ndarray):
        torch = self.torch
        dev = self.hs.device
        self.d_step.fill_(t)
        topk = torch.from_numpy(np.ascontiguousarray(sel_t, dtype=np.int32)).to(dev)
        q = torch.from_numpy(queries(self.w, t).view(np.int16)).to(dev)
        self.hs.step(self.d_step, topk, q, self.w.scale, self.rows, self.counts, self.out, self.lse)
        torch.cuda.synchronize(dev)
        return (self.rows.cpu().numpy(), self.counts.cpu().numpy())


def check_state(hs, dec, pairs, t):
    for (l, r) in pairs:
        owner, stamp = hs.export_state(r, l)
        st = dec.states[(l, r)]
        assert np.array_equal(owner, np.asarray(st.owner, np.int32)), f"owner t={t} l={l} r={r}"
        assert np.array_equal(stamp, np.asarray(st.stamp, np.int32)), f"stamp t={t} l={l} r={r}"


def check_hot_bytes(hs, w, dec, pairs, t):
    """Every occupied hot row equals the host row of its owner, bit for bit."""
    import torch

    for (l, r) in pairs:
        st = dec.states[(l, r)]
        slots = np.array([s for s, p in enumerate(st.owner) if p >= 0], dtype=np.int64)
        if slots.shape[0] == 0:
            continue
        owners = np.array([st.owner[s] for s in slots], dtype=np.int64)
        base = dec.hot_base(r)
        from tracegen.values import kv_key

        idx = torch.from_numpy(base + slots).to(hs.device)
        if w.kv_dtype == "fp8":
            got = hs.kv[l][idx].cpu().numpy()
            want = fill.rows_fp8(kv_key(w.seed, r, l), owners, w.latent_dim, w.fp8_scale(l))
        else:
            got = hs.kv[l][idx].view(torch.int16).cpu().numpy().view(np.uint16)
            want = fill.rows(kv_key(w.seed, r, l), owners, w.latent_dim)
        assert np.array_equal(got, want), f"hot row bytes t={t} l={l} r={r}"


# Worst secondary error metrics seen by check_attention (reported, see below).
ATTN_STATS = {"block": 0.0, "per_head": 0.0, "elementwise_floor": 0.0}


def attention_errors(o, o_ref):
    """Three error measures of O [H, 512] against the fp64 reference:
    block: max |O - ref| / max |ref| over the whole block (the bar);
    per_head: the same with each head normalised by its own max |ref|;
    elementwise_floor: max |O - ref| / max(|ref|, 1e-3 max |ref|) per element,
    which weighs outputs near zero heavily and is reported, not bounded."""
    d = np.abs(o - o_ref)
    den = np.abs(o_ref).max()
    block = d.max() / den
    hmax = np.abs(o_ref).max(axis=1)
    per_head = max((d[h].max() / hmax[h] for h in range(o.shape[0]) if hmax[h] > 0), default=0.0)
    floor = (d / np.maximum(np.abs(o_ref), 1e-3 * den)).max()
    return block, per_head, floor


def check_attention(run, dec, t, sel_t, pairs):
    """O within O_TOL of the oracle's, normalised per (layer, request) block
    and per head; lse within LSE_TOL.  Returns the worst block error."""
    worst = 0.0
    out = run.out
    lse = run.lse
    for (l, r) in pairs:
        g = l // run.w.index_share
        o_ref, lse_ref = dec.attend_one(t, l, r, sel_t[g][r])
        o = out[l, r].cpu().numpy().astype(np.float64)
        ls = lse[l, r].cpu().numpy().astype(np.float64)
        den = np.abs(o_ref).max()
        if den == 0:
            assert np.all(o == 0) and np.all(np.isneginf(ls)), f"empty attention t={t} l={l} r={r}"
            continue
        err, per_head, floor = attention_errors(o, o_ref)
        worst = max(worst, err)
        ATTN_STATS["block"] = max(ATTN_STATS["block"], err)
        ATTN_STATS["per_head"] = max(ATTN_STATS["per_head"], per_head)
        ATTN_STATS["elementwise_floor"] = max(ATTN_STATS["elementwise_floor"], floor)
        assert err <= O_TOL, f"O rel err {err:.3e} t={t} l={l} r={r}"
        assert per_head <= O_TOL, f"O per-head rel err {per_head:.3e} t={t} l={l} r={r}"
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(ls), fin), f"lse finiteness t={t} l={l} r={r}"
        lerr = np.abs(ls[fin] - lse_ref[fin]).max(initial=0.0)
        assert lerr <= LSE_TOL, f"lse abs err {lerr:.3e} t={t} l={l} r={r}"
    return worst


def run_and_compare(w, steps=None, attend_every=1, attend_pairs=None, state_pairs=None,
                    bytes_pairs=None, requests_for_oracle=None, label="", trace=None, setup=None,
                    host_coherent=0):
    """Run ``steps`` decode steps on the GPU and check each one (``trace``:
    the selections to use instead of the workload's own sorted trace;
    ``setup``: called with the pool before the first step; ``host_coherent``:
    the host pool's memory type)."""
    steps = w.steps if steps is None else steps
    tr = w.trace(steps) if trace is None else trace
    hs = make_pool(w, host_coherent=host_coherent)
    if setup is not None:
        setup(hs)
    run = GpuRun(w, hs)
    dec = OracleDecoder(w, requests=requests_for_oracle)
    all_pairs = [(l, r) for l in range(w.num_layers) for r in dec.requests]
    worst = 0.0
    for t in range(steps):
        rows, counts = run.step(t, tr[t])
        res = dec.resolve_step(t, tr[t])
        for (l, r), rr in res.items():
            assert np.array_equal(rows[l, r], np.asarray(rr.rows, np.int32)), f"{label} rows t={t} l={l} r={r}"
            assert tuple(int(x) for x in counts[l, r]) == (rr.n_resident, rr.n_hit, rr.n_miss), \
                f"{label} counts t={t} l={l} r={r}: gpu {tuple(counts[l, r])} oracle {(rr.n_resident, rr.n_hit, rr.n_miss)}"
        check_state(hs, dec, state_pairs if state_pairs is not None else all_pairs, t)
        if bytes_pairs is not None:
            check_hot_bytes(hs, w, dec, bytes_pairs, t)
        if t % attend_every == 0 or t == steps - 1:
            worst = max(worst, check_attention(run, dec, t, tr[t], attend_pairs if attend_pairs is not None else all_pairs))
    flags = hs.check_errors()
    assert flags == 0, f"device error flags {flags:#x}"
    log(f"{label}: {steps} steps ok, worst O rel err {worst:.3e} (block), {ATTN_STATS['per_head']:.3e} "
        f"(per head, all checks so far), elementwise with a 1e-3 floor {ATTN_STATS['elementwise_floor']:.3e}")
    return hs, run, dec
