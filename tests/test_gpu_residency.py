"""GPU tests of residency transitions: appending tokens into the resident
tail page, write-back of completed pages to the host pool, leasing and
dropping blocks, against the CPU oracle step by step (vLLM Hybrid HiSparse
blog, section "工作原理")."""

from __future__ import annotations

import types

import numpy as np
import pytest

from oracle.attention import attend_f64, bf16_bits_to_f64
from oracle.fp8 import e4m3_to_f64
from oracle.resolve import LruState, resolve
from tests.gpu_harness import LSE_TOL, O_TOL, log
from tracegen import fill, growing_selection_trace, kv_rows, q_block
from tracegen.residency import growing_schedule
from tracegen.values import kv_key

pytestmark = pytest.mark.gpu

PAGE = 64
FP8_SCALES = [2.0 ** -5, 0.0390625]


class Rows:
    """Stored rows of the test's pool format: bf16 bits or FP8 codes."""

    def __init__(self, seed, kv_dtype):
        self.seed, self.fp8 = seed, kv_dtype == "fp8"

    def stored(self, r, l, pos):
        return kv_rows(self.seed, r, l, pos, 576, fp8_scale=FP8_SCALES[l] if self.fp8 else None)

    def values(self, r, l, pos):
        x = self.stored(r, l, pos)
        return e4m3_to_f64(x) * FP8_SCALES[l] if self.fp8 else bf16_bits_to_f64(x)

    def device(self, torch, data):
        """A numpy row block as the tensor layout of the pool's KV tensors."""
        return torch.from_numpy(np.ascontiguousarray(data) if self.fp8 else data.view(np.int16))


def _setup(seed, ctx0, steps, L, H, K, B, keep=2, blocks_per_request=4, kv_dtype="bf16"):
    import torch

    from host_offloaded_kv_amd.hisparse import HiSparse

    R = len(ctx0)
    rw = Rows(seed, kv_dtype)
    sch = growing_schedule(ctx0, steps, PAGE, total_blocks=blocks_per_request * R, keep=keep)
    cfg = dict(num_requests=R, num_layers=L, index_share=L, top_k=K, hot_slots=B, page_size=PAGE, num_heads=H,
               resident_rows_per_layer=blocks_per_request * R * PAGE, ctx_len=list(ctx0),
               ctx_capacity=list(sch.capacity), kv_dtype=kv_dtype,
               kv_scale=FP8_SCALES[:L] if kv_dtype == "fp8" else None)
    hs = HiSparse(cfg, "cuda:0")
    for r in range(R):
        for l in range(L):
            host = hs.host_rows(r, l)
            host[ctx0[r]:] = 0  # rows not yet written must not match by accident
            if rw.fp8:
                fill.fill_ptr_fp8(hs.host_rows_ptr(r, l), kv_key(seed, r, l), 0, ctx0[r] * 576, FP8_SCALES[l])
            else:
                fill.fill_ptr(hs.host_rows_ptr(r, l), kv_key(seed, r, l), 0, ctx0[r] * 576)
        hs.set_block_table(r, np.asarray(sch.initial_bt[r], np.int32))
        # the resident page of position ctx0 already holds the positions below ctx0
        pg = ctx0[r] // PAGE
        blk = sch.initial_bt[r][pg]
        lo = pg * PAGE
        if lo < ctx0[r]:
            pos = list(range(lo, ctx0[r]))
            rows_idx = torch.arange(blk * PAGE, blk * PAGE + len(pos), device=hs.device)
            for l in range(L):
                kvl = hs.kv[l] if rw.fp8 else hs.kv[l].view(torch.int16)
                kvl[rows_idx] = rw.device(torch, rw.stored(r, l, pos)).to(hs.device)
    torch.cuda.synchronize()
    return hs, sch


@pytest.mark.parametrize("kv_dtype", ["bf16", "fp8"])
def test_append_writeback_drop_matches_oracle(kv_dtype):
    import torch

    seed, L, H, K, B = 21, 2, 16, 128, 256
    ctx0 = [300, 190, 450]
    steps = 150
    R = len(ctx0)
    rw = Rows(seed, kv_dtype)
    hs, sch = _setup(seed, ctx0, steps, L, H, K, B, kv_dtype=kv_dtype)
    trace = growing_selection_trace(seed, ctx0, K, steps, 1, 0.7, 0.8)
    dev = hs.device
    new_rows = torch.empty((L, R, 576), dtype=torch.uint8 if rw.fp8 else torch.int16, device=dev)
    d_step = torch.zeros(1, dtype=torch.int32, device=dev)
    topk = torch.empty((1, R, K), dtype=torch.int32, device=dev)
    q = torch.empty((L, R, H, 576), dtype=torch.int16, device=dev)
    rows = torch.empty((L, R, K), dtype=torch.int32, device=dev)
    counts = torch.empty((L, R, 3), dtype=torch.int32, device=dev)
    out = torch.empty((L, R, H, 512), dtype=torch.float32, device=dev)
    lse = torch.empty((L, R, H), dtype=torch.float32, device=dev)
    scale = 1.0 / np.sqrt(576.0)
    states = {(l, r): LruState(B) for l in range(L) for r in range(R)}
    def hot_base(r):
        return 4 * R * PAGE + r * B  # resident rows per layer, then B hot rows per request
    drops = leases = 0
    worst = 0.0
    for t in range(steps):
        for (r, pg, blk) in sch.pre[t]:
            hs.set_pages(r, pg, [blk])
            leases += 1
        pos = [ctx0[r] + t for r in range(R)]
        nr = np.stack([np.stack([rw.stored(r, l, [pos[r]])[0] for r in range(R)]) for l in range(L)])
        new_rows.copy_(rw.device(torch, nr))
        d_step.fill_(t)
        topk.copy_(torch.from_numpy(np.ascontiguousarray(trace[t])))
        qq = np.stack([np.stack([q_block(seed, t, l, r, H, 576) for r in range(R)]) for l in range(L)])
        q.copy_(torch.from_numpy(qq.view(np.int16)))
        hs.append(new_rows)
        hs.step(d_step, topk, q, scale, rows, counts, out, lse)
        hs.writeback()
        torch.cuda.synchronize(dev)
        g_rows, g_counts = rows.cpu().numpy(), counts.cpu().numpy()
        g_out, g_lse = out.cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        for l in range(L):
            for r in range(R):
                ctx = sch.ctx_at(t, r)
                res = resolve(states[(l, r)], trace[t][0][r], t, ctx, sch.bt_at[t][r], PAGE, hot_base(r))
                assert np.array_equal(g_rows[l, r], np.asarray(res.rows, np.int32)), f"rows t={t} l={l} r={r}"
                assert tuple(int(x) for x in g_counts[l, r]) == (res.n_resident, res.n_hit, res.n_miss), \
                    f"counts t={t} l={l} r={r}"
                if t % 10 == 0 or t == steps - 1:
                    sel = [int(p) for p in trace[t][0][r] if p >= 0]
                    o_ref, lse_ref = attend_f64(bf16_bits_to_f64(q_block(seed, t, l, r, H, 576)),
                                                rw.values(r, l, sel), scale, 512)
                    err = np.abs(g_out[l, r] - o_ref).max() / np.abs(o_ref).max()
                    worst = max(worst, err)
                    assert err <= O_TOL, f"O t={t} l={l} r={r} err {err:.3e}"
                    assert np.abs(g_lse[l, r] - lse_ref).max() <= LSE_TOL
        for (r, pg, _) in sch.post[t]:
            hs.set_pages(r, pg, [-1])
            drops += 1
    flags = hs.check_errors()
    assert flags == 0, f"device error flags {flags:#x}"
    ctx, held = hs.get_lengths()
    for r in range(R):
        assert ctx[r] == ctx0[r] + steps
        want_held = max(ctx0[r], ((ctx0[r] + steps) // PAGE) * PAGE)
        assert all(held[l, r] == want_held for l in range(L)), (held[:, r], want_held)
        for l in range(L):
            host = hs.host_rows(r, l)
            lo, hi = ctx0[r], want_held
            if hi > lo:
                assert np.array_equal(host[lo:hi], rw.stored(r, l, list(range(lo, hi)))), \
                    f"host rows of appended pages r={r} l={l}"
            assert not host[want_held:].any(), "rows past the written-back pages stay untouched"
    for l in range(L):
        for r in range(R):
            owner, stamp = hs.export_state(r, l)
            assert np.array_equal(owner, np.asarray(states[(l, r)].owner, np.int32))
            assert np.array_equal(stamp, np.asarray(states[(l, r)].stamp, np.int32))
    log(f"{kv_dtype}: {steps} growing steps ok: {leases} leases, {drops} drops, worst O rel err {worst:.3e}")
    assert leases > 0 and drops > 0
    hs.close()


def test_append_and_drop_errors():
    """Forced from the host: an append whose tail page is a placeholder is
    flagged and leaves the context; dropping a page the host pool does not
    hold yet is rejected."""
    import torch

    from host_offloaded_kv_amd.hisparse import HISPARSE_EINVAL, HISPARSE_ERR_APPEND, HiSparseError

    seed, L, H, K, B = 22, 2, 16, 64, 128
    ctx0 = [128, 100]
    hs, sch = _setup(seed, ctx0, 70, L, H, K, B)
    dev = hs.device
    new_rows = torch.zeros((L, 2, 576), dtype=torch.int16, device=dev)
    # request 0: ctx 128 starts page 2, which holds block 0; request 1: ctx 100 is inside page 1 (block 1)
    hs.set_pages(0, 2, [-1])  # allowed: page 2 holds no position yet, nothing to lose
    hs.append(new_rows)
    torch.cuda.synchronize(dev)
    assert hs.check_errors() & HISPARSE_ERR_APPEND
    ctx, held = hs.get_lengths()
    assert ctx[0] == 128 and ctx[1] == 101
    # page 1 of request 1 is resident and only partly held by the host pool
    with pytest.raises(HiSparseError) as ei:
        hs.set_pages(1, 1, [-1])
    assert ei.value.status == HISPARSE_EINVAL
    assert hs.check_errors() == 0
    hs.close()
