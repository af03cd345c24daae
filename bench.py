#!/usr/bin/env python3
"""Decode-step benchmark of the HiSparse path on one MI355X.

One step = RESOLVE (hit detection, LRU replacement, metadata update, miss
fetch over the host link) plus sparse MLA decode attention for every layer
of every request, i.e. one ``hisparse_step`` call.  Default workload: 32
requests x 131072-token context, 4 sparse layers sharing one top-2048
selection, 128 heads, 4096 hot slots per (request, layer), 64-token tail
page resident, seeded synthetic drift trace (retain 0.85).

Prints one JSON line on stdout; progress goes to stderr.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published
PCIE_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction, published


def pmc_ratio(workload: str, kernel: str, host_link: bool):
    """Counted bytes per algorithmic byte of `kernel` from the committed PMC
    summary of this workload (reads only for the host-link-bound fetch, reads
    plus writes otherwise), with the counted bytes per launch; None when there
    is no summary or the kernel's source file changed since it was taken.
    The counters come from other steps of the same trace than the timed
    ones, so they are carried over as a ratio to the algorithmic bytes."""
    import hashlib

    path = os.path.join(ROOT, "profiles", f"pmc_bytes_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        ks = json.load(f).get("kernels", {})
    names = {"sparse_mla_decode": ["decode_ws_unsplit", "decode_ws_split", "decode_ws_part1", "decode_ws_part2"],
             "sparse_mla_decode_fetch": ["decode_ws_fetch"]}.get(kernel, [kernel])
    es = [ks[n] for n in names if n in ks and "alg_bytes_per_launch" in ks[n]]
    if not es:
        return None
    for e in es:
        with open(os.path.join(ROOT, e["source"]), "rb") as f:
            if hashlib.sha256(f.read()).hexdigest()[:16] != e["source_sha256_16"]:
                return None
    # the fetching decode's counters cover HBM and host-link bytes together:
    # its ratio is to all its algorithmic bytes
    key = "read_per_alg_byte" if host_link and kernel != "sparse_mla_decode_fetch" else "traffic_per_alg_byte"
    n = sum(e["launches"] for e in es)
    ratio = sum(e[key] * e["launches"] for e in es) / n
    rd = sum(e["read_bytes_per_launch"] * e["launches"] for e in es) / n
    wr = sum(e["write_bytes_per_launch"] * e["launches"] for e in es) / n
    return ratio, rd, wr


def log(msg: str) -> None:
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def host_link_probe(torch, H, dev, nbytes=256 << 20, reps=5):
    """Measured host->device bandwidth: DMA copy, zero-copy kernel read, and a
    zero-copy gather of random whole rows (1152 and 576 bytes)."""
    stream = torch.cuda.current_stream(dev)
    host = torch.empty(nbytes, dtype=torch.uint8, pin_memory=True)
    host.fill_(1)
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    dst.copy_(host, non_blocking=True)
    e0.record(stream)
    for _ in range(reps):
        dst.copy_(host, non_blocking=True)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    dma = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    out = {"dma_h2d_GBs": round(dma, 2)}
    for coherent in (0, 1):
        h, d = H.hisparse_host_alloc(nbytes, coherent)
        try:
            ctypes_fill(h, nbytes)
            H.hisparse_stream_copy(dst.data_ptr(), d, nbytes, stream.cuda_stream)
            e0.record(stream)
            for _ in range(reps):
                H.hisparse_stream_copy(dst.data_ptr(), d, nbytes, stream.cuda_stream)
            e1.record(stream)
            torch.cuda.synchronize(dev)
            zc = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
            if not coherent:
                # random whole rows, the miss fetch's access pattern (64 MiB per pass)
                gen = torch.Generator(device=dev).manual_seed(12345)
                for row_bytes in (1152, 576):
                    n_rows = (64 << 20) // row_bytes
                    rows = torch.randint(0, nbytes // row_bytes, (n_rows,), generator=gen, device=dev,
                                         dtype=torch.int64)
                    H.hisparse_row_gather(dst.data_ptr(), d, rows.data_ptr(), n_rows, row_bytes, stream.cuda_stream)
                    e0.record(stream)
                    for _ in range(reps):
                        H.hisparse_row_gather(dst.data_ptr(), d, rows.data_ptr(), n_rows, row_bytes,
                                              stream.cuda_stream)
                    e1.record(stream)
                    torch.cuda.synchronize(dev)
                    out[f"random_{row_bytes}B_row_gather_GBs"] = round(
                        n_rows * row_bytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 2)
        finally:
            H.hisparse_host_free(h)
        out["zero_copy_read_GBs_" + ("coherent" if coherent else "noncoherent")] = round(zc, 2)
    # device-to-device copy with the same kernel (HBM reference)
    src = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    H.hisparse_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream.cuda_stream)
    e0.record(stream)
    for _ in range(reps):
        H.hisparse_stream_copy(dst.data_ptr(), src.data_ptr(), nbytes, stream.cuda_stream)
    e1.record(stream)
    torch.cuda.synchronize(dev)
    out["d2d_copy_GBs"] = round(2 * nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9, 1)
    return out


def residency_probe(torch, H, w, dev, ctx=8192):
    """Cost of the residency transitions at the workload's request, layer and
    head shape: the per-step append (one token per request, every layer) into
    leased tail pages, and the write-back once every (request, layer) has
    completed a page (one launch, zero-copy stores into the host pool)."""
    import numpy as np

    R, L, page = w.num_requests, w.num_layers, w.page_size
    cfg = dict(num_requests=R, num_layers=L, index_share=w.index_share, top_k=w.top_k, hot_slots=w.hot_slots,
               page_size=page, num_heads=w.num_heads, resident_rows_per_layer=R * page,
               ctx_len=[ctx] * R, ctx_capacity=[ctx + page] * R, kv_dtype=w.kv_dtype, kv_scale=w.kv_scale)
    hs = H.HiSparse(cfg, dev)
    row_bytes = hs.row_bytes
    try:
        for r in range(R):
            bt = np.full((ctx + page + page - 1) // page, -1, np.int32)
            bt[ctx // page] = r
            hs.set_block_table(r, bt)
        rows = torch.zeros((L, R, 576), dtype=torch.int16 if row_bytes == 1152 else torch.uint8, device=dev)
        stream = torch.cuda.current_stream(dev)
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        hs.append(rows)  # warm
        e0.record(stream)
        for _ in range(page - 1):
            hs.append(rows)
        e1.record(stream)
        hs.writeback()
        e2.record(stream)
        torch.cuda.synchronize(dev)
        if hs.check_errors():
            return None
        n_ctx, held = hs.get_lengths()
        if not (np.all(n_ctx == ctx + page) and np.all(held == ctx + page)):
            return None
        wb_bytes = R * L * page * row_bytes
        wb_ms = e1.elapsed_time(e2)
        return {"append_us": round(e0.elapsed_time(e1) * 1e3 / (page - 1), 2),
                "append_bytes": R * L * row_bytes,
                "writeback_us": round(wb_ms * 1e3, 2), "writeback_bytes": wb_bytes,
                "writeback_GBs": round(wb_bytes / (wb_ms * 1e-3) / 1e9, 2),
                "writeback_us_per_step_amortised": round(wb_ms * 1e3 / page, 2)}
    finally:
        hs.close()


def ctypes_fill(addr: int, nbytes: int) -> None:
    import ctypes

    ctypes.memset(addr, 1, nbytes)


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, trace, warmup, budget_s=12.0, one_thread_steps=2):
    """The CPU oracle, untuned, on a bounded sample of the same workload.

    Requests 0..5 (all, if fewer) of every layer; steps 0..warmup-1 are
    resolved untimed (they only build the LRU state, as the GPU's warm-up
    steps do), then steps from `warmup` on are timed until `budget_s` runs
    out.  Per step the time is split into RESOLVE (the pure-Python step
    LRU), row generation (the oracle regenerates from the counter-based
    generator every row and query it reads instead of holding a filled
    pool) and ATTEND (fp64 NumPy).  ATTEND is timed again on the first
    timed steps with the BLAS library held to one thread."""
    import numpy as np

    from oracle.attention import attend
    from oracle.step import OracleDecoder
    from tracegen import kv_rows, q_block

    try:
        from threadpoolctl import threadpool_info, threadpool_limits

        blas = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: no thread control
        threadpool_limits, blas = None, None
    reqs = list(range(min(6, w.num_requests)))
    dec = OracleDecoder(w, requests=reqs)
    units = [(l, r, i) for l in range(w.num_layers) for r in reqs for i in range(w.num_verify)]
    t0 = time.perf_counter()
    for t in range(min(warmup, trace.shape[0])):
        dec.resolve_step(t, trace[t])
    warm_s = time.perf_counter() - t0

    T = w.num_verify

    def gen(t, l, r, i):
        g = l // w.index_share
        sel = trace[t][g][r][i] if T > 1 else trace[t][g][r]
        pos = list(dict.fromkeys(int(p) for p in sel if p >= 0))
        q = q_block(w.seed, w.query_step(t, i), l, r, w.num_heads, w.latent_dim)
        return q, kv_rows(w.seed, r, l, pos, w.latent_dim)

    t_res = t_gen = t_att = 0.0
    steps = []
    t0 = time.perf_counter()
    for t in range(warmup, trace.shape[0]):
        a = time.perf_counter()
        dec.resolve_step(t, trace[t])
        b = time.perf_counter()
        t_res += b - a
        for (l, r, i) in units:
            c = time.perf_counter()
            q, x = gen(t, l, r, i)
            d = time.perf_counter()
            attend(q, x, w.scale, w.v_dim)
            e = time.perf_counter()
            t_gen += d - c
            t_att += e - d
        steps.append(t)
        if time.perf_counter() - t0 > budget_s:
            break
    n = len(steps)
    tokens = len(reqs) * n * w.num_verify
    total = t_res + t_gen + t_att
    one = None
    if threadpool_limits is not None and n:
        sub = steps[:one_thread_steps]
        data = [gen(t, l, r, i) for t in sub for (l, r, i) in units]
        with threadpool_limits(limits=1):
            a = time.perf_counter()
            for q, x in data:
                attend(q, x, w.scale, w.v_dim)
            att1 = (time.perf_counter() - a) / len(sub)
        per_step = (t_res + t_gen) / n + att1
        one = {"value": round(len(reqs) * w.num_verify / per_step, 3), "attend_s_per_step": round(att1, 4),
               "steps": len(sub)}
    return {"value": round(tokens / total, 3), "unit": "tokens/s",
            "cores": os.cpu_count(), "kind": "oracle",
            "sample": f"requests {reqs} x all {w.num_layers} layers x steps {steps[0]}..{steps[-1]} after "
                      f"{warmup} untimed warm-up steps (resolve + row generation + fp64 attention), {total:.1f} s",
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(),
            "affinity_cpus": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None,
            "blas_threads": blas,
            "split_s_per_step": {"resolve": round(t_res / n, 4), "row_generation": round(t_gen / n, 4),
                                 "attend": round(t_att / n, 4)},
            "warmup_resolve_s": round(warm_s, 2),
            "one_thread": one}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=14)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="r32_ctx128k_l4")
    ap.add_argument("--host-coherent", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-probe", action="store_true")
    ap.add_argument("--fetch-wg", type=int, default=0,
                    help="workgroups of each pipelined miss fetch of the step (0 = library default)")
    ap.add_argument("--tail-chunks", type=int, default=0,
                    help="request chunks of the last layer of a group (0 = library default)")
    ap.add_argument("--no-sync-path", action="store_true",
                    help="skip the replay of the same steps through the synchronous path")
    ap.add_argument("--no-graph", action="store_true", help="skip the captured-graph replay of the same steps")
    ap.add_argument("--no-decode-only", action="store_true", help="skip the decode-only timing")
    ap.add_argument("--no-residency", action="store_true", help="skip the append / write-back timing")
    ap.add_argument("--no-prefetch", action="store_true", help="skip the cross-step prefetch runs")
    ap.add_argument("--no-resident-first", action="store_true",
                    help="with separate fetches, decode each group's last layer in one launch after its fetch")
    ap.add_argument("--no-fetch-in-decode", action="store_true",
                    help="separate miss fetches (the layer pipeline) instead of the decode reading the filled rows "
                         "from the host pool")
    ap.add_argument("--policy", default="lru", choices=["lru", "fifo", "random"], help="replacement policy")
    ap.add_argument("--policy-seed", type=int, default=1, help="seed of the random replacement policy")
    ap.add_argument("--num-verify", type=int, default=1,
                    help="query tokens per request per step (multi-token verification); the value "
                         "then counts verified query tokens")
    ap.add_argument("--hot-slots", type=int, default=0,
                    help="hot slots per (request, layer); 0 = the workload's, or (T + 1) x top-K with "
                         "T = --num-verify > 1 verify tokens")
    ap.add_argument("--kv-dtype", default="bf16", choices=["bf16", "fp8"],
                    help="KV row format: bf16 (the named workloads) or FP8 E4M3 codes with a per-layer scale")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run 3 device-to-device copies of this size with the library's copy kernel "
                         "(a known-size reference for hardware byte counters)")
    ap.add_argument("--calib-host-mib", type=int, default=0,
                    help="also run 3 zero-copy reads of this size from a pinned host buffer into device memory "
                         "with the same copy kernel (the reference for counters of host-link reads)")
    ap.add_argument("--unsorted", action="store_true",
                    help="feed every selection in a shuffled (indexer) order instead of ascending")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on exactly one GPU: every (request, layer) is independent, and the benchmark "
              "measures one GPU's share; runs on several GPUs are not supported.", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from host_offloaded_kv_amd import hisparse as H
    from tracegen import named_workload, with_fp8
    from tracegen.populate import populate, queries

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    H.load()
    dev = torch.device("cuda:0")
    w = named_workload(args.workload)
    if args.kv_dtype == "fp8":
        w = with_fp8(w)
    w.num_verify = args.num_verify
    if args.hot_slots:
        w.hot_slots = args.hot_slots
    elif w.num_verify > 1:
        # the blog sizes the hot buffer (num_speculative_tokens + 2) x top-K
        w.hot_slots = max(w.hot_slots, (w.num_verify + 1) * w.top_k)
    n_steps = args.warmup + args.steps
    L, R, K, Hh, B = w.num_layers, w.num_requests, w.top_k, w.num_heads, w.hot_slots
    T = w.num_verify

    log(f"workload {w.name}: R={R} L={L} g={w.index_share} ctx={w.ctx_len[0]} H={Hh} K={K} B={B}")
    t0 = time.time()
    trace = w.trace(n_steps + 1)  # one step past the timed ones: the prediction of the last step
    if args.unsorted:
        rng = np.random.default_rng(2024)
        trace = trace.copy()
        flat = trace.reshape(-1, trace.shape[-1])
        for i in range(flat.shape[0]):
            flat[i] = rng.permutation(flat[i])
    log(f"trace generated ({n_steps} steps) in {time.time() - t0:.1f}s")
    cfg = w.config_dict()
    cfg["host_coherent"] = args.host_coherent
    t0 = time.time()
    hs = H.HiSparse(cfg, dev)
    row_bytes = hs.row_bytes
    log(f"pool created ({sum(w.ctx_len) * L * row_bytes / 1e9:.2f} GB pinned) in {time.time() - t0:.1f}s")
    t0 = time.time()
    populate(hs, w)
    pool_fill_s = time.time() - t0
    log(f"host pool filled and residency uploaded in {pool_fill_s:.1f}s")

    d_steps = torch.arange(n_steps, dtype=torch.int32, device=dev)
    d_topk = torch.from_numpy(trace).to(dev)  # [T][G][R][K]
    q_all = np.stack([queries(w, t) for t in range(n_steps)])
    d_q = torch.from_numpy(q_all.view(np.int16)).to(dev)  # [steps][L][R]([T])[H][576]
    d_rows = torch.empty((n_steps, L, R, T * K), dtype=torch.int32, device=dev)
    d_counts = torch.empty((n_steps, L, R, 3), dtype=torch.int32, device=dev)
    d_out = torch.empty((L, R * T, Hh, 512), dtype=torch.float32, device=dev)
    d_lse = torch.empty((L, R * T, Hh), dtype=torch.float32, device=dev)
    torch.cuda.synchronize(dev)
    log("inputs staged in HBM")

    stream = torch.cuda.current_stream(dev)
    hs.set_pipeline(0, args.fetch_wg, args.tail_chunks, -1 if args.no_resident_first else 0,
                    -1 if args.no_fetch_in_decode else 0)
    if args.policy != "lru":
        hs.set_replacement(args.policy, args.policy_seed)

    def step(t, s=None):
        H.hisparse_step(hs.pool, d_steps[t:t + 1].data_ptr(), d_topk[t].data_ptr(), d_q[t].data_ptr(), w.scale,
                        d_rows[t].data_ptr(), d_counts[t].data_ptr(), d_out.data_ptr(), d_lse.data_ptr(),
                        (s or stream).cuda_stream)

    def sync_step(t):
        # the same step through the synchronous path: resolve (metadata + one
        # fetch of the whole group), then decode layer by layer, one stream
        g = w.index_share
        for gi in range(w.groups):
            l0 = gi * g
            H.hisparse_resolve(hs.pool, l0, g, d_steps[t:t + 1].data_ptr(), d_topk[t, gi].data_ptr(),
                               d_rows[t, l0].data_ptr(), d_counts[t, l0].data_ptr(), stream.cuda_stream)
            for l in range(l0, l0 + g):
                H.hisparse_sparse_mla_decode(hs.pool, l, d_q[t, l].data_ptr(), d_rows[t, l].data_ptr(), w.scale,
                                             d_out[l].data_ptr(), d_lse[l].data_ptr(), stream.cuda_stream)

    def time_steps(fn, per_step=None):
        """Replays steps 0..n_steps from the empty state; returns ms of the timed ones.
        per_step (a dict) receives each step's own time in us: the warm-up steps
        (step 0 from the empty state, i.e. cold) and the timed ones, from events
        recorded between the steps on the same stream."""
        hs.reset_state()
        ev = lambda: torch.cuda.Event(enable_timing=True)
        warm = [ev() for _ in range(args.warmup + 1)]
        warm[0].record(stream)
        for t in range(args.warmup):
            fn(t)
            warm[t + 1].record(stream)
        torch.cuda.synchronize(dev)
        evs = [ev() for _ in range(args.steps + 1)]
        evs[0].record(stream)
        for i, t in enumerate(range(args.warmup, n_steps)):
            fn(t)
            evs[i + 1].record(stream)
        torch.cuda.synchronize(dev)
        if per_step is not None:
            per_step["warmup_us"] = [round(warm[i].elapsed_time(warm[i + 1]) * 1e3, 2) for i in range(args.warmup)]
            per_step["timed_us"] = [round(evs[i].elapsed_time(evs[i + 1]) * 1e3, 2) for i in range(args.steps)]
        return evs[0].elapsed_time(evs[-1])

    # 1) eager steps; every kernel is bracketed by HIP events on its stream
    for t in range(args.warmup):
        step(t)
    torch.cuda.synchronize(dev)
    log(f"{args.warmup} warmup steps done")
    H.hisparse_profile_enable(hs.pool, True)
    H.hisparse_profile_read(hs.pool)
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    ev0.record(stream)
    wall0 = time.perf_counter()
    for t in range(args.warmup, n_steps):
        step(t)
    ev1.record(stream)
    torch.cuda.synchronize(dev)
    wall = time.perf_counter() - wall0
    eager_ms = ev0.elapsed_time(ev1)
    prof_eager = H.hisparse_profile_read(hs.pool)
    H.hisparse_profile_enable(hs.pool, False)
    flags = hs.check_errors()
    if flags:
        log(f"device error flags {flags:#x}")
        return 1
    log(f"eager: {args.steps} steps in {eager_ms:.3f} ms (wall {wall * 1e3:.1f} ms)")
    counts = d_counts[args.warmup:].cpu().numpy().astype(np.int64)  # [K][L][R][3]

    # 2) the same steps as captured-graph replays (the timed region of the
    #    headline), with the kernel events captured into the timed graphs
    graph_ms, prof_graph, graph_steps = None, None, {}
    if not args.no_graph:
        log("captured-graph replay of the same steps")
        side = torch.cuda.Stream(device=dev)
        graphs = []
        hs.reset_state()
        side.wait_stream(stream)
        for t in range(n_steps):
            H.hisparse_profile_enable(hs.pool, t >= args.warmup)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=side):
                step(t, side)
            graphs.append(g)
        H.hisparse_profile_enable(hs.pool, False)
        torch.cuda.synchronize(dev)
        graph_ms = time_steps(lambda t: graphs[t].replay(), graph_steps)
        try:
            prof_graph = H.hisparse_profile_read(hs.pool)
            if not prof_graph or any(not (ms > 0) for _, ms in prof_graph.values()):
                log(f"kernel events inside graphs gave no usable times: {prof_graph}")
                prof_graph = None
        except H.HiSparseError as e:
            log(f"kernel events inside graphs not readable ({e}); kernel times from the eager pass")
            prof_graph = None
        log(f"graph replay: {graph_ms / args.steps * 1e3:.1f} us/step")
        if not np.array_equal(d_counts[args.warmup:].cpu().numpy(), counts):
            log("graph replay counts differ from the eager steps")
            return 1
        del graphs
    sync_ms = None
    if not args.no_sync_path:
        log("synchronous path (resolve, then per-layer decode, one stream)")
        sync_ms = time_steps(sync_step)
        log(f"synchronous path: {sync_ms / args.steps * 1e3:.1f} us/step")

    # 2b) cross-step prefetch (graph replays of hisparse_step_prefetch): the
    #     true next selection (the model-provided signal of the HiSparse
    #     summary article, section 04) and the current one reused (speculation
    #     that the selection does not move)
    prefetch = None
    if not args.no_prefetch:
        prefetch = {}
        pf_counts = torch.zeros((n_steps, L, R, 4), dtype=torch.int32, device=dev)
        for kind in ("exact_next", "reuse_current"):
            log(f"prefetch run ({kind})")
            side = torch.cuda.Stream(device=dev)
            hs.reset_state()
            side.wait_stream(stream)
            graphs = []
            for t in range(n_steps):
                nxt = d_topk[t + 1] if kind == "exact_next" else d_topk[t]
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g, stream=side):
                    H.hisparse_step_prefetch(hs.pool, d_steps[t:t + 1].data_ptr(), d_topk[t].data_ptr(),
                                             nxt.data_ptr(), d_q[t].data_ptr(), w.scale, d_rows[t].data_ptr(),
                                             d_counts[t].data_ptr(), d_out.data_ptr(), d_lse.data_ptr(),
                                             pf_counts[t].data_ptr(), side.cuda_stream)
                graphs.append(g)
            torch.cuda.synchronize(dev)
            graph_pf_ms = time_steps(lambda t: graphs[t].replay())
            del graphs

            def eager_pf(t):
                nxt = d_topk[t + 1] if kind == "exact_next" else d_topk[t]
                H.hisparse_step_prefetch(hs.pool, d_steps[t:t + 1].data_ptr(), d_topk[t].data_ptr(), nxt.data_ptr(),
                                         d_q[t].data_ptr(), w.scale, d_rows[t].data_ptr(), d_counts[t].data_ptr(),
                                         d_out.data_ptr(), d_lse.data_ptr(), pf_counts[t].data_ptr(),
                                         stream.cuda_stream)

            eager_pf_ms = time_steps(eager_pf)
            pf_ms = min(graph_pf_ms, eager_pf_ms)
            own = d_counts[args.warmup:].cpu().numpy().astype(np.int64)[..., 2]  # [steps][L][R]
            pfc = pf_counts[args.warmup:].cpu().numpy().astype(np.int64)
            host_rows = own.sum() + pfc[..., 2].sum()
            us = pf_ms / args.steps * 1e3
            prefetch[kind] = {
                "us_per_step": round(us, 2), "tokens_per_s": round(R * T * args.steps / (pf_ms * 1e-3), 2),
                "graph_replay_us_per_step": round(graph_pf_ms / args.steps * 1e3, 2),
                "eager_us_per_step": round(eager_pf_ms / args.steps * 1e3, 2),
                "own_misses_per_step": round(float(own.sum()) / args.steps, 1),
                "prefetched_rows_per_step": round(float(pfc[..., 2].sum()) / args.steps, 1),
                "dropped_per_step": round(float(pfc[..., 3].sum()) / args.steps, 1),
                "host_GBs_over_step": round(float(host_rows) * row_bytes / args.steps / (us * 1e-6) / 1e9, 2)}
            log(f"prefetch {kind}: {prefetch[kind]}")
        if hs.check_errors():
            log("device error flags after the prefetch runs")
            return 1

    # 3) decode alone: every layer of the last step, one launch per layer
    #    (default key splits), over rows that are already resident
    t_last = n_steps - 1
    dec_us = dec_layer_us = None
    if not args.no_decode_only:
        # (a) one launch per index-share group; (b) one launch per layer
        dec_reps = 10
        e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
        e0.record(stream)
        for _ in range(dec_reps):
            for gi in range(w.groups):
                l0 = gi * w.index_share
                H.hisparse_sparse_mla_decode_layers(hs.pool, l0, w.index_share, d_q[t_last, l0].data_ptr(),
                                                    d_rows[t_last, l0].data_ptr(), w.scale, d_out[l0].data_ptr(),
                                                    d_lse[l0].data_ptr(), stream.cuda_stream)
        e1.record(stream)
        for _ in range(dec_reps):
            for l in range(L):
                H.hisparse_sparse_mla_decode(hs.pool, l, d_q[t_last, l].data_ptr(), d_rows[t_last, l].data_ptr(),
                                             w.scale, d_out[l].data_ptr(), d_lse[l].data_ptr(), stream.cuda_stream)
        e2.record(stream)
        torch.cuda.synchronize(dev)
        dec_us = e0.elapsed_time(e1) * 1e3 / dec_reps
        dec_layer_us = e1.elapsed_time(e2) * 1e3 / dec_reps
    flags = hs.check_errors()
    if flags:
        log(f"device error flags {flags:#x} after the replays")
        return 1
    # decode workgroups that left the fp16 path for the exact fp32 one (0
    # for these inputs; the timings above would not be of the fast path)
    fallbacks = hs.decode_fallback_count()

    # the headline is the faster of the two timed modes, with the kernel
    # times recorded in that same mode
    use_graph = graph_ms is not None and prof_graph is not None and graph_ms <= eager_ms
    ms_total = graph_ms if use_graph else eager_ms
    prof = prof_graph if use_graph else prof_eager
    valid = counts.sum(axis=3)  # distinct valid positions per (step, l, r)
    entries = (d_rows[args.warmup:] >= 0).sum(dim=3).cpu().numpy().astype(np.int64)  # rows attended
    misses = counts[..., 2]
    ms_step = ms_total / args.steps
    tokens_per_s = R * T * args.steps / (ms_total * 1e-3)

    # algorithmic bytes per step (split partials and repeated reads are
    # overhead, not counted)
    host_bytes = misses.sum(axis=(1, 2)) * row_bytes  # per step
    attn_bytes = (entries.sum(axis=(1, 2)) * row_bytes
                  + L * R * T * (Hh * (576 * 2 + 512 * 4 + 4) + K * 4))
    attn_flops = entries.sum(axis=(1, 2)) * 2 * Hh * (576 + 512)
    meta_bytes = L * R * (2 * 3 * B * 4 + 2 * K * 4 + 12) + misses.sum(axis=(1, 2)) * 8
    hbm_step_bytes = attn_bytes + host_bytes + meta_bytes  # hot-row writes counted once in host_bytes
    last_valid = entries[-1].sum()
    dec_bytes = last_valid * row_bytes + L * R * T * (Hh * (576 * 2 + 512 * 4 + 4) + K * 4)

    kern = {}
    for name, (n, tot_ms) in prof.items():
        # algorithmic bytes of the timed steps, spread evenly over the launches
        avg_ms = tot_ms / n
        if name in ("fetch_rows", "sparse_mla_decode_fetch"):
            # host-link bytes: the missed rows (the decode that fetches moves
            # every filled row of its index-share group)
            alg = host_bytes.sum() / n
            bound, peak, unit = "host_link", PCIE_PEAK_GBS, "GB/s"
        elif name == "sparse_mla_decode":
            alg = attn_bytes.sum() / n
            bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        elif name == "resolve_meta":
            # bound by latency (dependent LDS phases of one workgroup per
            # (request, layer)); its HBM fraction is context only
            alg = meta_bytes.sum() / n
            bound, peak, unit = "latency", HBM_PEAK_GBS, "GB/s"
        else:
            alg = None  # split merge: overhead only
            bound, peak, unit = "hbm", HBM_PEAK_GBS, "GB/s"
        ach = alg / (avg_ms * 1e-3) / 1e9 if alg is not None else None
        kern[name] = {"launches": n, "avg_us": round(avg_ms * 1e3, 2),
                      "alg_bytes_per_launch": int(alg) if alg is not None else None,
                      "achieved": round(ach, 2) if ach is not None else None, "bound": bound, "peak": peak,
                      "unit": unit, "frac": round(ach / peak, 4) if (peak and ach is not None) else None,
                      "busy_share_of_step": round(tot_ms / ms_total, 4)}
    if "sparse_mla_decode_fetch" in kern:
        kf = kern["sparse_mla_decode_fetch"]
        kf["decode_alg_bytes_per_launch"] = int(attn_bytes.sum() / kf["launches"])
        kf["fp32_fallback_workgroups"] = int(fallbacks)
        kf["note"] = ("the step's only launch besides the metadata kernel: the decode of every layer of an index-share "
                      "group, reading the rows the step fills straight from the pinned host pool (and writing them to "
                      "their hot rows); bound by the host link")
    if "sparse_mla_decode" in kern:
        kern["sparse_mla_decode"]["fp32_fallback_workgroups"] = int(fallbacks)
        kern["sparse_mla_decode"]["in_step_note"] = (
            "in-step launches with separate fetches: the layers of an index-share group but the last decoded "
            "without key splits while the next layer's miss fetch streams, the last layer in two parts (resident "
            "rows beside the fetches, fetched rows after) or split over the whole GPU")
    dk = kern.get("sparse_mla_decode") or kern.get("sparse_mla_decode_fetch")
    if dk is not None and dec_us:
        # the decode alone (rows already resident): one launch over all layers of a group on all CUs
        ach_full = dec_bytes / (dec_us * 1e-6) / 1e9
        dk["full_gpu_launch"] = {
            "us": round(dec_us, 2), "alg_bytes": int(dec_bytes), "achieved": round(ach_full, 2),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(ach_full / HBM_PEAK_GBS, 4)}
    dom = max(prof.items(), key=lambda kv: kv[1][1])[0]
    d = kern[dom]
    pmc = pmc_ratio(w.name, dom, d["bound"] == "host_link") if T == 1 and args.kv_dtype == "bf16" else None
    traffic = None
    alg_for_traffic = d["alg_bytes_per_launch"]
    if dom == "sparse_mla_decode_fetch":
        # host reads and hot-row writes of the filled rows, and the decode's own bytes
        alg_for_traffic = int(2 * d["alg_bytes_per_launch"] + d["decode_alg_bytes_per_launch"])
    if pmc is not None and alg_for_traffic:
        # counted bytes of the timed launches: the counters' ratio to the
        # algorithmic bytes (host-link side: reads) times the timed launches'
        # algorithmic bytes
        traffic = int(pmc[0] * alg_for_traffic)
    roofline = {"bound": d["bound"], "achieved": d["achieved"], "peak": d["peak"], "unit": d["unit"],
                "frac": d["frac"], "traffic": traffic, "kernel": dom, "avg_us": d["avg_us"],
                "alg_bytes_per_launch": d["alg_bytes_per_launch"],
                "traffic_per_alg_byte": round(pmc[0], 4) if pmc else None,
                "traffic_alg_bytes_per_launch": alg_for_traffic,
                "counted_read_write_per_launch_pmc_steps": [int(pmc[1]), int(pmc[2])] if pmc else None}

    residency = None
    if not args.no_residency:
        log("residency transitions (append, write-back)")
        residency = residency_probe(torch, H, w, dev)
        log(f"residency: {residency}")

    probe = None
    if not args.no_probe:
        log("host-link probe")
        probe = host_link_probe(torch, H, dev)
        log(f"host-link probe: {probe}")
    measured_link = max(v for k, v in probe.items() if k != "d2d_copy_GBs") if probe else None
    for kn in ("fetch_rows", "sparse_mla_decode_fetch"):
        if kn in kern and measured_link:
            kern[kn]["frac_of_measured_link"] = round(kern[kn]["achieved"] / measured_link, 4)

    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device=dev)
        dst = torch.empty(nb, dtype=torch.uint8, device=dev)
        for _ in range(3):
            H.hisparse_stream_copy(dst.data_ptr(), src.data_ptr(), nb, stream.cuda_stream)
        torch.cuda.synchronize(dev)
        del src, dst
    if args.calib_host_mib:
        nb = args.calib_host_mib << 20
        h, d = H.hisparse_host_alloc(nb, 0)
        try:
            ctypes_fill(h, nb)
            dst = torch.empty(nb, dtype=torch.uint8, device=dev)
            for _ in range(3):
                H.hisparse_stream_copy(dst.data_ptr(), d, nb, stream.cuda_stream)
            torch.cuda.synchronize(dev)
            del dst
        finally:
            H.hisparse_host_free(h)

    cpu = None
    hs.close()
    del hs
    if not args.no_cpu_baseline:
        log("CPU oracle baseline")
        cpu = cpu_baseline(w, trace[:n_steps], args.warmup)
        log(f"cpu baseline: {cpu}")

    out = {
        "metric": "decode tokens/s (resolve + sparse MLA) at 128K ctx; achieved HBM & host GB/s",
        "value": round(tokens_per_s, 2),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "requests": R, "ctx": int(w.ctx_len[0]), "layers": L,
                   "index_share": w.index_share, "heads": Hh, "top_k": K, "hot_slots": B,
                   "seed": w.seed, "host_coherent": args.host_coherent, "policy": args.policy,
                   "kv_dtype": w.kv_dtype, "num_verify": T,
                   "selection_order": "shuffled (indexer order)" if args.unsorted else "ascending"},
        "roofline": roofline,
        "kernels": kern,
        "step": {"us": round(ms_step * 1e3, 2),
                 "hbm_GBs": round(float(hbm_step_bytes.mean()) / (ms_step * 1e-3) / 1e9, 2),
                 "host_GBs": round(float(host_bytes.mean()) / (ms_step * 1e-3) / 1e9, 2),
                 "miss_rate": round(float(misses.sum() / max(valid.sum(), 1)), 4),
                 "attn_gflop": round(float(attn_flops.mean()) / 1e9, 2)},
        "timing": {"timed_region": "graph replays" if use_graph else "eager steps",
                   "kernel_times_from": "graph replays" if use_graph else "eager steps",
                   "eager_us_per_step": round(eager_ms / args.steps * 1e3, 2),
                   "graph_replay_us_per_step": round(graph_ms / args.steps * 1e3, 2) if graph_ms else None,
                   # graph replays from the empty state: step 0 (cold: every entry misses) and the
                   # median of the timed steps, each from events between the replays
                   "cold_step0_us": graph_steps["warmup_us"][0] if graph_steps.get("warmup_us") else None,
                   "median_us_per_step": (round(float(np.median(graph_steps["timed_us"])), 2)
                                          if graph_steps.get("timed_us") else None),
                   "graph_replay_us_each_step": graph_steps.get("timed_us")},
        "layer_ahead": {"unit_fetch_workgroups": args.fetch_wg or None, "tail_chunks": args.tail_chunks or None,
                        "resident_first": not args.no_resident_first,
                        "fetch_in_decode": not args.no_fetch_in_decode,
                        "sync_path_us_per_step": round(sync_ms / args.steps * 1e3, 2) if sync_ms else None,
                        "sync_path_tokens_per_s": round(R * T * args.steps / (sync_ms * 1e-3), 2) if sync_ms else None},
        "prefetch": dict(prefetch, no_prefetch_us_per_step=round(ms_step * 1e3, 2)) if prefetch else None,
        "decode_only": {"alg_bytes": int(dec_bytes),
                        "per_group_launch": {"us_per_step": round(dec_us, 2), "launches": w.groups,
                                             "achieved_GBs": round(dec_bytes / (dec_us * 1e-6) / 1e9, 2),
                                             "frac_of_hbm": round(dec_bytes / (dec_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
                        "per_layer_launch": {"us_per_step": round(dec_layer_us, 2), "launches": L,
                                             "achieved_GBs": round(dec_bytes / (dec_layer_us * 1e-6) / 1e9, 2),
                                             "frac_of_hbm": round(dec_bytes / (dec_layer_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                                                                  4)}} if dec_us else None,
        "residency": residency,
        "host_link": probe,
        "gpu_host_pool_fill_s": round(pool_fill_s, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
