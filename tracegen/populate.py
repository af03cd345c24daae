"""Write a workload's generated inputs into a pool's memory (input setup only).

Works on any object that exposes ``host_rows_ptr(r, l)`` (host address of
the pinned pool rows of request r, layer l), ``set_block_table(r, bt)``,
``kv`` (list of per-layer device tensors [rows, 576], bf16 or uint8 FP8
codes) and ``device``;
it does not import the decode library.  Resident pages are copies of the
host rows they mirror.
"""

from __future__ import annotations

import numpy as np

from . import fill
from .values import kv_key, q_key


def fill_host_pool(hs, w) -> None:
    for r in range(w.num_requests):
        n = int(w.ctx_len[r]) * w.latent_dim
        for l in range(w.num_layers):
            if w.kv_dtype == "fp8":
                fill.fill_ptr_fp8(hs.host_rows_ptr(r, l), kv_key(w.seed, r, l), 0, n, w.fp8_scale(l))
            else:
                fill.fill_ptr(hs.host_rows_ptr(r, l), kv_key(w.seed, r, l), 0, n)


def upload_residency(hs, w) -> None:
    import torch

    for r in range(w.num_requests):
        bt = np.asarray(w.block_tables[r], dtype=np.int32)
        hs.set_block_table(r, bt)
        pages = np.nonzero(bt >= 0)[0]
        if pages.shape[0] == 0:
            continue
        off = np.arange(w.page_size)
        pos = (pages[:, None] * w.page_size + off[None, :]).reshape(-1)
        rows = (bt[pages][:, None].astype(np.int64) * w.page_size + off[None, :]).reshape(-1)
        keep = pos < w.ctx_len[r]
        pos, rows = pos[keep], rows[keep]
        idx = torch.from_numpy(rows).to(hs.device)
        for l in range(w.num_layers):
            host = hs.host_rows(r, l)
            if w.kv_dtype == "fp8":
                hs.kv[l][idx] = torch.from_numpy(np.ascontiguousarray(host[pos])).to(hs.device)
            else:
                data = torch.from_numpy(np.ascontiguousarray(host[pos]).view(np.int16)).to(hs.device)
                hs.kv[l].view(torch.int16)[idx] = data


def populate(hs, w) -> None:
    fill_host_pool(hs, w)
    upload_residency(hs, w)


def queries(w, t: int) -> np.ndarray:
    """bf16 bits [L][R][H][576] of step t's queries ([L][R][T][H][576] with
    T = num_verify > 1 verify tokens, token i using query counter t*T + i)."""
    T = w.num_verify
    out = np.empty((w.num_layers, w.num_requests, T, w.num_heads, w.latent_dim), np.uint16)
    for l in range(w.num_layers):
        for r in range(w.num_requests):
            for i in range(T):
                fill.fill_array(out[l, r, i], q_key(w.seed, w.query_step(t, i), l, r))
    return out[:, :, 0] if T == 1 else out
