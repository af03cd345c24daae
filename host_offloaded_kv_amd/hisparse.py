"""ctypes binding of ``libhisparse.so`` (the C ABI in ``include/hisparse.h``).

Argument marshalling only: every step of the decode path runs in the HIP
library.  Device buffers are passed as integer addresses (for example
``tensor.data_ptr()``) and streams as ``hipStream_t`` handles (for example
``torch.cuda.current_stream().cuda_stream``).  The functions keep the C
names; ``HiSparse`` below is a small convenience owner that allocates the
workspace and the KV tensors with PyTorch.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libhisparse.so")

HISPARSE_OK = 0
HISPARSE_EINVAL = -1
HISPARSE_ENOMEM = -2
HISPARSE_EHIP = -3
HISPARSE_EDEVICE = -4
HISPARSE_ESTATE = -5

# device error flag bits (hisparse_check_errors)
HISPARSE_ERR_RANGE = 1
HISPARSE_ERR_DUP = 2
HISPARSE_ERR_STEP = 4
HISPARSE_ERR_ROW = 8
HISPARSE_ERR_APPEND = 16
HISPARSE_ERR_UNMATERIALIZED = 32

# KV row formats (hisparse_config.kv_dtype)
HISPARSE_KV_BF16 = 0
HISPARSE_KV_FP8_E4M3 = 1
KV_DTYPES = {"bf16": HISPARSE_KV_BF16, "fp8": HISPARSE_KV_FP8_E4M3}
ROW_BYTES = {HISPARSE_KV_BF16: 1152, HISPARSE_KV_FP8_E4M3: 576}

# size of the fixed split-partial array of hisparse_sparse_mla_decode_layers_static
HISPARSE_STATIC_SCRATCH_BYTES = 64 << 20

# replacement policies (hisparse_set_replacement)
HISPARSE_POLICY_LRU = 0
HISPARSE_POLICY_FIFO = 1
HISPARSE_POLICY_RANDOM = 2
POLICIES = {"lru": HISPARSE_POLICY_LRU, "fifo": HISPARSE_POLICY_FIFO, "random": HISPARSE_POLICY_RANDOM}
ERR_RANGE = 1
ERR_DUP = 2
ERR_STEP = 4
ERR_ROW = 8

EXPORTED = (
    "hisparse_last_error", "hisparse_workspace_bytes", "hisparse_kv_rows_per_layer",
    "hisparse_create_pool", "hisparse_destroy_pool", "hisparse_host_rows",
    "hisparse_set_block_table", "hisparse_resolve", "hisparse_sparse_mla_decode",
    "hisparse_sparse_mla_decode_layers", "hisparse_sparse_mla_decode_layers_static",
    "hisparse_step", "hisparse_step_prefetch", "hisparse_prefetch", "hisparse_reset_state", "hisparse_set_pipeline",
    "hisparse_append", "hisparse_writeback", "hisparse_set_pages", "hisparse_get_lengths",
    "hisparse_set_replacement",
    "hisparse_export_state", "hisparse_check_errors", "hisparse_decode_fallback_count",
    "hisparse_host_alloc", "hisparse_host_free", "hisparse_stream_copy", "hisparse_row_gather",
    "hisparse_profile_enable", "hisparse_profile_read",
)


class hisparse_config(ctypes.Structure):
    _fields_ = [
        ("num_requests", ctypes.c_int32), ("num_layers", ctypes.c_int32),
        ("index_share", ctypes.c_int32), ("latent_dim", ctypes.c_int32),
        ("v_dim", ctypes.c_int32), ("top_k", ctypes.c_int32),
        ("hot_slots", ctypes.c_int32), ("page_size", ctypes.c_int32),
        ("num_heads", ctypes.c_int32), ("host_coherent", ctypes.c_int32),
        ("resident_rows_per_layer", ctypes.c_int64),
        ("ctx_len", ctypes.POINTER(ctypes.c_int64)),
        ("ctx_capacity", ctypes.POINTER(ctypes.c_int64)),
        ("kv_dtype", ctypes.c_int32), ("num_verify", ctypes.c_int32),
        ("kv_scale", ctypes.POINTER(ctypes.c_float)),
        ("host_pool_limit", ctypes.c_int64),
    ]


class hisparse_kernel_time(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char_p), ("launches", ctypes.c_int32), ("total_ms", ctypes.c_double)]


class HiSparseError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"hisparse status {status}: {msg}")
        self.status = status


_lib = None
_VP = ctypes.c_void_p
_I32 = ctypes.c_int32


def load() -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build()")
    try:
        # torch carries its own HIP runtime; load it first so that the
        # library binds to the same runtime instance as torch's tensors.
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    sigs = {
        "hisparse_last_error": (ctypes.c_char_p, []),
        "hisparse_workspace_bytes": (_I32, [ctypes.POINTER(hisparse_config), ctypes.POINTER(ctypes.c_size_t)]),
        "hisparse_kv_rows_per_layer": (_I32, [ctypes.POINTER(hisparse_config), ctypes.POINTER(ctypes.c_int64)]),
        "hisparse_create_pool": (_I32, [ctypes.POINTER(hisparse_config), _VP, ctypes.c_size_t,
                                        ctypes.POINTER(_VP), _VP, ctypes.POINTER(_VP)]),
        "hisparse_destroy_pool": (None, [_VP]),
        "hisparse_host_rows": (_VP, [_VP, _I32, _I32]),
        "hisparse_set_block_table": (_I32, [_VP, _I32, _VP, _I32, _VP]),
        "hisparse_resolve": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP, _VP]),
        "hisparse_sparse_mla_decode": (_I32, [_VP, _I32, _VP, _VP, ctypes.c_float, _VP, _VP, _VP]),
        "hisparse_sparse_mla_decode_layers": (_I32, [_VP, _I32, _I32, _VP, _VP, ctypes.c_float, _VP, _VP, _VP]),
        "hisparse_sparse_mla_decode_layers_static": (_I32, [_VP, _I32, _I32, _VP, _VP, ctypes.c_float, _VP, _VP,
                                                            _VP]),
        "hisparse_step": (_I32, [_VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _VP]),
        "hisparse_step_prefetch": (_I32, [_VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _VP, _VP]),
        "hisparse_prefetch": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP, _VP]),
        "hisparse_reset_state": (_I32, [_VP, _VP]),
        "hisparse_set_pipeline": (_I32, [_VP, _I32, _I32, _I32, _I32, _I32]),
        "hisparse_append": (_I32, [_VP, _VP, _VP]),
        "hisparse_set_replacement": (_I32, [_VP, _I32, ctypes.c_uint64, _VP]),
        "hisparse_writeback": (_I32, [_VP, _VP]),
        "hisparse_set_pages": (_I32, [_VP, _I32, _I32, _I32, _VP, _VP]),
        "hisparse_get_lengths": (_I32, [_VP, _VP, _VP, _VP]),
        "hisparse_export_state": (_I32, [_VP, _I32, _I32, _VP, _VP, _VP]),
        "hisparse_check_errors": (_I32, [_VP, _VP, ctypes.POINTER(ctypes.c_uint32)]),
        "hisparse_decode_fallback_count": (_I32, [_VP, _VP, ctypes.POINTER(ctypes.c_int64)]),
        "hisparse_host_alloc": (_I32, [ctypes.c_size_t, _I32, ctypes.POINTER(_VP), ctypes.POINTER(_VP)]),
        "hisparse_host_free": (None, [_VP]),
        "hisparse_stream_copy": (_I32, [_VP, _VP, ctypes.c_size_t, _VP]),
        "hisparse_row_gather": (_I32, [_VP, _VP, _VP, ctypes.c_int64, ctypes.c_int32, _VP]),
        "hisparse_profile_enable": (_I32, [_VP, _I32]),
        "hisparse_profile_read": (_I32, [_VP, ctypes.POINTER(hisparse_kernel_time), _I32, ctypes.POINTER(_I32)]),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != HISPARSE_OK:
        raise HiSparseError(status, load().hisparse_last_error().decode())


def make_config(cfg: dict) -> tuple[hisparse_config, object]:
    """Build a ``hisparse_config`` from a dict; returns (struct, keep-alive)."""
    ctx = (ctypes.c_int64 * len(cfg["ctx_len"]))(*[int(c) for c in cfg["ctx_len"]])
    cap = None
    if cfg.get("ctx_capacity") is not None:
        cap = (ctypes.c_int64 * len(cfg["ctx_capacity"]))(*[int(c) for c in cfg["ctx_capacity"]])
    scl = None
    if cfg.get("kv_scale") is not None:
        scl = (ctypes.c_float * len(cfg["kv_scale"]))(*[float(v) for v in cfg["kv_scale"]])
    c = hisparse_config(
        num_requests=cfg["num_requests"], num_layers=cfg["num_layers"],
        index_share=cfg.get("index_share", 1), latent_dim=cfg.get("latent_dim", 576),
        v_dim=cfg.get("v_dim", 512), top_k=cfg["top_k"], hot_slots=cfg["hot_slots"],
        page_size=cfg.get("page_size", 64), num_heads=cfg["num_heads"],
        host_coherent=cfg.get("host_coherent", 0),
        resident_rows_per_layer=cfg.get("resident_rows_per_layer", 0),
        ctx_len=ctypes.cast(ctx, ctypes.POINTER(ctypes.c_int64)),
        ctx_capacity=ctypes.cast(cap, ctypes.POINTER(ctypes.c_int64)) if cap is not None else None,
        kv_dtype=kv_dtype_code(cfg.get("kv_dtype", "bf16")), num_verify=cfg.get("num_verify", 1),
        kv_scale=ctypes.cast(scl, ctypes.POINTER(ctypes.c_float)) if scl is not None else None,
        host_pool_limit=int(cfg.get("host_pool_limit", 0)),
    )
    return c, (ctx, cap, scl)


def kv_dtype_code(v) -> int:
    return KV_DTYPES[v] if isinstance(v, str) else int(v)


def hisparse_last_error() -> str:
    return load().hisparse_last_error().decode()


def hisparse_workspace_bytes(cfg: hisparse_config) -> int:
    out = ctypes.c_size_t()
    _check(load().hisparse_workspace_bytes(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def hisparse_kv_rows_per_layer(cfg: hisparse_config) -> int:
    out = ctypes.c_int64()
    _check(load().hisparse_kv_rows_per_layer(ctypes.byref(cfg), ctypes.byref(out)))
    return out.value


def hisparse_create_pool(cfg: hisparse_config, d_workspace: int, ws_bytes: int, d_kv: list, stream: int) -> int:
    kv = (_VP * len(d_kv))(*d_kv)
    out = _VP()
    _check(load().hisparse_create_pool(ctypes.byref(cfg), d_workspace, ws_bytes, kv, stream, ctypes.byref(out)))
    return out.value


def hisparse_destroy_pool(pool: int) -> None:
    load().hisparse_destroy_pool(pool)


def hisparse_host_rows(pool: int, r: int, l: int) -> int:
    p = load().hisparse_host_rows(pool, r, l)
    if not p:
        raise HiSparseError(HISPARSE_EINVAL, hisparse_last_error())
    return p


def hisparse_set_block_table(pool: int, r: int, bt: np.ndarray, stream: int) -> None:
    bt = np.ascontiguousarray(bt, dtype=np.int32)
    _check(load().hisparse_set_block_table(pool, r, bt.ctypes.data, bt.shape[0], stream))


def hisparse_resolve(pool, layer_begin, n_layers, d_step, d_topk, d_rows, d_counts, stream) -> None:
    _check(load().hisparse_resolve(pool, layer_begin, n_layers, d_step, d_topk, d_rows, d_counts, stream))


def hisparse_sparse_mla_decode(pool, layer, d_q, d_rows, scale, d_out, d_lse, stream) -> None:
    _check(load().hisparse_sparse_mla_decode(pool, layer, d_q, d_rows, float(scale), d_out, d_lse, stream))


def hisparse_sparse_mla_decode_layers(pool, layer_begin, n_layers, d_q, d_rows, scale, d_out, d_lse, stream) -> None:
    _check(load().hisparse_sparse_mla_decode_layers(pool, layer_begin, n_layers, d_q, d_rows, float(scale), d_out,
                                                    d_lse, stream))


def hisparse_sparse_mla_decode_layers_static(pool, layer_begin, n_layers, d_q, d_rows, scale, d_out, d_lse,
                                             stream) -> None:
    _check(load().hisparse_sparse_mla_decode_layers_static(pool, layer_begin, n_layers, d_q, d_rows, float(scale),
                                                           d_out, d_lse, stream))


def hisparse_step(pool, d_step, d_topk, d_q, scale, d_rows, d_counts, d_out, d_lse, stream) -> None:
    _check(load().hisparse_step(pool, d_step, d_topk, d_q, float(scale), d_rows, d_counts, d_out, d_lse, stream))


def hisparse_step_prefetch(pool, d_step, d_topk, d_topk_next, d_q, scale, d_rows, d_counts, d_out, d_lse,
                           d_pf_counts, stream) -> None:
    _check(load().hisparse_step_prefetch(pool, d_step, d_topk, d_topk_next, d_q, float(scale), d_rows, d_counts,
                                         d_out, d_lse, d_pf_counts, stream))


def hisparse_prefetch(pool, layer_begin, n_layers, d_step, d_topk, d_counts, stream) -> None:
    _check(load().hisparse_prefetch(pool, layer_begin, n_layers, d_step, d_topk, d_counts, stream))


def hisparse_reset_state(pool: int, stream: int) -> None:
    _check(load().hisparse_reset_state(pool, stream))


def hisparse_set_pipeline(pool: int, group_fetch_workgroups: int = 0, unit_fetch_workgroups: int = 0,
                          tail_chunks: int = 0, resident_first: int = 0, fetch_in_decode: int = 0) -> None:
    _check(load().hisparse_set_pipeline(pool, group_fetch_workgroups, unit_fetch_workgroups, tail_chunks,
                                        resident_first, fetch_in_decode))


def hisparse_set_replacement(pool: int, policy: int, seed: int, stream: int) -> None:
    _check(load().hisparse_set_replacement(pool, policy, seed & ((1 << 64) - 1), stream))


def hisparse_append(pool: int, d_rows: int, stream: int) -> None:
    _check(load().hisparse_append(pool, d_rows, stream))


def hisparse_writeback(pool: int, stream: int) -> None:
    _check(load().hisparse_writeback(pool, stream))


def hisparse_set_pages(pool: int, r: int, first_page: int, blocks, stream: int) -> None:
    blocks = np.ascontiguousarray(blocks, dtype=np.int32)
    _check(load().hisparse_set_pages(pool, r, first_page, blocks.shape[0], blocks.ctypes.data, stream))


def hisparse_get_lengths(pool: int, num_requests: int, num_layers: int, stream: int):
    """(ctx [R], held [L][R]) as int32 arrays."""
    ctx = np.empty(num_requests, np.int32)
    held = np.empty((num_layers, num_requests), np.int32)
    _check(load().hisparse_get_lengths(pool, ctx.ctypes.data, held.ctypes.data, stream))
    return ctx, held


def hisparse_export_state(pool: int, r: int, l: int, hot_slots: int, stream: int):
    owner = np.empty(hot_slots, np.int32)
    stamp = np.empty(hot_slots, np.int32)
    _check(load().hisparse_export_state(pool, r, l, owner.ctypes.data, stamp.ctypes.data, stream))
    return owner, stamp


def hisparse_check_errors(pool: int, stream: int) -> int:
    v = ctypes.c_uint32()
    _check(load().hisparse_check_errors(pool, stream, ctypes.byref(v)))
    return v.value


def hisparse_decode_fallback_count(pool: int, stream: int) -> int:
    v = ctypes.c_int64()
    _check(load().hisparse_decode_fallback_count(pool, stream, ctypes.byref(v)))
    return v.value


def hisparse_host_alloc(nbytes: int, coherent: int = 0) -> tuple[int, int]:
    h, d = _VP(), _VP()
    _check(load().hisparse_host_alloc(nbytes, coherent, ctypes.byref(h), ctypes.byref(d)))
    return h.value, d.value


def hisparse_host_free(host: int) -> None:
    load().hisparse_host_free(host)


def hisparse_stream_copy(dst: int, src: int, nbytes: int, stream: int) -> None:
    _check(load().hisparse_stream_copy(dst, src, nbytes, stream))


def hisparse_row_gather(dst: int, src: int, d_rows: int, n_rows: int, row_bytes: int, stream: int) -> None:
    _check(load().hisparse_row_gather(dst, src, d_rows, n_rows, row_bytes, stream))


def hisparse_profile_enable(pool: int, enable: bool) -> None:
    _check(load().hisparse_profile_enable(pool, 1 if enable else 0))


def hisparse_profile_read(pool: int) -> dict:
    """{kernel name: (launches, total_ms)} since the last read."""
    arr = (hisparse_kernel_time * 8)()
    n = _I32()
    _check(load().hisparse_profile_read(pool, arr, 8, ctypes.byref(n)))
    return {arr[i].name.decode(): (arr[i].launches, arr[i].total_ms) for i in range(n.value)}


def host_array(addr: int, shape, dtype=np.uint16) -> np.ndarray:
    """NumPy view of host memory at ``addr`` (no copy)."""
    n = int(np.prod(shape))
    ct = {np.uint16: ctypes.c_uint16, np.int32: ctypes.c_int32, np.uint8: ctypes.c_uint8}[np.dtype(dtype).type]
    buf = (ct * n).from_address(addr)
    return np.ctypeslib.as_array(buf).reshape(shape)


class HiSparse:
    """Owner of one pool: allocates the workspace and KV tensors with torch.

    ``cfg`` is a dict with the ``hisparse_config`` fields (``ctx_len`` a
    list).  ``kv[l]`` is the bf16 KV tensor [kv_rows, 576] of layer l.
    """

    def __init__(self, cfg: dict, device="cuda"):
        import torch

        self.torch = torch
        self.cfg = dict(cfg)
        self.device = torch.device(device)
        self._c, self._keep = make_config(self.cfg)
        self.ws_bytes = hisparse_workspace_bytes(self._c)
        self.kv_rows = hisparse_kv_rows_per_layer(self._c)
        self.workspace = torch.empty(self.ws_bytes, dtype=torch.uint8, device=self.device)
        self.kv_dtype = kv_dtype_code(self.cfg.get("kv_dtype", "bf16"))
        self.row_bytes = ROW_BYTES[self.kv_dtype]
        # bf16 rows: [rows, 576] bfloat16; FP8 rows: [rows, 576] uint8 codes
        kv_torch_dtype = torch.bfloat16 if self.kv_dtype == HISPARSE_KV_BF16 else torch.uint8
        self.kv = [torch.zeros((self.kv_rows, 576), dtype=kv_torch_dtype, device=self.device)
                   for _ in range(self.cfg["num_layers"])]
        self.pool = hisparse_create_pool(self._c, self.workspace.data_ptr(), self.ws_bytes,
                                         [t.data_ptr() for t in self.kv], self.stream)

    @property
    def stream(self) -> int:
        return self.torch.cuda.current_stream(self.device).cuda_stream

    def host_rows_ptr(self, r: int, l: int) -> int:
        return hisparse_host_rows(self.pool, r, l)

    def host_rows(self, r: int, l: int) -> np.ndarray:
        """NumPy view of the host pool rows of (r, l): [capacity_r][576] bf16 bits
        (uint16) or FP8 E4M3 codes (uint8)."""
        cap = self.cfg.get("ctx_capacity") or self.cfg["ctx_len"]
        dt = np.uint16 if self.kv_dtype == HISPARSE_KV_BF16 else np.uint8
        return host_array(self.host_rows_ptr(r, l), (int(cap[r]), 576), dt)

    def set_block_table(self, r: int, bt) -> None:
        hisparse_set_block_table(self.pool, r, bt, self.stream)

    def resolve(self, layer_begin, n_layers, d_step, d_topk, d_rows, d_counts) -> None:
        hisparse_resolve(self.pool, layer_begin, n_layers, d_step.data_ptr(), d_topk.data_ptr(),
                         d_rows.data_ptr(), d_counts.data_ptr(), self.stream)

    def decode(self, layer, d_q, d_rows, scale, d_out, d_lse) -> None:
        hisparse_sparse_mla_decode(self.pool, layer, d_q.data_ptr(), d_rows.data_ptr(), scale,
                                   d_out.data_ptr(), d_lse.data_ptr(), self.stream)

    def decode_layers(self, layer_begin, n_layers, d_q, d_rows, scale, d_out, d_lse) -> None:
        hisparse_sparse_mla_decode_layers(self.pool, layer_begin, n_layers, d_q.data_ptr(), d_rows.data_ptr(), scale,
                                          d_out.data_ptr(), d_lse.data_ptr(), self.stream)

    def step(self, d_step, d_topk, d_q, scale, d_rows, d_counts, d_out, d_lse) -> None:
        hisparse_step(self.pool, d_step.data_ptr(), d_topk.data_ptr(), d_q.data_ptr(), scale,
                      d_rows.data_ptr(), d_counts.data_ptr(), d_out.data_ptr(), d_lse.data_ptr(), self.stream)

    def step_prefetch(self, d_step, d_topk, d_topk_next, d_q, scale, d_rows, d_counts, d_out, d_lse,
                      d_pf_counts=None) -> None:
        hisparse_step_prefetch(self.pool, d_step.data_ptr(), d_topk.data_ptr(), d_topk_next.data_ptr(), d_q.data_ptr(),
                               scale, d_rows.data_ptr(), d_counts.data_ptr(), d_out.data_ptr(), d_lse.data_ptr(),
                               d_pf_counts.data_ptr() if d_pf_counts is not None else None, self.stream)

    def prefetch(self, layer_begin, n_layers, d_step, d_topk, d_counts=None) -> None:
        hisparse_prefetch(self.pool, layer_begin, n_layers, d_step.data_ptr(), d_topk.data_ptr(),
                          d_counts.data_ptr() if d_counts is not None else None, self.stream)

    def reset_state(self) -> None:
        hisparse_reset_state(self.pool, self.stream)

    def set_pipeline(self, group_fetch_workgroups: int = 0, unit_fetch_workgroups: int = 0,
                     tail_chunks: int = 0, resident_first: int = 0, fetch_in_decode: int = 0) -> None:
        hisparse_set_pipeline(self.pool, group_fetch_workgroups, unit_fetch_workgroups, tail_chunks, resident_first,
                              fetch_in_decode)

    def set_replacement(self, policy: str, seed: int = 0) -> None:
        hisparse_set_replacement(self.pool, POLICIES[policy], seed, self.stream)

    def append(self, d_rows) -> None:
        hisparse_append(self.pool, d_rows.data_ptr(), self.stream)

    def writeback(self) -> None:
        hisparse_writeback(self.pool, self.stream)

    def set_pages(self, r: int, first_page: int, blocks) -> None:
        hisparse_set_pages(self.pool, r, first_page, blocks, self.stream)

    def get_lengths(self):
        return hisparse_get_lengths(self.pool, self.cfg["num_requests"], self.cfg["num_layers"], self.stream)

    def export_state(self, r: int, l: int):
        return hisparse_export_state(self.pool, r, l, self.cfg["hot_slots"], self.stream)

    def check_errors(self) -> int:
        return hisparse_check_errors(self.pool, self.stream)

    def decode_fallback_count(self) -> int:
        return hisparse_decode_fallback_count(self.pool, self.stream)

    def close(self) -> None:
        if getattr(self, "pool", None):
            hisparse_destroy_pool(self.pool)
            self.pool = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
