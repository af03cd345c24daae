"""The C-ABI library loads, exports every declared symbol, and validates
configurations on the host (no GPU needed: no compute call is made)."""

import ctypes
import os
import re

import pytest

from host_offloaded_kv_amd import hisparse as H

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    with open(os.path.join(ROOT, "include", "hisparse.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(hisparse_[a-z_]+)\s*\(", text)))


def test_every_declared_symbol_is_exported():
    lib = H.load()
    names = _declared()
    assert len(names) >= 15
    for n in names:
        assert hasattr(lib, n), n
    assert sorted(H.EXPORTED) == names


def _cfg(**kw):
    base = dict(num_requests=2, num_layers=4, index_share=4, top_k=2048, hot_slots=4096, num_heads=128,
                resident_rows_per_layer=128, ctx_len=[131072, 5000])
    base.update(kw)
    return H.make_config(base)


def test_sizes():
    c, keep = _cfg()
    assert H.hisparse_kv_rows_per_layer(c) == 128 + 2 * 4096
    ws = H.hisparse_workspace_bytes(c)
    # owner + stamp + order arrays alone are 3 * L * R * B * 4 bytes
    assert ws >= 3 * 4 * 2 * 4096 * 4


@pytest.mark.parametrize("bad", [
    dict(hot_slots=1000),            # B < K
    dict(top_k=0),
    dict(top_k=5000, hot_slots=8000),
    dict(hot_slots=17000),           # above 16384
    dict(index_share=3),             # L % g != 0
    dict(num_heads=24),              # not a multiple of 16
    dict(page_size=48),              # not a power of two
    dict(resident_rows_per_layer=100),
    dict(ctx_len=[0, 5]),
    dict(latent_dim=512),
    dict(kv_dtype=2),                        # unknown row format
    dict(num_verify=-1),
    dict(num_verify=3),                      # B = 4096 < T * K = 6144
    dict(num_verify=5, hot_slots=16384),     # T * K = 10240 > 8192
    dict(num_verify=2, hot_slots=4095),      # B < T * K
    dict(kv_dtype="fp8", kv_scale=[1.0, 0.0, 1.0, 1.0]),
    dict(kv_dtype="fp8", kv_scale=[1.0, float("nan"), 1.0, 1.0]),
])
def test_bad_configs_rejected(bad):
    c, keep = _cfg(**bad)
    with pytest.raises(H.HiSparseError) as ei:
        H.hisparse_workspace_bytes(c)
    assert ei.value.status == H.HISPARSE_EINVAL
    assert H.hisparse_last_error()


def test_row_formats_and_verify_tokens_size_the_workspace():
    c1, k1 = _cfg()
    c8, k8 = _cfg(kv_dtype="fp8", kv_scale=[0.5, 0.25, 1.0, 2.0])
    assert H.hisparse_workspace_bytes(c8) == H.hisparse_workspace_bytes(c1)  # device metadata does not depend on it
    assert H.hisparse_kv_rows_per_layer(c8) == H.hisparse_kv_rows_per_layer(c1)
    c2, k2 = _cfg(num_verify=2)  # miss lists and partials grow with the token axis
    assert H.hisparse_workspace_bytes(c2) > H.hisparse_workspace_bytes(c1)
    c0, k0 = _cfg(num_verify=0)  # 0 reads as 1
    assert H.hisparse_workspace_bytes(c0) == H.hisparse_workspace_bytes(c1)


def test_null_arguments_rejected():
    lib = H.load()
    assert lib.hisparse_workspace_bytes(None, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_resolve(None, 0, 1, None, None, None, None, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_step(None, None, None, None, 1.0, None, None, None, None, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_host_rows(None, 0, 0) is None
    assert lib.hisparse_stream_copy(None, None, 16, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_row_gather(None, None, None, 1, 1152, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_reset_state(None, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_set_replacement(None, 0, 0, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_sparse_mla_decode_layers(None, 0, 1, None, None, 1.0, None, None, None) == H.HISPARSE_EINVAL
    assert lib.hisparse_set_pipeline(None, 0, 0, 0, 0, 0) == H.HISPARSE_EINVAL
    assert lib.hisparse_decode_fallback_count(None, None, None) == H.HISPARSE_EINVAL
    c, keep = _cfg()
    out = ctypes.c_void_p()
    assert lib.hisparse_create_pool(ctypes.byref(c), None, 0, None, None, ctypes.byref(out)) == H.HISPARSE_EINVAL


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(H, "_lib", None)
    monkeypatch.setattr(H, "LIB_PATH", os.path.join(ROOT, "does_not_exist.so"))
    with pytest.raises(RuntimeError):
        H.load()


def _create(c, ws, ws_bytes, kv):
    lib = H.load()
    arr = (ctypes.c_void_p * len(kv))(*kv)
    out = ctypes.c_void_p()
    st = lib.hisparse_create_pool(ctypes.byref(c), ws, ws_bytes, arr, None, ctypes.byref(out))
    return st, out.value


def test_misaligned_and_short_buffers_rejected_before_any_device_call():
    """The pointer checks run before the library touches the device, so
    made-up aligned addresses reach them; nothing is dereferenced."""
    c, keep = _cfg()
    ws_bytes = H.hisparse_workspace_bytes(c)
    good_kv = [0x10000 + 0x1000 * l for l in range(4)]
    st, p = _create(c, 0x20000 + 128, ws_bytes, good_kv)  # workspace must be 256-byte aligned
    assert st == H.HISPARSE_EINVAL and p is None
    assert "d_workspace" in H.hisparse_last_error() and "aligned" in H.hisparse_last_error()
    bad_kv = list(good_kv)
    bad_kv[2] += 8  # KV tensors must be 16-byte aligned
    st, p = _create(c, 0x20000, ws_bytes, bad_kv)
    assert st == H.HISPARSE_EINVAL and "d_kv" in H.hisparse_last_error()
    st, p = _create(c, 0x20000, ws_bytes - 1, good_kv)  # one byte short
    assert st == H.HISPARSE_EINVAL and "workspace too small" in H.hisparse_last_error()


def test_host_pool_limit_gives_enomem_before_allocating():
    """A pool above its pinned-memory budget (the blog's per-replica
    host_pool_gib) is refused with ENOMEM before any allocation."""
    c, keep = _cfg()
    need = 4 * (131072 + 5000) * 1152
    ws_bytes = H.hisparse_workspace_bytes(c)
    kv = [0x10000 + 0x1000 * l for l in range(4)]
    c.host_pool_limit = need - 1
    st, p = _create(c, 0x20000, ws_bytes, kv)
    assert st == H.HISPARSE_ENOMEM and p is None
    assert str(need) in H.hisparse_last_error()
    c8, keep8 = _cfg(kv_dtype="fp8", host_pool_limit=need // 2 - 1)  # 576-byte rows need half
    st, p = _create(c8, 0x20000, H.hisparse_workspace_bytes(c8), kv)
    assert st == H.HISPARSE_ENOMEM and str(need // 2) in H.hisparse_last_error()
    c.host_pool_limit = -5
    st, p = _create(c, 0x20000, ws_bytes, kv)
    assert st == H.HISPARSE_EINVAL


def test_static_scratch_size_matches_header():
    with open(os.path.join(ROOT, "include", "hisparse.h")) as f:
        m = re.search(r"#define HISPARSE_STATIC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == H.HISPARSE_STATIC_SCRATCH_BYTES


def test_mtp3_at_top_k_2048_is_accepted():
    """The blog's MTP3 setting at K = 2048: T = 4, B = (T + 1) K = 10240."""
    c, keep = _cfg(num_verify=4, hot_slots=10240)
    assert H.hisparse_workspace_bytes(c) > 0
    assert H.hisparse_kv_rows_per_layer(c) == 128 + 2 * 10240
