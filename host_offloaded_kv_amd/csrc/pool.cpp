// Host side of the C ABI: configuration checks, the pinned host pool,
// workspace carving, block tables, and the enqueue entry points.
//
// The pool layout follows the HiSparse summary article (section 02): the
// authoritative full KV of every request and sparse layer sits in pinned
// host DRAM, and the device keeps B slots per (request, layer).  Mixed
// residency (vLLM Hybrid HiSparse blog, "工作原理") adds a per-request block
// table whose resident entries are read in place and never evicted.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <climits>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "internal.h"

namespace hs {
hipError_t set_resolve_lds_limit(int device, size_t bytes);

namespace {
thread_local std::string g_last_error;

inline size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

int ilog2_exact(int v) {
  int b = 0;
  while ((1 << b) < v) ++b;
  return (1 << b) == v ? b : -1;
}

int64_t capacity_of(const hisparse_config* c, int r) {
  return c->ctx_capacity ? c->ctx_capacity[r] : c->ctx_len[r];
}

hisparse_status check_config(const hisparse_config* c) {
  if (!c) {
    set_error("config is NULL");
    return HISPARSE_EINVAL;
  }
  if (c->num_requests < 1 || c->num_layers < 1 || c->index_share < 1 || c->index_share > kMaxIndexShare ||
      c->num_layers % c->index_share) {
    set_error("need num_requests >= 1, num_layers >= 1, 1 <= index_share <= 64 and num_layers % index_share == 0");
    return HISPARSE_EINVAL;
  }
  if (c->latent_dim != kLatent || c->v_dim != kVDim) {
    set_error("latent_dim must be 576 and v_dim 512");
    return HISPARSE_EINVAL;
  }
  if (c->kv_dtype != HISPARSE_KV_BF16 && c->kv_dtype != HISPARSE_KV_FP8_E4M3) {
    set_error("kv_dtype must be HISPARSE_KV_BF16 or HISPARSE_KV_FP8_E4M3");
    return HISPARSE_EINVAL;
  }
  const int T = c->num_verify < 1 ? 1 : c->num_verify;
  if (c->num_verify < 0 || (int64_t)T * c->top_k > kMaxSelection) {
    set_error("num_verify must be >= 0 and num_verify * top_k <= 8192");
    return HISPARSE_EINVAL;
  }
  if (c->kv_scale && c->kv_dtype == HISPARSE_KV_FP8_E4M3) {
    for (int l = 0; l < c->num_layers; ++l)
      if (!(std::isfinite(c->kv_scale[l]) && c->kv_scale[l] > 0.f)) {
        set_error("kv_scale[" + std::to_string(l) + "] must be finite and positive");
        return HISPARSE_EINVAL;
      }
  }
  if (c->top_k < 1 || c->top_k > kMaxTopK) {
    set_error("top_k must be in [1, 4096]");
    return HISPARSE_EINVAL;
  }
  if (c->hot_slots < c->top_k * (c->num_verify < 1 ? 1 : c->num_verify) || c->hot_slots > kMaxHotSlots) {
    set_error("hot_slots must satisfy num_verify * top_k <= hot_slots <= 16384");
    return HISPARSE_EINVAL;
  }
  if (c->page_size < 1 || ilog2_exact(c->page_size) < 0 || c->page_size > (1 << 20)) {
    set_error("page_size must be a power of two");
    return HISPARSE_EINVAL;
  }
  if (c->num_heads < 16 || c->num_heads % 16 || c->num_heads > kMaxHeads) {
    set_error("num_heads must be a multiple of 16 in [16, 256]");
    return HISPARSE_EINVAL;
  }
  if (c->resident_rows_per_layer < 0 || c->resident_rows_per_layer % c->page_size) {
    set_error("resident_rows_per_layer must be a non-negative multiple of page_size");
    return HISPARSE_EINVAL;
  }
  if (!c->ctx_len) {
    set_error("ctx_len is NULL");
    return HISPARSE_EINVAL;
  }
  for (int r = 0; r < c->num_requests; ++r) {
    if (c->ctx_len[r] < 1 || c->ctx_len[r] > (int64_t{1} << 30)) {
      set_error("ctx_len[" + std::to_string(r) + "] must be in [1, 2^30]");
      return HISPARSE_EINVAL;
    }
    if (capacity_of(c, r) < c->ctx_len[r] || capacity_of(c, r) > (int64_t{1} << 30)) {
      set_error("ctx_capacity[" + std::to_string(r) + "] must be in [ctx_len[r], 2^30]");
      return HISPARSE_EINVAL;
    }
  }
  const int64_t rows = c->resident_rows_per_layer + (int64_t)c->num_requests * c->hot_slots;
  if (rows >= (int64_t{1} << 31)) {
    set_error("KV tensor rows per layer must stay below 2^31");
    return HISPARSE_EINVAL;
  }
  if ((int64_t)c->num_layers * c->num_requests > 8192) {
    set_error("num_layers * num_requests must be <= 8192");
    return HISPARSE_EINVAL;
  }
  return HISPARSE_OK;
}

int verify_tokens(const hisparse_config* c) { return c->num_verify < 1 ? 1 : c->num_verify; }

Layout make_layout(const hisparse_config* c) {
  Layout L{};
  const size_t R = c->num_requests, NL = c->num_layers, B = c->hot_slots;
  const size_t T = verify_tokens(c), W = T * c->top_k;  // decode sees R * T query sets
  int64_t bt_entries = 0;
  for (size_t r = 0; r < R; ++r) bt_entries += (capacity_of(c, (int)r) + c->page_size - 1) / c->page_size;
  L.bt_entries = bt_entries;
  // Split partials, sized for every decode launch the pool can make: any
  // number of layers of one index-share group over all R * T query sets
  // (hisparse_sparse_mla_decode_layers, hisparse_step), and one layer over
  // any request chunk (the chunked last layer of hisparse_step).
  size_t part = 0;
  int smax = 1;
  auto need = [&](int n_layers, size_t nsets) {
    const int sn = decode_splits(n_layers, (int)nsets, c->num_heads, c->top_k);
    smax = std::max(smax, sn);
    if (sn > 1) part = std::max(part, (size_t)sn * n_layers * nsets * c->num_heads * kPartW);
  };
  for (int n = 1; n <= c->index_share; ++n) need(n, R * T);
  for (size_t nreq = 1; nreq <= R; ++nreq) need(1, nreq * T);
  if (T == 1) {
    // a group's last layer decoded in two parts (resident rows first)
    int before = 1, after = 0;
    resident_first_splits((int)R, c->num_heads, c->top_k, &before, &after);
    smax = std::max(smax, before + after);
    part = std::max(part, (size_t)(before + after) * R * c->num_heads * kPartW);
  }
  L.splits_max = smax;
  L.partial_floats = part;
  size_t off = 0;
  L.owner = off; off = align256(off + NL * R * B * 4);
  L.stamp = off; off = align256(off + NL * R * B * 4);
  L.lru = off; off = align256(off + NL * R * B * 4);
  L.last_t = off; off = align256(off + NL * R * 4);
  L.miss_count = off; off = align256(off + NL * R * 4);
  L.fetch = off; off = align256(off + NL * R * W * 8);
  L.pf_miss_count = off; off = align256(off + NL * R * 4);
  L.pf_fetch = off; off = align256(off + NL * R * W * 8);
  L.fill_mask = off; off = align256(off + NL * R * ((W + 63) / 64) * 8);
  L.bt = off; off = align256(off + (size_t)bt_entries * 4);
  L.bt_off = off; off = align256(off + R * 4);
  L.ctx = off; off = align256(off + R * 4);
  L.cap = off; off = align256(off + R * 4);
  L.hv = off; off = align256(off + NL * R * 4);
  L.host_rows = off; off = align256(off + NL * R * 8);
  L.kv_ptrs = off; off = align256(off + NL * 8);
  L.kv_scale = off; off = align256(off + NL * 4);
  L.err = off; off = align256(off + 4);
  L.fallback_count = off; off = align256(off + 4);
  L.partial = off; off = align256(off + part * 4);
  int64_t ctx_sum = 0;
  for (size_t r = 0; r < R; ++r) ctx_sum += capacity_of(c, (int)r);
  L.posmap_entries = (int64_t)NL * ctx_sum;
  L.posmap = off; off = align256(off + (size_t)L.posmap_entries * 2);
  L.map_off = off; off = align256(off + R * 8);
  L.total = off;
  return L;
}

hisparse_status check_ptr(const void* p, size_t align, const char* what) {
  if (!p) {
    set_error(std::string(what) + " is NULL");
    return HISPARSE_EINVAL;
  }
  if ((uintptr_t)p % align) {
    set_error(std::string(what) + " is not " + std::to_string(align) + "-byte aligned");
    return HISPARSE_EINVAL;
  }
  return HISPARSE_OK;
}

}  // namespace

void set_error(const std::string& msg) { g_last_error = msg; }

hisparse_status hip_fail(hipError_t e, const char* what) {
  g_last_error = std::string(what) + ": " + hipGetErrorString(e);
  return HISPARSE_EHIP;
}

void prof_begin(hisparse_pool* p, int kid, hipStream_t s) {
  Profiler& pr = p->prof;
  if (!pr.on) return;
  if (pr.n >= kProfCap) {
    pr.overflow = true;
    return;
  }
  pr.kid[pr.n] = kid;
  (void)hipEventRecord(pr.ev[2 * pr.n], s);
}

void prof_end(hisparse_pool* p, hipStream_t s) {
  Profiler& pr = p->prof;
  if (!pr.on || pr.n >= kProfCap) return;
  (void)hipEventRecord(pr.ev[2 * pr.n + 1], s);
  ++pr.n;
}

}  // namespace hs

using namespace hs;

extern "C" {

const char* hisparse_last_error(void) { return g_last_error.c_str(); }

hisparse_status hisparse_workspace_bytes(const hisparse_config* cfg, size_t* bytes) {
  hisparse_status st = check_config(cfg);
  if (st) return st;
  if (!bytes) {
    set_error("bytes is NULL");
    return HISPARSE_EINVAL;
  }
  *bytes = make_layout(cfg).total;
  return HISPARSE_OK;
}

hisparse_status hisparse_kv_rows_per_layer(const hisparse_config* cfg, int64_t* rows) {
  hisparse_status st = check_config(cfg);
  if (st) return st;
  if (!rows) {
    set_error("rows is NULL");
    return HISPARSE_EINVAL;
  }
  *rows = cfg->resident_rows_per_layer + (int64_t)cfg->num_requests * cfg->hot_slots;
  return HISPARSE_OK;
}

hisparse_status hisparse_create_pool(const hisparse_config* cfg, void* d_workspace, size_t ws_bytes,
                                     void* const* d_kv, void* stream, hisparse_pool** out) {
  hisparse_status st = check_config(cfg);
  if (st) return st;
  if (!out) {
    set_error("out is NULL");
    return HISPARSE_EINVAL;
  }
  *out = nullptr;
  if ((st = check_ptr(d_workspace, 256, "d_workspace"))) return st;
  if (!d_kv) {
    set_error("d_kv is NULL");
    return HISPARSE_EINVAL;
  }
  for (int l = 0; l < cfg->num_layers; ++l)
    if ((st = check_ptr(d_kv[l], 16, "d_kv[l]"))) return st;
  const Layout lay = make_layout(cfg);
  if (ws_bytes < lay.total) {
    set_error("workspace too small: need " + std::to_string(lay.total) + " bytes");
    return HISPARSE_EINVAL;
  }
  if (cfg->host_pool_limit < 0) {
    set_error("host_pool_limit must be >= 0");
    return HISPARSE_EINVAL;
  }
  if (cfg->host_pool_limit > 0) {
    const int64_t rb = cfg->kv_dtype == HISPARSE_KV_FP8_E4M3 ? kRowBytesFp8 : kRowBytes;
    int64_t need = 0;
    for (int r = 0; r < cfg->num_requests; ++r) need += (int64_t)cfg->num_layers * capacity_of(cfg, r) * rb;
    if (need > cfg->host_pool_limit) {
      set_error("the pinned host pool needs " + std::to_string(need) + " bytes, above host_pool_limit " +
                std::to_string(cfg->host_pool_limit));
      return HISPARSE_ENOMEM;
    }
  }
  hipStream_t s = (hipStream_t)stream;

  hisparse_pool* p = new (std::nothrow) hisparse_pool();
  if (!p) {
    set_error("out of host memory");
    return HISPARSE_ENOMEM;
  }
  p->cfg = *cfg;
  const int R = cfg->num_requests, NL = cfg->num_layers;
  p->ctx.assign(cfg->ctx_len, cfg->ctx_len + R);
  p->cfg.ctx_len = p->ctx.data();
  p->cap.resize(R);
  for (int r = 0; r < R; ++r) p->cap[r] = capacity_of(cfg, r);
  p->cfg.ctx_capacity = p->cap.data();
  p->lay = lay;
  p->ws = (char*)d_workspace;
  p->kv.resize(NL);
  for (int l = 0; l < NL; ++l) p->kv[l] = (unsigned char*)d_kv[l];
  p->row_bytes = cfg->kv_dtype == HISPARSE_KV_FP8_E4M3 ? kRowBytesFp8 : kRowBytes;
  p->kv_scale.assign(NL, 1.f);
  if (cfg->kv_scale && cfg->kv_dtype == HISPARSE_KV_FP8_E4M3)
    for (int l = 0; l < NL; ++l) p->kv_scale[l] = cfg->kv_scale[l];
  p->cfg.kv_scale = p->kv_scale.data();
  p->kv_rows = cfg->resident_rows_per_layer + (int64_t)R * cfg->hot_slots;
  p->T = verify_tokens(cfg);
  p->W = p->T * cfg->top_k;
  hipError_t e = hipGetDevice(&p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetDevice");
  }
  e = static_scratch_address(p->device, &p->static_scratch);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipGetSymbolAddress(static split scratch)");
  }
  p->resolve_lds = resolve_lds_bytes(p->W, cfg->hot_slots, false, p->T == 1);
  int max_lds = 0;
  e = hipDeviceGetAttribute(&max_lds, hipDeviceAttributeMaxSharedMemoryPerBlock, p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  p->max_lds = max_lds;
  e = hipDeviceGetAttribute(&p->num_cus, hipDeviceAttributeMultiprocessorCount, p->device);
  if (e != hipSuccess) {
    delete p;
    return hip_fail(e, "hipDeviceGetAttribute");
  }
  if ((size_t)max_lds < p->resolve_lds) {
    set_error("resolve needs " + std::to_string(p->resolve_lds) + " bytes of LDS, device allows " +
              std::to_string(max_lds));
    delete p;
    return HISPARSE_EDEVICE;
  }
  {
    // allow the largest metadata launch of any policy that fits the device
    const size_t lds_random = resolve_lds_bytes(p->W, cfg->hot_slots, true, p->T == 1);
    const size_t lim = lds_random <= (size_t)max_lds ? lds_random : p->resolve_lds;
    if (lim > 65536 && (e = set_resolve_lds_limit(p->device, lim)) != hipSuccess) {
      delete p;
      return hip_fail(e, "hipFuncSetAttribute(resolve LDS)");
    }
  }

  // Pinned, device-mapped host pool: one allocation per request holding
  // its L layers back to back.
  const unsigned flags = hipHostMallocMapped | (cfg->host_coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
  p->host_alloc.assign(R, nullptr);
  p->host_rows.assign((size_t)NL * R, nullptr);
  p->host_rows_dev.assign((size_t)NL * R, 0);
  for (int r = 0; r < R; ++r) {
    const size_t per_layer = (size_t)p->cap[r] * p->row_bytes;
    void* h = nullptr;
    e = hipHostMalloc(&h, per_layer * NL, flags);
    if (e != hipSuccess || !h) {
      (void)hipGetLastError();
      set_error("hipHostMalloc of " + std::to_string(per_layer * NL) + " bytes failed for request " +
                std::to_string(r));
      hisparse_destroy_pool(p);
      return HISPARSE_ENOMEM;
    }
    p->host_alloc[r] = h;
    void* dptr = nullptr;
    e = hipHostGetDevicePointer(&dptr, h, 0);
    if (e != hipSuccess) {
      hisparse_destroy_pool(p);
      return hip_fail(e, "hipHostGetDevicePointer");
    }
    for (int l = 0; l < NL; ++l) {
      p->host_rows[(size_t)l * R + r] = (unsigned char*)h + per_layer * l;
      p->host_rows_dev[(size_t)l * R + r] = (uint64_t)((char*)dptr + per_layer * l);
    }
  }

  // Carve the workspace.
  char* w = p->ws;
  p->owner = (int32_t*)(w + lay.owner);
  p->stamp = (int32_t*)(w + lay.stamp);
  p->lru = (int32_t*)(w + lay.lru);
  p->last_t = (int32_t*)(w + lay.last_t);
  p->miss_count = (int32_t*)(w + lay.miss_count);
  p->fetch = (int2*)(w + lay.fetch);
  p->pf_miss_count = (int32_t*)(w + lay.pf_miss_count);
  p->pf_fetch = (int2*)(w + lay.pf_fetch);
  p->fill_mask = (uint64_t*)(w + lay.fill_mask);
  p->mask_words = (p->W + 63) / 64;
  p->bt = (int32_t*)(w + lay.bt);
  p->bt_off = (int32_t*)(w + lay.bt_off);
  p->ctx_d = (int32_t*)(w + lay.ctx);
  p->cap_d = (int32_t*)(w + lay.cap);
  p->hv_d = (int32_t*)(w + lay.hv);
  p->host_rows_d = (uint64_t*)(w + lay.host_rows);
  p->kv_d = (unsigned char**)(w + lay.kv_ptrs);
  p->kv_scale_d = (float*)(w + lay.kv_scale);
  p->err = (uint32_t*)(w + lay.err);
  p->partial = (float*)(w + lay.partial);
  p->fallback_count = (uint32_t*)(w + lay.fallback_count);
  p->posmap = (int16_t*)(w + lay.posmap);
  p->map_off = (int64_t*)(w + lay.map_off);

  std::vector<int32_t> bt_off(R), ctx32(R), cap32(R);
  std::vector<int64_t> map_off(R);
  int64_t acc_m = 0;
  for (int r = 0; r < R; ++r) {
    map_off[r] = acc_m;
    acc_m += p->cap[r];
  }
  p->n_pages.resize(R);
  int64_t acc = 0;
  for (int r = 0; r < R; ++r) {
    bt_off[r] = (int32_t)acc;
    p->n_pages[r] = (int32_t)((p->cap[r] + cfg->page_size - 1) / cfg->page_size);
    acc += p->n_pages[r];
    ctx32[r] = (int32_t)p->ctx[r];
    cap32[r] = (int32_t)p->cap[r];
  }
  p->init_ctx32 = ctx32;
  p->init_hv32.resize((size_t)NL * R);
  for (int l = 0; l < NL; ++l)
    for (int r = 0; r < R; ++r) p->init_hv32[(size_t)l * R + r] = ctx32[r];
  std::vector<uint64_t> kvp(NL);
  for (int l = 0; l < NL; ++l) kvp[l] = (uint64_t)p->kv[l];
  if ((e = hipMemcpyAsync(p->bt_off, bt_off.data(), R * 4, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(p->map_off, map_off.data(), R * 8, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(p->cap_d, cap32.data(), R * 4, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(p->host_rows_d, p->host_rows_dev.data(), (size_t)NL * R * 8, hipMemcpyHostToDevice, s)) !=
          hipSuccess ||
      (e = hipMemcpyAsync(p->kv_d, kvp.data(), (size_t)NL * 8, hipMemcpyHostToDevice, s)) != hipSuccess ||
      (e = hipMemcpyAsync(p->kv_scale_d, p->kv_scale.data(), (size_t)NL * 4, hipMemcpyHostToDevice, s)) !=
          hipSuccess ||
      (e = launch_workspace_init(p, s)) != hipSuccess || (e = hipStreamSynchronize(s)) != hipSuccess) {
    hisparse_destroy_pool(p);
    return hip_fail(e, "workspace initialisation");
  }
  // Side stream and events of the overlapped step (default priority).
  p->ev_fetch.assign(cfg->index_share - 1 + kMaxTailChunks, nullptr);
  if ((e = hipStreamCreateWithFlags(&p->fetch_stream, hipStreamNonBlocking)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&p->ev_meta, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventCreateWithFlags(&p->ev_prefetch, hipEventDisableTiming)) != hipSuccess) {
    hisparse_destroy_pool(p);
    return hip_fail(e, "stream/event creation");
  }
  for (auto& ev : p->ev_fetch) {
    if ((e = hipEventCreateWithFlags(&ev, hipEventDisableTiming)) != hipSuccess) {
      hisparse_destroy_pool(p);
      return hip_fail(e, "event creation");
    }
  }
  *out = p;
  return HISPARSE_OK;
}

void hisparse_destroy_pool(hisparse_pool* p) {
  if (!p) return;
  (void)hipDeviceSynchronize();
  for (hipEvent_t e : p->prof.ev) (void)hipEventDestroy(e);
  for (hipEvent_t e : p->ev_fetch)
    if (e) (void)hipEventDestroy(e);
  if (p->ev_meta) (void)hipEventDestroy(p->ev_meta);
  if (p->ev_prefetch) (void)hipEventDestroy(p->ev_prefetch);
  if (p->fetch_stream) (void)hipStreamDestroy(p->fetch_stream);
  for (void* h : p->host_alloc)
    if (h) (void)hipHostFree(h);
  delete p;
}

void* hisparse_host_rows(hisparse_pool* p, int32_t r, int32_t l) {
  if (!p || r < 0 || r >= p->cfg.num_requests || l < 0 || l >= p->cfg.num_layers) {
    set_error("hisparse_host_rows: bad argument");
    return nullptr;
  }
  return p->host_rows[(size_t)l * p->cfg.num_requests + r];
}

hisparse_status hisparse_set_block_table(hisparse_pool* p, int32_t r, const int32_t* host_bt, int32_t n_pages,
                                         void* stream) {
  if (!p || !host_bt || r < 0 || r >= p->cfg.num_requests) {
    set_error("hisparse_set_block_table: bad argument");
    return HISPARSE_EINVAL;
  }
  if (n_pages != p->n_pages[r]) {
    set_error("hisparse_set_block_table: n_pages must be ceil(capacity_r / page_size) = " +
              std::to_string(p->n_pages[r]));
    return HISPARSE_EINVAL;
  }
  const int64_t nblocks = p->cfg.resident_rows_per_layer / p->cfg.page_size;
  for (int i = 0; i < n_pages; ++i) {
    if (host_bt[i] < -1 || host_bt[i] >= nblocks) {
      set_error("hisparse_set_block_table: block id out of range at page " + std::to_string(i));
      return HISPARSE_EINVAL;
    }
  }
  int32_t off = 0;
  for (int i = 0; i < r; ++i) off += p->n_pages[i];
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(p->bt + off, host_bt, (size_t)n_pages * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_set_block_table");
}

namespace {
// prefetch: the metadata pass of a prefetch (d_rows unused, d_counts
// [n_layers][R][4] or NULL, miss lists in the prefetch arrays).
hisparse_status enqueue_resolve(hisparse_pool* p, int32_t layer_begin, int32_t n_layers, const int32_t* d_step,
                                const int32_t* d_topk, int32_t* d_rows, int32_t* d_counts, hipStream_t s,
                                bool prefetch = false) {
  ResolveArgs a;
  a.prefetch = prefetch ? 1 : 0;
  a.step = d_step;
  a.topk = d_topk;
  a.rows = d_rows;
  a.counts = d_counts;
  a.owner = p->owner;
  a.stamp = p->stamp;
  a.lru = p->lru;
  a.last_t = p->last_t;
  a.miss_count = (prefetch ? p->pf_miss_count : p->miss_count) + (size_t)layer_begin * p->cfg.num_requests;
  a.fetch = (prefetch ? p->pf_fetch : p->fetch) + (size_t)layer_begin * p->cfg.num_requests * p->W;
  a.bt = p->bt;
  a.bt_off = p->bt_off;
  a.ctx = p->ctx_d;
  a.err = p->err;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.num_requests = p->cfg.num_requests;
  a.top_k = p->W;
  a.tok_k = p->cfg.top_k;
  a.hot_slots = p->cfg.hot_slots;
  int ps = 0;
  while ((1 << ps) < p->cfg.page_size) ++ps;
  a.page_shift = ps;
  a.resident_rows = p->cfg.resident_rows_per_layer;
  a.policy = p->policy;
  a.policy_seed = p->policy_seed;
  // The fill mask serves the decode that fetches and the two-part decode.
  a.fill_mask = !prefetch ? p->fill_mask + (size_t)layer_begin * p->cfg.num_requests * p->mask_words : nullptr;
  a.posmap = p->posmap;
  a.map_off = p->map_off;
  a.map_layer_stride = p->lay.posmap_entries / p->cfg.num_layers;
  hipError_t e = launch_meta(p, a, s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "resolve metadata launch");
}

// Miss fetch of requests [r0, r0 + nreq) of layers [layer, layer +
// n_layers) (nreq < R only with one layer): their miss lists, stored per
// (layer, request) by the metadata kernel, are copied from the host pool.
hisparse_status enqueue_fetch(hisparse_pool* p, int32_t layer, int32_t n_layers, int32_t r0, int32_t nreq, int grid,
                              hipStream_t s, bool prefetch = false) {
  const int R = p->cfg.num_requests;
  FetchArgs f;
  f.miss_count = (prefetch ? p->pf_miss_count : p->miss_count) + (size_t)layer * R + r0;
  f.fetch = (prefetch ? p->pf_fetch : p->fetch) + ((size_t)layer * R + r0) * p->W;
  f.host_rows = p->host_rows_d;
  f.kv = p->kv_d;
  f.layer_begin = layer;
  f.n_pairs = n_layers * nreq;
  f.num_requests = nreq;
  f.request_begin = r0;
  f.total_requests = R;
  f.top_k = p->W;
  f.hot_slots = p->cfg.hot_slots;
  f.row_chunks = p->row_bytes / 16;
  f.resident_rows = p->cfg.resident_rows_per_layer;
  f.hv = p->hv_d;
  f.err = p->err;
  hipError_t e = launch_fetch(p, f, grid, s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "miss fetch launch");
}

// splits: key-range splits per (layer, request, head group); 0 picks the
// count that fills the GPU (decode_splits).
// nreq: query sets per layer covered by the pointers -- requests times
// verify tokens, for all requests or a chunk of them when one layer is
// decoded piecewise.
// use_static: split partials in the fixed device array instead of the
// workspace (hisparse_sparse_mla_decode_layers_static).
// part: one part of a layer decoded resident rows first -- part 1 (rows in
// place before the step's fetch) or 2 (rows it fills) -- writing partial
// slots [split_base, split_base + splits) of split_total, merged by
// combine_splits after the launch of part 2; or, with merge_from > 0, part
// 2 in one launch that merges part 1's slots [0, merge_from) itself.
// fetch_sel: non-null when the decode fetches the rows this step fills
// from the host pool (the launch's selection, [R][K]).
struct PartSpec {
  int part = 0, split_base = 0, split_total = 0, merge_from = 0, head_group = 0;
  bool combine = true;
  const int32_t* fetch_sel = nullptr;
};

hisparse_status enqueue_decode(hisparse_pool* p, int32_t layer_begin, int32_t n_layers, int32_t nreq,
                               const uint16_t* d_q, const int32_t* d_rows, float scale, float* d_out, float* d_lse,
                               hipStream_t s, int splits = 0, bool use_static = false, PartSpec ps = PartSpec()) {
  DecodeArgs a;
  a.q = d_q;
  a.rows = d_rows;
  a.kv = p->kv_d;
  a.kv_scale = p->kv_scale_d;
  a.kv_dtype = p->cfg.kv_dtype;
  a.out = d_out;
  a.lse = d_lse;
  a.partial = use_static ? p->static_scratch : p->partial;
  a.fallback_count = p->fallback_count;
  a.err = p->err;
  a.layer_begin = layer_begin;
  a.n_layers = n_layers;
  a.num_requests = nreq;
  a.num_heads = p->cfg.num_heads;
  a.top_k = p->cfg.top_k;
  a.splits = splits > 0 ? splits : decode_splits(n_layers, nreq, p->cfg.num_heads, p->cfg.top_k);
  a.split_base = ps.split_base;
  a.split_total = ps.split_total > 0 ? ps.split_total : a.splits;
  a.out_partial = a.split_total > 1 || ps.part == 1 ? 1 : 0;
  a.part = ps.part;
  a.merge_from = ps.merge_from;
  a.head_group = ps.head_group;
  a.fetch = ps.fetch_sel != nullptr ? 1 : 0;
  a.tokens = (int32_t)p->T;
  a.sel = ps.fetch_sel;
  a.host_rows = p->host_rows_d;
  a.hv = p->hv_d;
  a.total_requests = p->cfg.num_requests;
  a.hot_slots = p->cfg.hot_slots;
  a.resident_rows = p->cfg.resident_rows_per_layer;
  a.mask_words = p->mask_words;
  a.fill_mask = p->fill_mask + ((size_t)layer_begin * p->cfg.num_requests) * p->mask_words;
  if ((ps.part != 0 && (n_layers != 1 || nreq != p->cfg.num_requests || p->T != 1)) ||
      (ps.merge_from > 0 && (a.splits != 1 || a.split_total != 1 || ps.merge_from > kMaxMergeSlots)) ||
      (a.fetch && (ps.part != 0 || (size_t)nreq != (size_t)p->cfg.num_requests * p->T))) {
    set_error("bad two-part decode launch");
    return HISPARSE_EINVAL;
  }
  const size_t part_floats =
      a.out_partial ? (size_t)a.split_total * n_layers * nreq * p->cfg.num_heads * kPartW : 0;
  if (use_static && part_floats * sizeof(float) > HISPARSE_STATIC_SCRATCH_BYTES) {
    set_error("decode launch needs " + std::to_string(part_floats * sizeof(float)) +
              " bytes of split partials; the static scratch holds " +
              std::to_string(HISPARSE_STATIC_SCRATCH_BYTES));
    return HISPARSE_EINVAL;
  }
  if (!use_static && part_floats > p->lay.partial_floats) {
    // cannot happen for the launches the workspace is sized for; refuse
    // rather than write past the partial region
    set_error("decode launch needs more split partials than the workspace holds");
    return HISPARSE_EINVAL;
  }
  a.kv_rows = p->kv_rows;
  a.scale_log2 = scale * 1.4426950408889634f;
  hipError_t e = launch_decode(p, a, s, ps.combine);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "decode launch");
}
}  // namespace

hisparse_status hisparse_resolve(hisparse_pool* p, int32_t layer_begin, int32_t n_layers, const int32_t* d_step,
                                 const int32_t* d_topk, int32_t* d_rows, int32_t* d_counts, void* stream) {
  if (!p || !d_step || !d_topk || !d_rows || !d_counts) {
    set_error("hisparse_resolve: NULL argument");
    return HISPARSE_EINVAL;
  }
  const int g = p->cfg.index_share;
  if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > p->cfg.num_layers ||
      layer_begin / g != (layer_begin + n_layers - 1) / g) {
    set_error("hisparse_resolve: layers must lie inside one index-share group");
    return HISPARSE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  hisparse_status st = enqueue_resolve(p, layer_begin, n_layers, d_step, d_topk, d_rows, d_counts, s);
  if (st) return st;
  return enqueue_fetch(p, layer_begin, n_layers, 0, p->cfg.num_requests, p->fetch_wg_all, s);
}

hisparse_status hisparse_sparse_mla_decode(hisparse_pool* p, int32_t layer, const uint16_t* d_q,
                                           const int32_t* d_rows, float scale, float* d_out, float* d_lse,
                                           void* stream) {
  if (!p || !d_q || !d_rows || !d_out || !d_lse) {
    set_error("hisparse_sparse_mla_decode: NULL argument");
    return HISPARSE_EINVAL;
  }
  if (layer < 0 || layer >= p->cfg.num_layers) {
    set_error("hisparse_sparse_mla_decode: layer out of range");
    return HISPARSE_EINVAL;
  }
  if ((uintptr_t)d_q % 16) {
    set_error("hisparse_sparse_mla_decode: d_q must be 16-byte aligned");
    return HISPARSE_EINVAL;
  }
  if (!std::isfinite(scale)) {
    set_error("hisparse_sparse_mla_decode: scale must be finite");
    return HISPARSE_EINVAL;
  }
  return enqueue_decode(p, layer, 1, p->cfg.num_requests * p->T, d_q, d_rows, scale, d_out, d_lse,
                        (hipStream_t)stream);
}

namespace {
hisparse_status decode_layers_impl(const char* fn, hisparse_pool* p, int32_t layer_begin, int32_t n_layers,
                                   const uint16_t* d_q, const int32_t* d_rows, float scale, float* d_out,
                                   float* d_lse, void* stream, bool use_static) {
  const std::string f(fn);
  if (!p || !d_q || !d_rows || !d_out || !d_lse) {
    set_error(f + ": NULL argument");
    return HISPARSE_EINVAL;
  }
  const int g = p->cfg.index_share;
  if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > p->cfg.num_layers ||
      layer_begin / g != (layer_begin + n_layers - 1) / g) {
    set_error(f + ": layers must lie inside one index-share group");
    return HISPARSE_EINVAL;
  }
  if ((uintptr_t)d_q % 16) {
    set_error(f + ": d_q must be 16-byte aligned");
    return HISPARSE_EINVAL;
  }
  if (!std::isfinite(scale)) {
    set_error(f + ": scale must be finite");
    return HISPARSE_EINVAL;
  }
  return enqueue_decode(p, layer_begin, n_layers, p->cfg.num_requests * p->T, d_q, d_rows, scale, d_out, d_lse,
                        (hipStream_t)stream, 0, use_static);
}
}  // namespace

hisparse_status hisparse_sparse_mla_decode_layers(hisparse_pool* p, int32_t layer_begin, int32_t n_layers,
                                                  const uint16_t* d_q, const int32_t* d_rows, float scale, float* d_out,
                                                  float* d_lse, void* stream) {
  return decode_layers_impl("hisparse_sparse_mla_decode_layers", p, layer_begin, n_layers, d_q, d_rows, scale, d_out,
                            d_lse, stream, false);
}

hisparse_status hisparse_sparse_mla_decode_layers_static(hisparse_pool* p, int32_t layer_begin, int32_t n_layers,
                                                         const uint16_t* d_q, const int32_t* d_rows, float scale,
                                                         float* d_out, float* d_lse, void* stream) {
  return decode_layers_impl("hisparse_sparse_mla_decode_layers_static", p, layer_begin, n_layers, d_q, d_rows, scale,
                            d_out, d_lse, stream, true);
}

namespace {
// The prefetch part of hisparse_step_prefetch: for every index-share group,
// the metadata pass over the predicted selection and the fetch of the filled
// rows, on the side stream fs, then an event the caller's stream joins.
hisparse_status enqueue_step_prefetch(hisparse_pool* p, const int32_t* d_step, const int32_t* d_next,
                                      int32_t* d_pf_counts, hipStream_t fs) {
  const auto& c = p->cfg;
  const size_t R = c.num_requests, W = p->W;
  const int G = c.index_share;
  for (int g = 0; g < c.num_layers / G; ++g) {
    const int l0 = g * G;
    hisparse_status st = enqueue_resolve(p, l0, G, d_step, d_next + (size_t)g * R * W, nullptr,
                                         d_pf_counts ? d_pf_counts + (size_t)l0 * R * 4 : nullptr, fs, true);
    if (st) return st;
    if ((st = enqueue_fetch(p, l0, G, 0, (int)R, p->fetch_wg_unit, fs, true))) return st;
  }
  hipError_t e = hipEventRecord(p->ev_prefetch, fs);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "prefetch event");
}

// One decode step (hisparse_step); with d_next, also the prefetch of the
// predicted next selections on the side stream, behind the step's own
// fetches and beside its decodes (hisparse_step_prefetch).
//
// The prefetch is enqueued on the side stream right after the last group's
// own fetches (with the fetch in the decode: its metadata kernel) and before
// that group's decodes.  It writes only the hot rows of slots this step did
// not touch and its own miss lists, so it races with nothing the step reads.
// Enqueued in that order, a captured graph keeps the prefetch on the
// fetches' chain (one queue) and the decodes on their own: enqueued after
// the decodes, the prefetch became a third chain that a graph launch queued
// ahead of the decodes, serialising them behind its fetch.
// A step with a prefetch decodes its last group in unsplit launches that
// leave the prefetch's copy kPrefetchCopyCUs compute units (its 32
// workgroups fill the host link), where a layer has at least
// kPrefetchLayerWorkgroups (query set, head group) workgroups.
constexpr int kPrefetchLayerWorkgroups = 32;
constexpr int kPrefetchCopyCUs = 32;

// One index-share group of a step with the fetch in the decode: the
// metadata kernel, then one decode launch over the group's layers that
// reads the rows the step fills straight from the host pool (and writes
// them to their hot rows), on `s` alone.  With a prefetch (d_next), the
// last group forks it onto the side stream after its metadata kernel, and
// decodes in unsplit launches of as many layers as leave the prefetch's
// copy its CUs: a launch over the whole group would hold every CU, and the
// copy, which needs few, would wait for it.
hisparse_status fetching_group(hisparse_pool* p, int g, const int32_t* d_step, const int32_t* d_topk,
                               const int32_t* d_next, const uint16_t* d_q, float scale, int32_t* d_rows,
                               int32_t* d_counts, float* d_out, float* d_lse, int32_t* d_pf_counts, hipStream_t s,
                               const std::string& f) {
  const auto& c = p->cfg;
  const size_t R = c.num_requests, K = c.top_k, H = c.num_heads, T = p->T, W = p->W;
  const int G = c.index_share, l0 = g * G;
  const bool last = g + 1 == c.num_layers / G;
  hisparse_status st = enqueue_resolve(p, l0, G, d_step, d_topk + (size_t)g * R * W, d_rows + (size_t)l0 * R * W,
                                       d_counts + (size_t)l0 * R * 3, s);
  if (st) return st;
  if (d_next && last) {
    hipError_t e;
    if ((e = hipEventRecord(p->ev_meta, s)) != hipSuccess ||
        (e = hipStreamWaitEvent(p->fetch_stream, p->ev_meta, 0)) != hipSuccess)
      return hip_fail(e, (f + ": fork").c_str());
    if ((st = enqueue_step_prefetch(p, d_step, d_next, d_pf_counts, p->fetch_stream))) return st;
  }
  PartSpec ps;
  ps.fetch_sel = d_topk + (size_t)g * R * W;
  const int lw = layer_workgroups((int)(R * T), (int)H);
  int per = G, splits = fetch_decode_splits(G, (int)(R * T), (int)H, (int)K);
  if (d_next && last && G > 1 && lw >= kPrefetchLayerWorkgroups && G * lw > p->num_cus - kPrefetchCopyCUs) {
    per = std::max(1, (p->num_cus - kPrefetchCopyCUs) / lw);
    splits = 1;
  }
  for (int i = 0; i < G; i += per) {
    const int n = std::min(per, G - i);
    const size_t pr = (size_t)(l0 + i) * R * T;  // first query set of the launch
    if ((st = enqueue_decode(p, l0 + i, n, (int)(R * T), d_q + pr * H * kLatent, d_rows + pr * K, scale,
                             d_out + pr * H * kVDim, d_lse + pr * H, s, splits, false, ps)))
      return st;
  }
  return HISPARSE_OK;
}

hisparse_status step_impl(const char* fn, hisparse_pool* p, const int32_t* d_step, const int32_t* d_topk,
                          const int32_t* d_next, const uint16_t* d_q, float scale, int32_t* d_rows,
                          int32_t* d_counts, float* d_out, float* d_lse, int32_t* d_pf_counts, void* stream) {
  const std::string f(fn);
  if (!p || !d_step || !d_topk || !d_q || !d_rows || !d_counts || !d_out || !d_lse) {
    set_error(f + ": NULL argument");
    return HISPARSE_EINVAL;
  }
  if ((uintptr_t)d_q % 16 || !std::isfinite(scale)) {
    set_error(f + ": d_q must be 16-byte aligned and scale finite");
    return HISPARSE_EINVAL;
  }
  const auto& c = p->cfg;
  const size_t R = c.num_requests, K = c.top_k, H = c.num_heads;
  const size_t T = p->T, W = p->W;  // verify tokens; the decode sees R * T query sets per layer
  const int G = c.index_share;
  hipStream_t s = (hipStream_t)stream;
  hipStream_t fs = p->fetch_stream;
  const int C = std::min<int>(p->tail_chunks, (int)R);
  const bool pf = d_next != nullptr;
  // The group's last layer in two parts: the rows in place before its fetch
  // are decoded beside the fetch, the fetched rows after it.
  const bool rf = T == 1 && C == 1 &&
                  (p->resident_first > 0 || (p->resident_first == 0 && resident_first_pays((int)R, (int)H)));
  int rf_before = 1, rf_after = 0;
  if (rf) resident_first_splits((int)R, (int)H, (int)K, &rf_before, &rf_after);
  // The fetch in the decode (fetching_group) takes every step without
  // tail chunks unless hisparse_set_pipeline switched it off.
  const bool fused = C == 1 && p->fetch_in_decode >= 0;
  hipError_t e;
  for (int g = 0; g < c.num_layers / G; ++g) {
    const int l0 = g * G;
    if (fused) {
      hisparse_status st = fetching_group(p, g, d_step, d_topk, d_next, d_q, scale, d_rows, d_counts, d_out, d_lse,
                                          d_pf_counts, s, f);
      if (st) return st;
      continue;
    }
    // One metadata launch for the whole group (its layers share the
    // selection).  Then a pipeline of units on two streams: the side stream
    // fetches unit after unit, the caller's stream decodes unit u as soon
    // as its fetch is done, overlapping the fetches of the units after it.
    // Units: each layer but the last, whole; the last layer in C request
    // chunks, so that only the last chunk's decode is exposed.  A whole
    // layer decoded under a later fetch runs unsplit (64 CUs or fewer, no
    // partials); chunks of the last layer are split to fill the GPU.
    hisparse_status st = enqueue_resolve(p, l0, G, d_step, d_topk + (size_t)g * R * W, d_rows + (size_t)l0 * R * W,
                                         d_counts + (size_t)l0 * R * 3, s);
    if (st) return st;
    if (G == 1 && C == 1 && !rf) {
      // One layer, one unit, decoded whole: its fetch and decode have
      // nothing to overlap, so they run on `stream` with the whole-group
      // fetch shape; a prefetch forks off after the fetch.
      const size_t pr = (size_t)l0 * R * T;  // first query set of the layer
      if ((st = enqueue_fetch(p, l0, 1, 0, (int)R, p->fetch_wg_all, s))) return st;
      if (pf && g + 1 == c.num_layers / G) {
        if ((e = hipEventRecord(p->ev_meta, s)) != hipSuccess || (e = hipStreamWaitEvent(fs, p->ev_meta, 0)) != hipSuccess)
          return hip_fail(e, (f + ": fork").c_str());
        if ((st = enqueue_step_prefetch(p, d_step, d_next, d_pf_counts, fs))) return st;
      }
      st = enqueue_decode(p, l0, 1, (int)(R * T), d_q + pr * H * kLatent, d_rows + pr * K, scale,
                          d_out + pr * H * kVDim, d_lse + pr * H, s);
      if (st) return st;
      continue;
    }
    if ((e = hipEventRecord(p->ev_meta, s)) != hipSuccess || (e = hipStreamWaitEvent(fs, p->ev_meta, 0)) != hipSuccess)
      return hip_fail(e, (f + ": fork").c_str());
    struct Unit {
      int layer, r0, nreq, splits;
    };
    Unit units[kMaxIndexShare - 1 + kMaxTailChunks];
    int nu = 0;
    for (int i = 0; i + 1 < G; ++i) units[nu++] = {l0 + i, 0, (int)R, 1};
    for (int ch = 0; ch < C; ++ch) {
      const int r0 = (int)(R * ch / C), r1 = (int)(R * (ch + 1) / C);
      units[nu++] = {l0 + G - 1, r0, r1 - r0, 0};
    }
    auto decode = [&](const Unit& un, int splits, PartSpec ps) {
      const size_t pr = ((size_t)un.layer * R + un.r0) * T;  // first query set of the unit
      return enqueue_decode(p, un.layer, 1, (int)(un.nreq * T), d_q + pr * H * kLatent, d_rows + pr * K, scale,
                            d_out + pr * H * kVDim, d_lse + pr * H, s, splits, false, ps);
    };
    if (rf) {
      // Part 1 of the last layer: its entries whose rows are in place
      // before this step's fetches (which never write them), decoded
      // beside the group's first fetch.
      PartSpec ps;
      ps.part = 1;
      ps.split_total = rf_before + rf_after;
      ps.combine = false;
      if ((st = decode(units[nu - 1], rf_before, ps))) return st;
    }
    for (int u = 0; u < nu; ++u) {
      if ((st = enqueue_fetch(p, units[u].layer, 1, units[u].r0, units[u].nreq, p->fetch_wg_unit, fs))) return st;
      if ((e = hipEventRecord(p->ev_fetch[u], fs)) != hipSuccess) return hip_fail(e, (f + ": fetch event").c_str());
    }
    if (pf && g + 1 == c.num_layers / G && (st = enqueue_step_prefetch(p, d_step, d_next, d_pf_counts, fs))) return st;
    for (int u = 0; u < nu; ++u) {
      if ((e = hipStreamWaitEvent(s, p->ev_fetch[u], 0)) != hipSuccess) return hip_fail(e, (f + ": join").c_str());
      if (rf && u + 1 == nu) {
        // Part 2: the entries the fetch filled, merged with part 1.
        PartSpec ps;
        ps.part = 2;
        if (rf_after == 0) {
          ps.merge_from = rf_before;
          ps.head_group = 16;
          if ((st = decode(units[u], 1, ps))) return st;
        } else {
          ps.split_base = rf_before;
          ps.split_total = rf_before + rf_after;
          if ((st = decode(units[u], rf_after, ps))) return st;
        }
        continue;
      }
      if ((st = decode(units[u], units[u].splits, PartSpec()))) return st;
    }
  }
  // `stream` waits for the prefetch, which also joins the fork for capture.
  if (pf && (e = hipStreamWaitEvent(s, p->ev_prefetch, 0)) != hipSuccess)
    return hip_fail(e, (f + ": prefetch join").c_str());
  return HISPARSE_OK;
}
}  // namespace

hisparse_status hisparse_step(hisparse_pool* p, const int32_t* d_step, const int32_t* d_topk, const uint16_t* d_q,
                              float scale, int32_t* d_rows, int32_t* d_counts, float* d_out, float* d_lse,
                              void* stream) {
  return step_impl("hisparse_step", p, d_step, d_topk, nullptr, d_q, scale, d_rows, d_counts, d_out, d_lse, nullptr,
                   stream);
}

hisparse_status hisparse_step_prefetch(hisparse_pool* p, const int32_t* d_step, const int32_t* d_topk,
                                       const int32_t* d_topk_next, const uint16_t* d_q, float scale, int32_t* d_rows,
                                       int32_t* d_counts, float* d_out, float* d_lse, int32_t* d_pf_counts,
                                       void* stream) {
  if (!d_topk_next) {
    set_error("hisparse_step_prefetch: d_topk_next is NULL");
    return HISPARSE_EINVAL;
  }
  return step_impl("hisparse_step_prefetch", p, d_step, d_topk, d_topk_next, d_q, scale, d_rows, d_counts, d_out,
                   d_lse, d_pf_counts, stream);
}

hisparse_status hisparse_prefetch(hisparse_pool* p, int32_t layer_begin, int32_t n_layers, const int32_t* d_step,
                                  const int32_t* d_topk, int32_t* d_counts, void* stream) {
  if (!p || !d_step || !d_topk) {
    set_error("hisparse_prefetch: NULL argument");
    return HISPARSE_EINVAL;
  }
  const int g = p->cfg.index_share;
  if (layer_begin < 0 || n_layers < 1 || layer_begin + n_layers > p->cfg.num_layers ||
      layer_begin / g != (layer_begin + n_layers - 1) / g) {
    set_error("hisparse_prefetch: layers must lie inside one index-share group");
    return HISPARSE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  hisparse_status st = enqueue_resolve(p, layer_begin, n_layers, d_step, d_topk, nullptr, d_counts, s, true);
  if (st) return st;
  return enqueue_fetch(p, layer_begin, n_layers, 0, p->cfg.num_requests, p->fetch_wg_all, s, true);
}

hisparse_status hisparse_reset_state(hisparse_pool* p, void* stream) {
  if (!p) {
    set_error("hisparse_reset_state: pool is NULL");
    return HISPARSE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipStreamSynchronize(p->fetch_stream);
  if (e == hipSuccess) e = launch_state_reset(p, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_reset_state");
}

hisparse_status hisparse_append(hisparse_pool* p, const void* d_rows, void* stream) {
  if (!p || !d_rows) {
    set_error("hisparse_append: NULL argument");
    return HISPARSE_EINVAL;
  }
  if ((uintptr_t)d_rows % 16) {
    set_error("hisparse_append: d_rows must be 16-byte aligned");
    return HISPARSE_EINVAL;
  }
  AppendArgs a;
  a.rows = (const unsigned char*)d_rows;
  a.row_chunks = p->row_bytes / 16;
  a.kv = p->kv_d;
  a.ctx = p->ctx_d;
  a.capacity = p->cap_d;
  a.bt = p->bt;
  a.bt_off = p->bt_off;
  a.err = p->err;
  a.num_layers = p->cfg.num_layers;
  a.num_requests = p->cfg.num_requests;
  a.page_shift = ilog2_exact(p->cfg.page_size);
  hipError_t e = launch_append(p, a, (hipStream_t)stream);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_append");
}

hisparse_status hisparse_writeback(hisparse_pool* p, void* stream) {
  if (!p) {
    set_error("hisparse_writeback: pool is NULL");
    return HISPARSE_EINVAL;
  }
  WritebackArgs a;
  a.row_chunks = p->row_bytes / 16;
  a.kv = p->kv_d;
  a.host_rows = p->host_rows_d;
  a.ctx = p->ctx_d;
  a.hv = p->hv_d;
  a.bt = p->bt;
  a.bt_off = p->bt_off;
  a.err = p->err;
  a.num_layers = p->cfg.num_layers;
  a.num_requests = p->cfg.num_requests;
  a.page_shift = ilog2_exact(p->cfg.page_size);
  hipError_t e = launch_writeback(p, a, (hipStream_t)stream);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_writeback");
}

hisparse_status hisparse_get_lengths(hisparse_pool* p, int32_t* host_ctx, int32_t* host_held, void* stream) {
  if (!p || !host_ctx || !host_held) {
    set_error("hisparse_get_lengths: NULL argument");
    return HISPARSE_EINVAL;
  }
  const size_t R = p->cfg.num_requests, L = p->cfg.num_layers;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(host_ctx, p->ctx_d, R * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(host_held, p->hv_d, L * R * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_get_lengths");
}

hisparse_status hisparse_set_pages(hisparse_pool* p, int32_t r, int32_t first_page, int32_t n,
                                   const int32_t* host_blocks, void* stream) {
  if (!p || !host_blocks || r < 0 || r >= p->cfg.num_requests || first_page < 0 || n < 1 ||
      first_page + n > p->n_pages[r]) {
    set_error("hisparse_set_pages: bad argument");
    return HISPARSE_EINVAL;
  }
  const int64_t nblocks = p->cfg.resident_rows_per_layer / p->cfg.page_size;
  for (int i = 0; i < n; ++i) {
    if (host_blocks[i] < -1 || host_blocks[i] >= nblocks) {
      set_error("hisparse_set_pages: block id out of range at page " + std::to_string(first_page + i));
      return HISPARSE_EINVAL;
    }
  }
  hipStream_t s = (hipStream_t)stream;
  const size_t R = p->cfg.num_requests, L = p->cfg.num_layers;
  int32_t off = 0;
  for (int i = 0; i < r; ++i) off += p->n_pages[i];
  // A page may become a placeholder only once every layer's host pool holds
  // every position of it that exists (the write-back has run), so that a
  // later miss reads correct rows.
  std::vector<int32_t> held(L * R), cur(n);
  int32_t ctx_now = 0;
  hipError_t e = hipMemcpyAsync(held.data(), p->hv_d, L * R * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(cur.data(), p->bt + off + first_page, (size_t)n * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(&ctx_now, p->ctx_d + r, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hisparse_set_pages");
  int64_t min_held = INT64_MAX;
  for (size_t l = 0; l < L; ++l) min_held = std::min<int64_t>(min_held, held[l * R + r]);
  for (int i = 0; i < n; ++i) {
    // positions of the page that exist so far
    const int64_t page_end = std::min<int64_t>((int64_t)(first_page + i + 1) * p->cfg.page_size, ctx_now);
    if (host_blocks[i] < 0 && cur[i] >= 0 && page_end > min_held) {
      set_error("hisparse_set_pages: page " + std::to_string(first_page + i) +
                " is not yet held by the host pool (run hisparse_writeback after it completes)");
      return HISPARSE_EINVAL;
    }
  }
  e = hipMemcpyAsync(p->bt + off + first_page, host_blocks, (size_t)n * 4, hipMemcpyHostToDevice, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_set_pages");
}

hisparse_status hisparse_set_replacement(hisparse_pool* p, int32_t policy, uint64_t seed, void* stream) {
  if (!p || (policy != HISPARSE_POLICY_LRU && policy != HISPARSE_POLICY_FIFO && policy != HISPARSE_POLICY_RANDOM)) {
    set_error("hisparse_set_replacement: bad argument");
    return HISPARSE_EINVAL;
  }
  if (policy == HISPARSE_POLICY_RANDOM) {
    // random replacement sorts the unpinned slots in LDS beside the miss list
    const size_t need = resolve_lds_bytes(p->W, p->cfg.hot_slots, true, p->T == 1);
    if (need > (size_t)p->max_lds) {
      set_error("hisparse_set_replacement: random replacement needs " + std::to_string(need) +
                " bytes of LDS at this selection width and slot count, the device allows " +
                std::to_string(p->max_lds));
      return HISPARSE_EDEVICE;
    }
  }
  p->policy = policy;
  p->policy_seed = seed;
  return hisparse_reset_state(p, stream);
}

hisparse_status hisparse_set_pipeline(hisparse_pool* p, int32_t group_fetch_workgroups,
                                      int32_t unit_fetch_workgroups, int32_t tail_chunks, int32_t resident_first,
                                      int32_t fetch_in_decode) {
  if (!p || group_fetch_workgroups < 0 || group_fetch_workgroups > 65536 || unit_fetch_workgroups < 0 ||
      unit_fetch_workgroups > 65536 || tail_chunks < 0 || tail_chunks > kMaxTailChunks || resident_first < -1 ||
      resident_first > 1 || fetch_in_decode < -1 || fetch_in_decode > 1) {
    set_error("hisparse_set_pipeline: bad argument");
    return HISPARSE_EINVAL;
  }
  p->fetch_wg_all = group_fetch_workgroups > 0 ? group_fetch_workgroups : kDefaultGroupFetchWorkgroups;
  p->fetch_wg_unit = unit_fetch_workgroups > 0 ? unit_fetch_workgroups : kDefaultUnitFetchWorkgroups;
  p->tail_chunks = tail_chunks > 0 ? tail_chunks : kDefaultTailChunks;
  p->resident_first = resident_first;
  p->fetch_in_decode = fetch_in_decode;
  return HISPARSE_OK;
}

hisparse_status hisparse_export_state(hisparse_pool* p, int32_t r, int32_t l, int32_t* host_owner,
                                      int32_t* host_stamp, void* stream) {
  if (!p || !host_owner || !host_stamp || r < 0 || r >= p->cfg.num_requests || l < 0 || l >= p->cfg.num_layers) {
    set_error("hisparse_export_state: bad argument");
    return HISPARSE_EINVAL;
  }
  const size_t B = p->cfg.hot_slots;
  const size_t pair = (size_t)l * p->cfg.num_requests + r;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipMemcpyAsync(host_owner, p->owner + pair * B, B * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(host_stamp, p->stamp + pair * B, B * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_export_state");
}

hisparse_status hisparse_check_errors(hisparse_pool* p, void* stream, uint32_t* flags) {
  if (!p || !flags) {
    set_error("hisparse_check_errors: bad argument");
    return HISPARSE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, p->err, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemsetAsync(p->err, 0, 4, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hisparse_check_errors");
  *flags = v;
  return HISPARSE_OK;
}

hisparse_status hisparse_decode_fallback_count(hisparse_pool* p, void* stream, int64_t* count) {
  if (!p || !count) {
    set_error("hisparse_decode_fallback_count: bad argument");
    return HISPARSE_EINVAL;
  }
  hipStream_t s = (hipStream_t)stream;
  uint32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, p->fallback_count, 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess) e = hipMemsetAsync(p->fallback_count, 0, 4, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e, "hisparse_decode_fallback_count");
  *count = v;
  return HISPARSE_OK;
}

hisparse_status hisparse_profile_enable(hisparse_pool* p, int32_t enable) {
  if (!p) {
    set_error("hisparse_profile_enable: pool is NULL");
    return HISPARSE_EINVAL;
  }
  Profiler& pr = p->prof;
  if (enable && pr.ev.empty()) {
    pr.ev.resize(2 * kProfCap);
    pr.kid.resize(kProfCap);
    for (auto& e : pr.ev) {
      hipError_t err = hipEventCreate(&e);
      if (err != hipSuccess) return hip_fail(err, "hipEventCreate");
    }
  }
  pr.on = enable != 0;  // launches recorded so far are kept until the next read
  return HISPARSE_OK;
}

hisparse_status hisparse_profile_read(hisparse_pool* p, hisparse_kernel_time* out, int32_t max, int32_t* n) {
  static const char* names[kKCount] = {"resolve_meta", "fetch_rows", "sparse_mla_decode", "combine_splits",
                                       "sparse_mla_decode_fetch"};
  if (!p || !out || !n || max < 0) {
    set_error("hisparse_profile_read: bad argument");
    return HISPARSE_EINVAL;
  }
  Profiler& pr = p->prof;
  double total[kKCount] = {};
  int cnt[kKCount] = {};
  for (int i = 0; i < pr.n; ++i) {
    hipError_t e = hipEventSynchronize(pr.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
    float ms = 0.f;
    e = hipEventElapsedTime(&ms, pr.ev[2 * i], pr.ev[2 * i + 1]);
    if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
    total[pr.kid[i]] += ms;
    cnt[pr.kid[i]] += 1;
  }
  const bool overflow = pr.overflow;
  pr.n = 0;
  pr.overflow = false;
  int k = 0;
  for (int i = 0; i < kKCount; ++i) {
    if (!cnt[i]) continue;
    if (k < max) out[k] = hisparse_kernel_time{names[i], cnt[i], total[i]};
    ++k;
  }
  *n = k < max ? k : max;
  if (overflow) {
    set_error("hisparse_profile_read: more than 8192 launches since the last read; later ones were not timed");
    return HISPARSE_ESTATE;
  }
  return HISPARSE_OK;
}

hisparse_status hisparse_host_alloc(size_t bytes, int32_t coherent, void** host, void** dev) {
  if (!host || !dev || bytes == 0) {
    set_error("hisparse_host_alloc: bad argument");
    return HISPARSE_EINVAL;
  }
  const unsigned flags = hipHostMallocMapped | (coherent ? hipHostMallocCoherent : hipHostMallocNonCoherent);
  void* h = nullptr;
  hipError_t e = hipHostMalloc(&h, bytes, flags);
  if (e != hipSuccess || !h) {
    (void)hipGetLastError();
    set_error("hipHostMalloc failed");
    return HISPARSE_ENOMEM;
  }
  void* d = nullptr;
  e = hipHostGetDevicePointer(&d, h, 0);
  if (e != hipSuccess) {
    (void)hipHostFree(h);
    return hip_fail(e, "hipHostGetDevicePointer");
  }
  *host = h;
  *dev = d;
  return HISPARSE_OK;
}

void hisparse_host_free(void* host) {
  if (host) (void)hipHostFree(host);
}

hisparse_status hisparse_stream_copy(void* dst, const void* src, size_t bytes, void* stream) {
  if (!dst || !src || bytes % 16 || (uintptr_t)dst % 16 || (uintptr_t)src % 16) {
    set_error("hisparse_stream_copy: pointers and size must be 16-byte multiples");
    return HISPARSE_EINVAL;
  }
  if (bytes == 0) return HISPARSE_OK;
  hipError_t e = launch_stream_copy(dst, src, bytes, (hipStream_t)stream);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_stream_copy");
}

hisparse_status hisparse_row_gather(void* dst, const void* src, const int64_t* d_rows, int64_t n_rows,
                                    int32_t row_bytes, void* stream) {
  if (!dst || !src || (n_rows > 0 && !d_rows) || n_rows < 0 || row_bytes <= 0 || row_bytes % 16 ||
      (uintptr_t)dst % 16 || (uintptr_t)src % 16 || (uintptr_t)d_rows % 8) {
    set_error("hisparse_row_gather: bad argument (16-byte aligned pointers, row_bytes a positive multiple of 16)");
    return HISPARSE_EINVAL;
  }
  if (n_rows == 0) return HISPARSE_OK;
  hipError_t e = launch_row_gather(dst, src, d_rows, n_rows, row_bytes, (hipStream_t)stream);
  return e == hipSuccess ? HISPARSE_OK : hip_fail(e, "hisparse_row_gather");
}

}  // extern "C"
