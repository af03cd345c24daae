// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "hisparse.h"

namespace hs {

constexpr int kLatent = 576;         // values per KV row
constexpr int kVDim = 512;           // value width (the "nope" part)
constexpr int kRowBytes = kLatent * 2;      // bf16 row
constexpr int kRowChunks = kRowBytes / 16;  // 16-byte chunks per bf16 row (72)
constexpr int kRowBytesFp8 = kLatent;       // FP8 E4M3 row (36 chunks)
constexpr int kPartW = kVDim + 4;           // split partial: o[512], m, l (rounded weights), l (exact), pad
constexpr int kMaxTopK = 4096;       // K: entries of one token's selection
constexpr int kMaxSelection = 8192;  // T * K: entries one RESOLVE covers (verify tokens concatenated)
constexpr int kMaxHotSlots = 16384;  // B (slot ids stay below 2^15: the position map is int16)
constexpr int kMaxHeads = 256;
// Workgroups of the miss fetch: a whole-group fetch (hisparse_resolve) owns
// the GPU; a per-layer fetch of the overlapped step leaves most CUs to the
// decode running beside it.
constexpr int kDefaultGroupFetchWorkgroups = 256;
constexpr int kDefaultUnitFetchWorkgroups = 32;
// The last layer of an index-share group can be fetched and decoded in
// request chunks, so that only the last chunk's decode is exposed; each
// chunk's decode then pays the per-workgroup cost (Q load, partial write)
// over fewer key tiles, which on MI355X made 2 or more chunks slower.
constexpr int kDefaultTailChunks = 1;
constexpr int kMaxTailChunks = 16;
constexpr int kMaxIndexShare = 64;

// Per-launch description of the fan-out copy of missed rows.
// Pair pr of a launch is (layer layer_begin + pr / num_requests, request
// request_begin + pr % num_requests); its miss list is pr of the arrays.
struct FetchArgs {
  const int32_t* miss_count;   // [n_pairs]
  const int2* fetch;           // [n_pairs][K] (position, slot)
  const uint64_t* host_rows;   // [L*R] device-visible address of pool rows of (l, r)
  unsigned char* const* kv;    // [L] device pointers of the KV tensors (device array)
  const int32_t* hv;           // [L][R] positions below hv[l][r] are held by the host pool
  uint32_t* err;
  int32_t layer_begin;
  int32_t n_pairs;             // layers * num_requests
  int32_t num_requests;        // requests per layer in this launch
  int32_t request_begin;
  int32_t total_requests;      // R of the pool
  int32_t top_k;
  int32_t hot_slots;
  int32_t row_chunks;          // 16-byte chunks per row (72 bf16, 36 FP8)
  int64_t resident_rows;
};

// Append of one token per request (all layers) into the tail page.
struct AppendArgs {
  const unsigned char* rows;   // [L][R] new rows
  unsigned char* const* kv;    // [L] device array of KV tensor pointers
  int32_t* ctx;                // [R] current context lengths (advanced)
  const int32_t* capacity;     // [R]
  const int32_t* bt;           // concatenated block tables
  const int32_t* bt_off;       // [R]
  uint32_t* err;
  int32_t num_layers;
  int32_t num_requests;
  int32_t page_shift;
  int32_t row_chunks;
};

// Copy of completed pages from their resident blocks to the host pool.
struct WritebackArgs {
  unsigned char* const* kv;    // [L]
  const uint64_t* host_rows;   // [L*R] device-visible address of the pool rows of (l, r)
  const int32_t* ctx;          // [R]
  int32_t* hv;                 // [L][R] (advanced)
  const int32_t* bt;
  const int32_t* bt_off;
  uint32_t* err;
  int32_t num_layers;
  int32_t num_requests;
  int32_t page_shift;
  int32_t row_chunks;
};

struct ResolveArgs {
  const int32_t* step;     // device scalar t
  const int32_t* topk;     // [R][K]
  int32_t* rows;           // [n_layers][R][K]
  int32_t* counts;         // [n_layers][R][3]
  int32_t* owner;          // [L][R][B]
  int32_t* stamp;          // [L][R][B]
  int32_t* lru;            // [L][R][B] slots in ascending (stamp, slot)
  int32_t* last_t;         // [L][R]
  int32_t* miss_count;     // [n_layers][R] (pair order of this call)
  int2* fetch;             // [n_layers][R][K]
  const int32_t* bt;       // concatenated block tables
  const int32_t* bt_off;   // [R]
  const int32_t* ctx;      // [R]
  uint32_t* err;
  int32_t layer_begin;
  int32_t n_layers;
  int32_t num_requests;
  int32_t top_k;            // selection width: num_verify * K
  int32_t tok_k;            // K: entries per verify token (a repeat inside one token's list is an error)
  int32_t hot_slots;
  int32_t page_shift;
  int64_t resident_rows;
  int32_t policy;           // HISPARSE_POLICY_*
  uint64_t policy_seed;     // random replacement: SplitMix64 seed
  int32_t prefetch;         // 1: prefetch of a predicted selection (no row ids; slots stamped t are
                            // pinned; hits pinned without a stamp; misses beyond the free slots
                            // dropped); counts then holds [n_layers][R][4] (resident, hit, filled,
                            // dropped) or is NULL
  uint64_t* fill_mask;      // [n_layers][R][ceil(top_k / 64)]: bit j set when entry j's row is filled by
                            // this call (a miss); NULL: not written
  int16_t* posmap;          // [L][sum ctx] position -> slot (-1: not in the hot buffer)
  const int64_t* map_off;   // [R] offset of request r within a layer's map
  int64_t map_layer_stride; // sum of ctx_r
};

struct DecodeArgs {
  const uint16_t* q;       // [n_layers][R][H][576]
  const int32_t* rows;     // [n_layers][R][K]
  const unsigned char* const* kv;  // [L] device array of KV tensor pointers
  const float* kv_scale;   // [L] FP8 row scales (device)
  float* out;              // [n_layers][R][H][512]
  float* lse;              // [n_layers][R][H]
  float* partial;          // [n_layers][R][split_total][H][kPartW] when split_total > 1
  uint32_t* fallback_count;  // workgroups that took the exact fp32 path (read and cleared by the host)
  uint32_t* err;
  int32_t layer_begin;
  int32_t n_layers;
  int32_t num_requests;
  int32_t num_heads;
  int32_t top_k;
  int32_t splits;          // key-range splits of this launch
  int32_t split_base;      // partial slot of the launch's split 0
  int32_t split_total;     // partial slots per (query set, head)
  int32_t out_partial;     // 1: the launch writes partial slots (merged later); 0: O and lse
  int32_t part;            // entries attended: 0 all; 1 those whose row was in place before this step's
                           // fetch (fill_mask bit clear); 2 those filled by it (bit set)
  const uint64_t* fill_mask;  // [n_layers][total_requests][mask_words], one bit per selection entry
                              // of a (layer, request), all verify tokens (part != 0, fetch)
  int32_t mask_words;
  int32_t head_group;      // heads per workgroup (16, 32 or 64); 0: the default for num_heads
  // Fetch in the decode: the entries this step fills (fill_mask) are read
  // from the host pool and written to their hot rows (rows holds those
  // rows' ids) by the head groups that read them.
  int32_t fetch;
  int32_t tokens;              // verify tokens: query set q is token q % tokens of request q / tokens
  const int32_t* sel;          // [R][top_k] positions of each query set (its layers share them)
  const uint64_t* host_rows;   // [L * total_requests] device-visible addresses of the host pool rows
  const int32_t* hv;           // [L][total_requests] positions below hv[l][r] are held by the host pool
  int32_t total_requests;
  int32_t hot_slots;
  int64_t resident_rows;       // rows of the KV tensor before the hot buffers
  int32_t merge_from;      // > 0: partial slots [0, merge_from) of every (query set, head), written by an
                           // earlier launch over other entries, are merged into this launch's O and lse
                           // (which then has one split and split_total 1)
  int64_t kv_rows;         // rows per KV tensor
  float scale_log2;        // scale * log2(e)
  int32_t kv_dtype;        // HISPARSE_KV_BF16 or HISPARSE_KV_FP8_E4M3
};

// Workspace carving, computed identically for sizing and for creation.
struct Layout {
  size_t owner, stamp, lru, last_t, miss_count, fetch, pf_miss_count, pf_fetch, fill_mask, bt, bt_off, ctx, cap, hv,
      host_rows, kv_ptrs, kv_scale, err, fallback_count, partial, posmap, map_off, total;
  int64_t bt_entries;
  int64_t posmap_entries;   // L * sum ctx_r
  size_t partial_floats;   // floats of the split-partial region
  int32_t splits_max;      // largest split count any decode launch uses
};

}  // namespace hs

namespace hs {
enum KernelId { kKMeta = 0, kKFetch = 1, kKDecode = 2, kKCombine = 3, kKDecodeFetch = 4, kKCount = 5 };
constexpr int kProfCap = 8192;
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<int> kid;
  int n = 0;
  bool overflow = false;
};
}  // namespace hs

struct hisparse_pool {
  hisparse_config cfg;
  hs::Profiler prof;
  std::vector<int64_t> ctx;             // context length at creation
  std::vector<int64_t> cap;             // capacity (host rows, block-table pages, map entries)
  std::vector<int32_t> n_pages;         // block-table pages per request: ceil(cap / page_size)
  std::vector<int32_t> init_ctx32;      // [R] lengths at creation (source of resets)
  std::vector<int32_t> init_hv32;       // [L][R] host-held prefix at creation (= ctx_len)
  int device = 0;
  hs::Layout lay;
  char* ws = nullptr;
  std::vector<void*> host_alloc;        // one pinned allocation per request
  std::vector<unsigned char*> host_rows;  // [L*R] host addresses (index l*R + r)
  std::vector<uint64_t> host_rows_dev;  // [L*R] device-visible addresses
  std::vector<unsigned char*> kv;       // [L]
  std::vector<float> kv_scale;          // [L] FP8 row scales (1 for bf16)
  int64_t kv_rows = 0;
  int32_t row_bytes = hs::kRowBytes;    // bytes per KV row (1152 bf16, 576 FP8)
  size_t resolve_lds = 0;
  int max_lds = 0;                      // LDS bytes per workgroup the device allows
  int num_cus = 0;                      // compute units of the device
  int32_t policy = HISPARSE_POLICY_LRU;
  uint64_t policy_seed = 0;
  int32_t T = 1;                        // verify tokens per request per step
  int32_t W = 0;                        // resolve selection width T * K
  // device views into the workspace
  int32_t *owner, *stamp, *lru, *last_t, *miss_count, *bt, *bt_off, *ctx_d, *cap_d, *hv_d;
  int16_t* posmap;
  int64_t* map_off;
  int2* fetch;
  int32_t* pf_miss_count;               // prefetch miss lists, apart from the step's own (a prefetch
  int2* pf_fetch;                       // runs while the step's fetch may still read those)
  uint64_t* fill_mask;                  // [L][R][mask_words] entries filled by the last RESOLVE
  int32_t mask_words = 0;               // ceil(K / 64)
  uint64_t* host_rows_d;
  unsigned char** kv_d;
  float* kv_scale_d;
  uint32_t* err;
  float* partial;
  float* static_scratch = nullptr;  // fixed split-partial array of this pool's device
  uint32_t* fallback_count;
  // Overlapped step: per-layer miss fetches run on fetch_stream (default
  // priority) while the caller's stream decodes earlier layers.
  hipStream_t fetch_stream = nullptr;
  hipEvent_t ev_meta = nullptr;
  hipEvent_t ev_prefetch = nullptr;     // end of the in-step prefetch on the side stream
  std::vector<hipEvent_t> ev_fetch;  // one per pipelined unit of an index-share group
  int fetch_wg_all = hs::kDefaultGroupFetchWorkgroups;   // workgroups of a whole-group fetch
  int fetch_wg_unit = hs::kDefaultUnitFetchWorkgroups;   // workgroups of a pipelined fetch
  int tail_chunks = hs::kDefaultTailChunks;              // request chunks of a group's last layer
  // A group's last layer decoded in two parts: rows in place before its
  // fetch (beside the fetches), then the fetched rows.  -1 never, 0 where
  // the part after the fetch fills enough workgroups, 1 always.
  int resident_first = 0;
  // hisparse_step reads the rows a step fills from the host pool inside the
  // decode (-1: separate fetches; 0, 1: where it applies).
  int fetch_in_decode = 0;
};

namespace hs {
void set_error(const std::string& msg);
hisparse_status hip_fail(hipError_t e, const char* what);

// profiling marks around a launch (no-ops unless enabled)
void prof_begin(hisparse_pool* p, int kid, hipStream_t s);
void prof_end(hisparse_pool* p, hipStream_t s);

// resolve.hip
size_t resolve_lds_bytes(int selection_width, int hot_slots, bool random_policy, bool one_token);
hipError_t launch_workspace_init(hisparse_pool* p, hipStream_t s);
hipError_t launch_state_reset(hisparse_pool* p, hipStream_t s);
hipError_t launch_meta(hisparse_pool* p, const ResolveArgs& a, hipStream_t s);
hipError_t launch_fetch(hisparse_pool* p, const FetchArgs& a, int grid, hipStream_t s);
hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s);
hipError_t launch_row_gather(void* dst, const void* src, const int64_t* rows, int64_t n_rows, int row_bytes,
                             hipStream_t s);

// residency.hip
hipError_t launch_append(hisparse_pool* p, const AppendArgs& a, hipStream_t s);
hipError_t launch_writeback(hisparse_pool* p, const WritebackArgs& a, hipStream_t s);

// decode.hip
int decode_splits(int n_layers, int num_requests, int num_heads, int top_k);
// Key splits of a decode that fetches the rows it fills (at most
// decode_splits, so the workspace's partials cover it).
int fetch_decode_splits(int n_layers, int num_requests, int num_heads, int top_k);
// (query set, head group) workgroups of one layer's unsplit decode.
int layer_workgroups(int num_requests, int num_heads);
// A layer decoded resident rows first: `before` key splits for the part
// beside the fetches; after the fetch either one launch without key splits
// that also merges the first part's partials (*after = 0), or `after` key
// splits and combine_splits.  resident_first_pays: whether the merging
// launch has enough workgroups (the default of hisparse_set_pipeline).
constexpr int kMaxMergeSlots = 4;
void resident_first_splits(int num_requests, int num_heads, int top_k, int* before, int* after);
bool resident_first_pays(int num_requests, int num_heads);
// Device address of the fixed split-partial array on `device` (which must
// be current), looked up once per device and kept.
hipError_t static_scratch_address(int device, float** out);
// combine: merge the split partials after the launch (when split_total > 1).
hipError_t launch_decode(hisparse_pool* p, const DecodeArgs& a, hipStream_t s, bool combine = true);
}  // namespace hs
