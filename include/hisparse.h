/*
 * hisparse.h -- C ABI of the MI355X (gfx950) HiSparse decode path.
 *
 * What the library computes (sources: the HiSparse summary article
 * "显存占用直降30倍！大模型稀疏注意力解码KV缓存方案HiSparse夯爆了", section 02,
 * and the vLLM blog "GLM 5.3 优化（一）：vLLM 的 Hybrid HiSparse 混合稀疏卸载",
 * section "工作原理"):
 *
 *   The full latent KV of every request and sparse layer lives in a pinned,
 *   device-mapped host pool.  On the device each (request, layer) owns a
 *   fixed buffer of B "hot" rows; a per-request block table marks 64-token
 *   pages that are GPU-resident (read in place, never evicted).  Every
 *   decode step the indexer names K logical positions per request; RESOLVE
 *   turns each into a row id of the layer's KV tensor:
 *     - position on a resident page  -> block * page_size + offset
 *     - position already in the hot buffer (hit) -> hot row, LRU refreshed
 *     - otherwise (miss) -> an LRU victim slot, whose row is fetched from
 *       the host pool by GPU loads over the host link.
 *   Sparse MLA decode attention then runs over the resolved rows.
 *
 * Row ids index one KV tensor per layer: rows [0, resident_rows_per_layer)
 * hold resident pages (block b = rows [b*page_size, (b+1)*page_size)), and
 * rows [resident_rows_per_layer + r*B, ... + B) are the hot rows of request
 * r.  A KV row is latent_dim = 576 values (512 "nope" + 64 rope), stored
 * as bf16 or as FP8 E4M3 codes with a per-layer scale (kv_dtype); the value
 * vector is its first v_dim = 512 values.
 *
 * Replacement rule (exact; the pages say only that LRU metadata drives
 * replacement and that the current selection must be served): every slot
 * starts empty (owner -1, stamp -1); a call at step t stamps every slot it
 * touches with t; slots hit or filled by a call cannot be evicted by the
 * same call; victims are the untouched slots with the smallest (stamp,
 * slot); the i-th smallest missing position fills the i-th victim.
 *
 * Conventions
 *   - Status: every function returns HISPARSE_OK (0) or a negative code;
 *     hisparse_last_error() gives a message for the calling thread's last
 *     failure.  No exception crosses the ABI.
 *   - Ownership: the caller owns every device buffer (workspace, KV tensors,
 *     inputs, outputs) and the stream; the library owns the pinned host pool
 *     and the opaque pool handle.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  resolve,
 *     decode and step only enqueue kernels (no host synchronisation, no
 *     allocation) and read the step index from device memory, so they can be
 *     captured in a HIP graph.  Calls on one stream run in order; a pool is
 *     not thread-safe.
 *   - Host-checkable errors (bad sizes, null pointers, B < K, ...) return
 *     HISPARSE_EINVAL and enqueue nothing.  Errors only the device can see
 *     set bits in a device flag word, read (and cleared) by
 *     hisparse_check_errors; the offending entry is treated as padding.
 */
#ifndef HISPARSE_H
#define HISPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t hisparse_status;
#define HISPARSE_OK 0
#define HISPARSE_EINVAL (-1) /* invalid argument or configuration */
#define HISPARSE_ENOMEM (-2) /* pinned host allocation failed */
#define HISPARSE_EHIP (-3)   /* a HIP runtime call failed */
#define HISPARSE_EDEVICE (-4) /* device does not support the launch (LDS, arch) */
#define HISPARSE_ESTATE (-5)  /* call not valid in the pool's state */

/* Device error flag bits (hisparse_check_errors). */
#define HISPARSE_ERR_RANGE 1u /* a selected position outside [-1, ctx_r) */
#define HISPARSE_ERR_DUP 2u   /* a position repeated within one token's selection (later copies dropped) */
#define HISPARSE_ERR_STEP 4u  /* step index negative or below the last one seen by a (request, layer) */
#define HISPARSE_ERR_ROW 8u   /* decode saw a row id outside the KV tensor (treated as padding) */
#define HISPARSE_ERR_APPEND 16u /* append with the tail page not resident or the context full (not appended) */
#define HISPARSE_ERR_UNMATERIALIZED 32u /* a row was needed from the host pool before it was written there */

/* KV row formats (hisparse_config.kv_dtype).  The vLLM Hybrid HiSparse blog
 * (measurements section) runs its benchmark with an FP8 KV cache; the blog
 * does not describe the format, so the reading here is the plainest one:
 * every latent value is one OCP FP8 E4M3 code (bias 7, no infinities, 0x7F
 * and 0xFF are NaN, largest finite 448), and the row of layer l stands for
 * x = decode(code) * kv_scale[l]. */
#define HISPARSE_KV_BF16 0     /* 576 bf16 values per row, 1152 bytes */
#define HISPARSE_KV_FP8_E4M3 1 /* 576 FP8 E4M3 codes per row, 576 bytes */

/* Replacement policies (hisparse_set_replacement). */
#define HISPARSE_POLICY_LRU 0    /* victims: least recently used first (default) */
#define HISPARSE_POLICY_FIFO 1   /* victims: earliest filled first; a hit does not refresh */
#define HISPARSE_POLICY_RANDOM 2 /* victims: empty slots, then a per-call random order */

typedef struct hisparse_pool hisparse_pool;

typedef struct {
  int32_t num_requests;  /* R >= 1 */
  int32_t num_layers;    /* L >= 1 sparse layers */
  int32_t index_share;   /* g: consecutive layers sharing one selection, 1..64; L % g == 0 */
  int32_t latent_dim;    /* must be 576 */
  int32_t v_dim;         /* must be 512 */
  int32_t top_k;         /* K: positions per selection, 1..4096 */
  int32_t hot_slots;     /* B: hot rows per (request, layer), num_verify * K <= B <= 16384 */
  int32_t page_size;     /* tokens per page, a power of two (64) */
  int32_t num_heads;     /* H: query heads, a multiple of 16, <= 256 */
  int32_t host_coherent; /* 0: coarse-grained (non-coherent) pinned pool, 1: coherent */
  int64_t resident_rows_per_layer; /* rows of each KV tensor reserved for resident pages (multiple of page_size) */
  const int64_t* ctx_len; /* [R] host array, context length per request (>= 1); copied */
  const int64_t* ctx_capacity; /* [R] host array or NULL (= ctx_len): the length the context may
                                  grow to by hisparse_append; sizes the host pool, the block
                                  table and the position map; copied */
  int32_t kv_dtype;      /* HISPARSE_KV_BF16 (0) or HISPARSE_KV_FP8_E4M3 (1): format of the
                            host pool rows and of the KV tensors */
  int32_t num_verify;    /* T >= 1 query tokens per request per step (1 + speculative tokens);
                            0 is read as 1.  T > 1 is multi-token verification (see below) */
  const float* kv_scale; /* [L] host array or NULL (= 1.0): scale of each layer's FP8 rows
                            (finite, > 0); ignored for bf16 rows; copied */
  int64_t host_pool_limit; /* bytes of pinned host memory the pool may take, 0 = no limit.  The
                              vLLM Hybrid HiSparse blog sizes the pinned pool per replica
                              (host_pool_gib, appendix "附录：复现我们的结果"); a pool needing
                              more (sum over r of L * capacity_r * row bytes) is refused with
                              HISPARSE_ENOMEM before anything is allocated */
} hisparse_config;

/* Multi-token verification (num_verify = T > 1).  The vLLM Hybrid HiSparse
 * blog says that speculative decoding runs through a per-step replayable
 * resolver plan whose verification steps share the request's hot state, and
 * that the hot buffer must hold every verification token at once.  Reading:
 * each step carries T query tokens per request (1 + speculative tokens),
 * each with its own K-entry selection; one RESOLVE per (request, layer)
 * covers the T selections concatenated (token-major, width T*K): a position
 * selected by several tokens is resolved once, at its earliest entry, and
 * every copy gets that row; a repeat inside one token's list is an error
 * (HISPARSE_ERR_DUP, padding).  Counts are over the distinct positions.
 * Requires T*K <= 8192 and B >= T*K (the blog sizes B = (T + 1) * K, so
 * MTP3 at K = 2048 is T = 4, B = 10240).
 * Selections, row ids, queries and outputs then carry a token axis after
 * the request axis: d_topk [..][R][T][K], d_rows [..][R][T][K],
 * d_q [..][R][T][H][576], d_out [..][R][T][H][512], d_lse [..][R][T][H];
 * d_counts stays [..][R][3]. */

/* Message describing the calling thread's last failure ("" if none). */
const char* hisparse_last_error(void);

/* Bytes of device workspace the caller must provide to hisparse_create_pool
 * (metadata, block tables, miss lists, attention partials). */
hisparse_status hisparse_workspace_bytes(const hisparse_config* cfg, size_t* bytes);

/* Rows each layer's KV tensor must have: resident_rows_per_layer + R * B. */
hisparse_status hisparse_kv_rows_per_layer(const hisparse_config* cfg, int64_t* rows);

/* Create a pool on the current device.  The pool is the two-level store
 * of the HiSparse summary article, section 02: the authoritative full KV of
 * every request and sparse layer in pinned host DRAM, and B device slots per
 * (request, layer) with a page table and LRU metadata.  The vLLM Hybrid
 * HiSparse blog ("与 vLLM 其余部分的组合", appendix "附录：复现我们的结果")
 * allocates that pinned pool per data-parallel replica, sized in whole host
 * blocks; here one pool serves one GPU's requests.
 *   d_workspace: device buffer of at least hisparse_workspace_bytes bytes,
 *                256-byte aligned; owned by the caller, must outlive the pool.
 *   d_kv:        host array of L device pointers; d_kv[l] is a tensor of
 *                [kv_rows_per_layer] rows in the pool's row format (576 bf16
 *                or 576 FP8 codes), 16-byte aligned, caller-owned.
 *   stream:      used to initialise the workspace (synchronised before return).
 * Allocates the pinned, device-mapped host pool: request r, layer l holds
 * capacity_r rows (filled by the caller via hisparse_host_rows).
 * Every slot starts empty and every page host-only.
 * Errors: EINVAL (bad config, null or misaligned pointers, workspace too
 * small), ENOMEM (the pool exceeds host_pool_limit, or the pinned
 * allocation failed), EHIP, EDEVICE. */
hisparse_status hisparse_create_pool(const hisparse_config* cfg, void* d_workspace, size_t ws_bytes,
                                     void* const* d_kv, void* stream, hisparse_pool** out);

/* Free the host pool and the handle (device buffers stay the caller's).
 * Synchronises the device first.  NULL is ignored. */
void hisparse_destroy_pool(hisparse_pool* pool);

/* Host address of the pool rows of (request r, layer l), [capacity_r] rows
 * in the pool's row format (bf16 bits [576] or FP8 E4M3 codes [576]),
 * row-major, for the caller to fill before resolving.  NULL on a bad
 * argument. */
void* hisparse_host_rows(hisparse_pool* pool, int32_t r, int32_t l);

/* Set the block table of request r (mixed residency, vLLM Hybrid HiSparse
 * blog, "工作原理": residency is tracked per page; resident pages are read in
 * place, the others are placeholders whose rows live in the host pool):
 * host_bt[page] is the resident block id
 * of that page, or -1 (host-only placeholder); n_pages must equal
 * ceil(capacity_r / page_size).  Block ids must satisfy
 * (id + 1) * page_size <= resident_rows_per_layer.  The library never edits
 * a block table, so resident pages (the tail included) are never evicted.
 * The caller must keep resident rows equal to the host rows they mirror.
 * Synchronous.  Errors: EINVAL. */
hisparse_status hisparse_set_block_table(hisparse_pool* pool, int32_t r, const int32_t* host_bt,
                                         int32_t n_pages, void* stream);

/* RESOLVE layers [layer_begin, layer_begin + n_layers), which share one
 * selection (they must lie in one index-share group).  RESOLVE is the fused
 * per-layer step of the HiSparse summary article, section 02 (hit
 * detection, LRU replacement, metadata update and host fetch; logical
 * positions in, physical rows out), with the residency rule of the vLLM
 * Hybrid HiSparse blog, "工作原理" (resident tokens read in place, hot
 * tokens refresh their LRU entry, a miss copies one row into an LRU slot).
 *   d_step:   device int32 scalar, the step index t (>= 0, non-decreasing
 *             per (request, layer)); read on the device.
 *   d_topk:   device int32 [R][K] logical positions, -1 = padding, any order.
 *   d_rows:   device int32 [n_layers][R][K] out: row id per entry (-1 for padding).
 *   d_counts: device int32 [n_layers][R][3] out: (resident, hit, miss).
 * Enqueues the metadata kernel (one 16-wavefront workgroup per (request,
 * layer)) and one miss fetch over all n_layers (zero-copy 16-byte loads
 * from the host pool into hot rows), both on `stream`. */
hisparse_status hisparse_resolve(hisparse_pool* pool, int32_t layer_begin, int32_t n_layers,
                                 const int32_t* d_step, const int32_t* d_topk, int32_t* d_rows,
                                 int32_t* d_counts, void* stream);

/* Sparse MLA decode attention of one layer over resolved rows.  The HiSparse
 * summary article, section 02, fixes that only the placement of KV changes:
 * selected positions, scores and outputs are those of attention over the
 * full KV (exactness); the vLLM Hybrid HiSparse blog (Fig. 1 text, "一个块池")
 * puts resident and hot rows in one KV tensor, so the kernel sees ordinary
 * rows.
 *   d_q:    device bf16 [R][H][576]
 *   d_rows: device int32 [R][K] row ids of this layer (-1 = skip)
 *   scale:  softmax scale applied to q . x
 *   d_out:  device fp32 [R][H][512] out: softmax(scale q X^T) X[:, :512]
 *   d_lse:  device fp32 [R][H] out: log-sum-exp of the scaled scores
 * A request with no valid row gets O = 0 and lse = -inf. */
hisparse_status hisparse_sparse_mla_decode(hisparse_pool* pool, int32_t layer, const uint16_t* d_q,
                                           const int32_t* d_rows, float scale, float* d_out,
                                           float* d_lse, void* stream);

/* Sparse MLA decode of layers [layer_begin, layer_begin + n_layers) in one
 * launch (the layers must lie in one index-share group, whose row-id
 * arrays hisparse_resolve fills together).  Same arithmetic as
 * hisparse_sparse_mla_decode per layer; a launch over several layers
 * needs fewer key splits to fill the GPU (none for 4 layers x 32 requests
 * x 128 heads).
 *   d_q [n_layers][R][H][576], d_rows [n_layers][R][K],
 *   d_out [n_layers][R][H][512], d_lse [n_layers][R][H].
 * Errors: EINVAL (layers outside one group, null or misaligned pointers). */
hisparse_status hisparse_sparse_mla_decode_layers(hisparse_pool* pool, int32_t layer_begin, int32_t n_layers,
                                                  const uint16_t* d_q, const int32_t* d_rows, float scale,
                                                  float* d_out, float* d_lse, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * launch as hisparse_sparse_mla_decode_layers, with the key-split partials
 * kept in a fixed device array of HISPARSE_STATIC_SCRATCH_BYTES that the
 * library holds on every GPU it runs on until the process ends, instead of
 * in the pool's workspace.  Allocates nothing.  Results are bit-identical
 * to hisparse_sparse_mla_decode_layers.  The array is shared by every pool
 * on a GPU and keeps the last call's contents (each launch writes every
 * partial it reads, so nothing needs clearing); calls that overlap on one
 * GPU -- on different streams, or under different pools -- race on it and
 * must be ordered by the caller.  Errors: EINVAL when the launch needs more
 * partials than the array holds (the message gives both sizes), and the
 * checks of hisparse_sparse_mla_decode_layers. */
#define HISPARSE_STATIC_SCRATCH_BYTES ((size_t)64 << 20)
hisparse_status hisparse_sparse_mla_decode_layers_static(hisparse_pool* pool, int32_t layer_begin, int32_t n_layers,
                                                         const uint16_t* d_q, const int32_t* d_rows, float scale,
                                                         float* d_out, float* d_lse, void* stream);

/* One decode step over every layer: for each index-share group, RESOLVE all
 * of its layers with the group's selection, then decode each layer.
 * By default (fetch_in_decode of hisparse_set_pipeline) the decode itself
 * reads the rows the step fills from the host pool, one launch per group;
 * the rest of this comment describes the pipeline of separate fetches.
 *   d_topk [L/g][R][K], d_q [L][R][H][576], d_rows [L][R][K],
 *   d_counts [L][R][3], d_out [L][R][H][512], d_lse [L][R][H].
 * Layer-ahead fetch (the shared selection of an index-share group is known
 * before the group's first layer is decoded; HiSparse summary article,
 * sections 03-04, on prefetch): after the group's metadata kernel, the miss
 * fetches run unit by unit on a stream the pool owns -- each layer but the
 * last whole, the last layer in request chunks (hisparse_set_pipeline) --
 * and the decode of a unit waits (by event) only for that unit's fetch, so
 * it overlaps the fetches of the units after it (a whole layer is decoded
 * without key splits, on few CUs; chunks of the last layer are split to
 * fill the GPU).  With one verify token and the last layer in one piece,
 * that layer can be decoded in two parts (resident_first of
 * hisparse_set_pipeline): its entries whose rows were already in place
 * (resident pages and hits, which no fetch of the step writes) right after
 * the metadata kernel, beside the group's fetches, then the entries its
 * fetch fills, and the two parts' sums are merged -- attention over a set
 * of keys splits into any partition (the summary article, section 02: the
 * outputs are those of attention over the selected keys, wherever they
 * live).  Otherwise a group of one layer fetched in one piece has nothing
 * to overlap and runs resolve, fetch and decode on `stream` alone.
 * `stream` waits for every fetch
 * before the call's last decode, so work enqueued on `stream` afterwards
 * sees the whole step; under graph capture the side stream is forked from
 * and joined back into `stream`.  Row ids, counts and the LRU state are
 * identical to hisparse_resolve followed by hisparse_sparse_mla_decode per
 * layer; O and lse agree to rounding (an unsplit layer sums its keys in
 * another order). */
hisparse_status hisparse_step(hisparse_pool* pool, const int32_t* d_step, const int32_t* d_topk,
                              const uint16_t* d_q, float scale, int32_t* d_rows, int32_t* d_counts,
                              float* d_out, float* d_lse, void* stream);

/* ---- cross-step prefetch (HiSparse summary article, sections 03-04:
 * fetching the rows a coming step will select before it asks for them
 * hides host I/O; a selection the model provides beats speculation) ----
 * The pages give the effect, not the mechanism.  Reading: a prefetch issued
 * during step t with a predicted selection S' (same layout as d_topk)
 * leaves every slot stamped t alone (the running step's selection, which
 * its attention may still read, and earlier fills of this step) and every
 * slot holding a position of S' (pinned, stamp unchanged); the positions of
 * S' neither resident nor in the buffer are filled, smallest first, into
 * the remaining slots in the policy's victim order, with stamp t, and
 * fetched from the host pool; misses beyond the free slots are dropped
 * (largest positions first).  No row ids are produced: the coming step's
 * RESOLVE finds the filled rows as hits.  With the exact next selection and
 * room for its misses, the next step has no miss and the same rows and
 * state as without prefetch.  Range and repeat errors set the same flags as
 * RESOLVE; a step index below the last one seen sets HISPARSE_ERR_STEP and
 * prefetches nothing. */

/* Prefetch S' into layers [layer_begin, layer_begin + n_layers) (one
 * index-share group) during the step whose index d_step holds.
 *   d_topk:   device int32 [R][T*K] predicted selection.
 *   d_counts: device int32 [n_layers][R][4] out, or NULL: (resident, hit,
 *             filled, dropped) per (layer, request).
 * Enqueues the metadata kernel and the fetch of the filled rows on
 * `stream`; the prefetch keeps its own miss lists, so it may overlap a
 * fetch of the running step.  Errors: EINVAL. */
hisparse_status hisparse_prefetch(hisparse_pool* pool, int32_t layer_begin, int32_t n_layers, const int32_t* d_step,
                                  const int32_t* d_topk, int32_t* d_counts, void* stream);

/* hisparse_step, followed by the prefetch of d_topk_next ([L/g][R][T*K],
 * the predicted selections of the next step) into every layer: the prefetch
 * runs on the pool's side stream after all of this step's metadata kernels
 * (with separate fetches: after its miss fetches) and beside the last
 * group's decode, and `stream` waits for it before the call's work ends
 * (graph-capturable like hisparse_step).  d_pf_counts: device int32
 * [L][R][4] out, or NULL (as hisparse_prefetch's d_counts).  Row ids,
 * counts, O and lse of this step are those of hisparse_step.
 * Errors: EINVAL. */
hisparse_status hisparse_step_prefetch(hisparse_pool* pool, const int32_t* d_step, const int32_t* d_topk,
                                       const int32_t* d_topk_next, const uint16_t* d_q, float scale, int32_t* d_rows,
                                       int32_t* d_counts, float* d_out, float* d_lse, int32_t* d_pf_counts,
                                       void* stream);

/* Return every (request, layer) to the empty state (owner -1, stamp -1,
 * no step seen) and every context to its length at creation (host pool
 * held up to that length); block tables and host rows are kept.  Waits for
 * the pool's own stream, enqueues memory fills (not graph-capturable) and
 * synchronises `stream`.  Errors: EINVAL, EHIP. */
hisparse_status hisparse_reset_state(hisparse_pool* pool, void* stream);

/* ---- residency transitions (vLLM Hybrid HiSparse blog, "工作原理") ----
 * Per request the device keeps the current context length ctx_r (starts
 * at ctx_len[r]) and, per layer, the length held_lr of the prefix the host
 * pool holds (starts at ctx_len[r]: the caller fills those host rows).
 * RESOLVE and decode read ctx_r on the device, so a step after appends
 * accepts the new positions. */

/* Append one token per request: d_rows [L][R] rows in the pool's row
 * format (16-byte aligned)
 * is the new token's latent row of every layer, written to the resident
 * block of the request's tail page (page ctx_r / page_size) at row ctx_r %
 * page_size; then ctx_r += 1.  The caller leases the tail block with
 * hisparse_set_pages before the append that starts a new page.  A request
 * whose tail page is a placeholder, or whose context is at capacity, is
 * left unchanged and sets HISPARSE_ERR_APPEND.  Enqueue only
 * (graph-capturable). */
hisparse_status hisparse_append(hisparse_pool* pool, const void* d_rows, void* stream);

/* Materialise completed pages: for every (layer, request), copy the rows
 * [held_lr, floor(ctx_r / page_size) * page_size) from their resident
 * blocks into the host pool (one launch for all layers, zero-copy 16-byte
 * stores), then held_lr = that bound.  The GPU keeps serving those pages;
 * afterwards they may be turned into placeholders without another copy.
 * A completed page that is already a placeholder sets
 * HISPARSE_ERR_UNMATERIALIZED and leaves held_lr.  Enqueue only
 * (graph-capturable). */
hisparse_status hisparse_writeback(hisparse_pool* pool, void* stream);

/* Change block-table entries [first_page, first_page + n) of request r:
 * host_blocks[i] is a resident block id or -1 (placeholder).  Turning a
 * resident page into a placeholder requires every layer's host pool to
 * hold every position of the page below ctx_r (after hisparse_writeback),
 * so that later misses read correct rows; otherwise EINVAL and nothing
 * changes.  A newly leased block
 * holds whatever the caller puts there (hisparse_append writes the rows of
 * the tail page).  Synchronises `stream`.  Errors: EINVAL, EHIP. */
hisparse_status hisparse_set_pages(hisparse_pool* pool, int32_t r, int32_t first_page, int32_t n,
                                   const int32_t* host_blocks, void* stream);

/* Read ctx_r ([R]) and held_lr ([L][R]) into host arrays.  Synchronises
 * `stream`.  Errors: EINVAL, EHIP. */
hisparse_status hisparse_get_lengths(hisparse_pool* pool, int32_t* host_ctx, int32_t* host_held, void* stream);

/* Replacement policy of every (request, layer), for the comparison in the
 * HiSparse summary article (section 04: LRU against FIFO and random
 * replacement).  All policies pin the current selection and fill the i-th
 * smallest missing position into the i-th victim; the victims are the
 * unpinned slots in ascending order of
 *   LRU:    (step of last use, slot);
 *   FIFO:   (step of the fill, slot) -- stamps hold fill steps;
 *   RANDOM: empty slots first (by slot), then (priority, slot), where the
 *           priority of slot s is SplitMix64(k ^ s) >> 33 with
 *           k = SplitMix64(SplitMix64(SplitMix64(seed) ^ t) ^ (layer << 32 | r))
 *           and SplitMix64(x) the generator's output for state x (add
 *           0x9E3779B97F4A7C15, then its mixing function).
 * Resets the pool to the empty state (as hisparse_reset_state, so it
 * synchronises `stream`).  Errors: EINVAL, EHIP. */
hisparse_status hisparse_set_replacement(hisparse_pool* pool, int32_t policy, uint64_t seed, void* stream);

/* Tuning of the fetch and of hisparse_step's pipeline (0 = default):
 *   group_fetch_workgroups: 1024-thread workgroups of the whole-group miss
 *     fetch of hisparse_resolve (default 256);
 *   unit_fetch_workgroups: workgroups of each pipelined fetch of
 *     hisparse_step (default 32), which leave the other CUs to the decode
 *     running beside them;
 *   tail_chunks: request chunks the last layer of an index-share group is
 *     fetched and decoded in (default 1, at most 16, capped at R);
 *   resident_first: with one verify token and one tail chunk, the last
 *     layer of an index-share group can be decoded in two parts -- the
 *     entries whose rows were in place before this step's fetches
 *     (resident pages and hits) beside the fetches, the entries its fetch
 *     fills after it -- with the parts' softmax sums merged.  With at least
 *     32 (request, head group) workgroups the second part is one launch
 *     without key splits that merges the first; with fewer, both parts are
 *     split and combine_splits merges them.  1: always; -1: never (one
 *     launch after the fetch); 0 (default): where the merging launch
 *     applies, i.e. with at least 32 such workgroups;
 *   fetch_in_decode: 0 or 1 (default): with one tail chunk,
 *     hisparse_step and hisparse_step_prefetch have no separate miss fetch:
 *     one decode launch per index-share group reads the rows the step fills
 *     straight from the pinned host pool into its tiles and writes them to
 *     their hot rows (with one verify token the head groups share the
 *     writes; with several, an entry that shares a filled row with an
 *     earlier token's entry reads it from the host pool too), so the step
 *     is the metadata kernel and that launch on `stream`; -1: separate
 *     fetches (the layer pipeline above).
 * Results do not depend on these settings, except the rounding of O and
 * lse of the chunked or two-part layer.  Errors: EINVAL. */
hisparse_status hisparse_set_pipeline(hisparse_pool* pool, int32_t group_fetch_workgroups,
                                      int32_t unit_fetch_workgroups, int32_t tail_chunks, int32_t resident_first,
                                      int32_t fetch_in_decode);

/* Copy the LRU state of (request r, layer l) -- the slot owners and LRU
 * stamps that the HiSparse summary article, section 02, keeps per device
 * slot -- to host arrays of B int32:
 * owner (logical position per slot, -1 empty) and stamp (step of last use,
 * -1 never).  Synchronises the stream.  Errors: EINVAL, EHIP. */
hisparse_status hisparse_export_state(hisparse_pool* pool, int32_t r, int32_t l, int32_t* host_owner,
                                      int32_t* host_stamp, void* stream);

/* Read and clear the device error flags (HISPARSE_ERR_* bits).  The pages
 * do not describe error handling; an indexer emits K distinct positions
 * (HiSparse summary article, section 01), so a repeat or an out-of-range
 * position is the caller's error, flagged here and treated as padding.
 * Synchronises the stream. */
hisparse_status hisparse_check_errors(hisparse_pool* pool, void* stream, uint32_t* flags);

/* Read and clear the number of decode workgroups (one per layer, query
 * set, head group and key split) that took the exact fp32 path since the
 * last call or pool creation.  The decode scores the bf16 values as given
 * and multiplies P by the V part (the first 512 values) of each row in fp16
 * (exact for bf16 values of magnitude below 2^16).  A workgroup whose rows
 * hold a V value of magnitude 2^16 or more, or whose rows or queries hold
 * an inf or a NaN (any staged row counts, also the filler row of a -1
 * entry), computes its result again in fp32 on the values as given, which
 * is correct but far slower.  A nonzero count
 * thus flags inputs outside the fast path; results do not depend on it
 * beyond rounding.  Synchronises the stream.  Errors: EINVAL, EHIP. */
hisparse_status hisparse_decode_fallback_count(hisparse_pool* pool, void* stream, int64_t* count);

/* ---- measurement helpers (not on the decode path) ---- */

/* Per-kernel timing with HIP events recorded on the launch stream around
 * every kernel the pool enqueues (resolve metadata "resolve_meta", miss
 * fetch "fetch_rows", decode "sparse_mla_decode", the decode that also
 * fetches "sparse_mla_decode_fetch", split merge "combine_splits").  Off
 * by default; while on, each launch adds two event
 * records.  Up to 8192 launches are kept between reads; switching the
 * profiler on or off keeps them.  Launches enqueued under HIP graph capture
 * record their events when the graph is replayed. */
typedef struct {
  const char* name;   /* kernel name (static storage) */
  int32_t launches;   /* launches timed since the last read */
  double total_ms;    /* summed event-measured duration */
} hisparse_kernel_time;

hisparse_status hisparse_profile_enable(hisparse_pool* pool, int32_t enable);
/* Synchronises on the recorded events, fills up to `max` entries (one per
 * kernel that ran) and clears the record.  *n receives the entry count. */
hisparse_status hisparse_profile_read(hisparse_pool* pool, hisparse_kernel_time* out, int32_t max, int32_t* n);

/* Pinned, device-mapped host buffer with the pool's flags; *host and *dev
 * receive the host address and the device-visible address. */
hisparse_status hisparse_host_alloc(size_t bytes, int32_t coherent, void** host, void** dev);
void hisparse_host_free(void* host);

/* Copy `bytes` (a multiple of 16) from src to dst with the same 16-byte
 * vector-load kernel the miss fetch uses; src may be a device-mapped host
 * address (zero-copy read over the host link) or device memory. */
hisparse_status hisparse_stream_copy(void* dst, const void* src, size_t bytes, void* stream);

/* Gather rows with the miss fetch's access pattern, for measuring the host
 * link under it: row i of dst (row_bytes bytes, a positive multiple of 16)
 * receives row d_rows[i] of src, for i < n_rows.  d_rows is a device array
 * of n_rows int64 indices, which the caller keeps within src (they are not
 * checked); src may be a device-mapped host address or device memory.
 * Pointers 16-byte aligned (d_rows 8).  Errors: EINVAL, EHIP. */
hisparse_status hisparse_row_gather(void* dst, const void* src, const int64_t* d_rows, int64_t n_rows,
                                    int32_t row_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* HISPARSE_H */
