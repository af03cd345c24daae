// RESOLVE for gfx950: hit detection, LRU replacement, metadata update and
// the host fetch of every miss.
//
// The operation follows the HiSparse summary article ("显存占用直降30倍！…
// HiSparse夯爆了", section 02: a fused RESOLVE per sparse layer over a B-slot
// device buffer with a position->slot page table and LRU metadata, rows
// fetched from pinned host memory on a miss) and the vLLM Hybrid HiSparse
// blog (section "工作原理": resident tokens read in place, hot tokens read
// with their LRU entry refreshed, a miss copies a single row into an LRU
// slot, nothing on the decode path waits for the CPU).
//
// Design on CDNA4:
//  * resolve_meta: one 4-wavefront workgroup per (request, layer).  The
//    slot owner, stamp and LRU-order arrays and the position->slot page
//    table (an open-addressing hash rebuilt from the owner array on every
//    call) live in LDS.  Misses are compacted with wavefront ballots in
//    ascending position order; victims are the first unpinned slots of a
//    persistent array that lists all slots in ascending (stamp, slot) order,
//    so victim choice is a ballot scan with no sort.  After the fills the
//    order array is rebuilt as [untouched slots with stamp < t, in old
//    order] ++ [slots with stamp == t, by slot index], which keeps it
//    sorted.  Only the owner and stamp entries that change are written back.
//  * fetch_rows: a fan-out copy over the whole GPU.  Each workgroup scans
//    the per-(request, layer) miss counts in LDS, then the grid walks a flat
//    index of 16-byte chunks over every missed row (72 chunks per 1152-byte
//    row), so a wavefront's loads cover 1 KiB of contiguous host memory.
//    Loads are zero-copy reads of the pinned, device-mapped pool over the
//    host link.
#include "internal.h"

#include <climits>

namespace hs {
namespace {

__device__ __forceinline__ uint32_t hash_pos(int32_t p, int bits) {
  return ((uint32_t)p * 0x9E3779B1u) >> (32 - bits);
}

__device__ __forceinline__ uint64_t lanemask_lt() {
  const int lane = threadIdx.x & 63;
  return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ void wait_vmem_and_sync() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

int ceil_log2(int64_t v) {
  int b = 0;
  while ((int64_t{1} << b) < v) ++b;
  return b;
}

constexpr int kMetaThreads = 256;  // 4 wavefronts per (request, layer)
constexpr int kMetaWaves = kMetaThreads / 64;

struct LdsMap {
  size_t owner, stamp, lru, sel, mpos, mj, vic, btv, flag, missf, region, total;
};

__host__ __device__ inline size_t round16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ inline LdsMap lds_map(int K, int B, int hash_bits, int seen_bits) {
  LdsMap m;
  m.owner = 0;
  m.stamp = m.owner + 4 * (size_t)B;
  m.lru = m.stamp + 4 * (size_t)B;
  m.sel = m.lru + 4 * (size_t)B;
  m.mpos = m.sel + 4 * (size_t)K;
  m.mj = m.mpos + 4 * (size_t)K;
  m.vic = m.mj + 4 * (size_t)K;
  m.btv = m.vic + 4 * (size_t)K;
  m.flag = round16(m.btv + 4 * (size_t)K);
  m.missf = m.flag + round16((size_t)B);
  m.region = m.missf + round16((size_t)K);
  const size_t hash_bytes = (size_t)4 << hash_bits;
  const size_t seen_bytes = (size_t)8 << seen_bits;  // also holds the miss sort (<= K entries)
  m.total = m.region + (hash_bytes > seen_bytes ? hash_bytes : seen_bytes);
  return m;
}

// Direct-to-LDS copy of n int32 by one workgroup: wave w issues chunks
// w, w+4, ... of 64 dwords; lanes past n are masked off.
__device__ __forceinline__ void g2l_block(int32_t* lds, const int32_t* g, int n, int wid, int lane) {
  for (int c = wid * 64; c < n; c += kMetaThreads)
    if (c + lane < n) __builtin_amdgcn_global_load_lds(g + c + lane, (lds_void*)(lds + c), 4, 0, 0);
}

// Exclusive prefix over the per-wave counts in cnt[0..kMetaWaves).
__device__ __forceinline__ int wave_base(const int* cnt, int wid, int* total) {
  int base = 0, tot = 0;
#pragma unroll
  for (int w2 = 0; w2 < kMetaWaves; ++w2) {
    const int c = cnt[w2];
    base += w2 < wid ? c : 0;
    tot += c;
  }
  *total = tot;
  return base;
}

// One workgroup (4 wavefronts) per (request, layer).  Element-wise passes
// are split over all 256 threads; the order-preserving compactions (the
// miss list in ascending position, the victims in (stamp, slot) order, the
// rebuilt order array) give each wave a contiguous quarter of the input,
// count with ballots, exchange the four counts through LDS and then write
// at base + ballot prefix.
__global__ __launch_bounds__(kMetaThreads) void resolve_meta(ResolveArgs a, int seen_bits) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int cnt_s[2][kMetaWaves];
  __shared__ int red_s[2][kMetaWaves];
  const int B = a.hot_slots, K = a.top_k, R = a.num_requests;
  const LdsMap M = lds_map(K, B, a.hash_bits, seen_bits);
  int32_t* owner_s = (int32_t*)(smem + M.owner);
  int32_t* stamp_s = (int32_t*)(smem + M.stamp);
  int32_t* lru_s = (int32_t*)(smem + M.lru);
  int32_t* sel_s = (int32_t*)(smem + M.sel);
  int32_t* mpos_s = (int32_t*)(smem + M.mpos);
  int32_t* mj_s = (int32_t*)(smem + M.mj);
  int32_t* vic_s = (int32_t*)(smem + M.vic);
  int32_t* btv_s = (int32_t*)(smem + M.btv);
  unsigned char* flag_s = smem + M.flag;
  unsigned char* missf_s = smem + M.missf;
  int32_t* hash_s = (int32_t*)(smem + M.region);
  unsigned long long* kv64_s = (unsigned long long*)(smem + M.region);

  const int tid = threadIdx.x;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const uint64_t lt = lanemask_lt();
  const int li = blockIdx.x / R;
  const int r = blockIdx.x - li * R;
  const int l = a.layer_begin + li;
  const size_t pair = (size_t)l * R + r;    // state index
  const size_t cpair = (size_t)li * R + r;  // output index of this call
  int32_t* rows_out = a.rows + cpair * K;
  const int32_t* topk = a.topk + (size_t)r * K;
  const int t = *a.step;
  const int ctx = a.ctx[r];
  const int64_t hot_base = a.resident_rows + (int64_t)r * B;
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;

  if (t < 0 || t < a.last_t[pair]) {
    for (int j = tid; j < K; j += kMetaThreads) rows_out[j] = -1;
    if (tid == 0) {
      a.counts[cpair * 3 + 0] = 0;
      a.counts[cpair * 3 + 1] = 0;
      a.counts[cpair * 3 + 2] = 0;
      a.miss_count[cpair] = 0;
      atomicOr(a.err, HISPARSE_ERR_STEP);
    }
    return;
  }

  int32_t* owner_g = a.owner + pair * B;
  int32_t* stamp_g = a.stamp + pair * B;
  int32_t* lru_g = a.lru + pair * B;
  // State and selection arrive together through direct-to-LDS loads.
  g2l_block(owner_s, owner_g, B, wid, lane);
  g2l_block(stamp_s, stamp_g, B, wid, lane);
  g2l_block(lru_s, lru_g, B, wid, lane);
  g2l_block(sel_s, topk, K, wid, lane);
  for (int i = tid; i < (int)(round16(B) / 4); i += kMetaThreads) ((uint32_t*)flag_s)[i] = 0u;
  wait_vmem_and_sync();

  // Selection: validate the range; note whether it is strictly ascending
  // with padding only at the end (then it has no repeats and its misses
  // come out already in ascending order).
  uint32_t errbits = 0;
  for (int j = tid; j < K; j += kMetaThreads) {
    const int p = sel_s[j];
    if (p < -1 || p >= ctx) {
      errbits |= HISPARSE_ERR_RANGE;
      sel_s[j] = -1;
    }
  }
  __syncthreads();
  bool bad = false;
  for (int j = tid; j + 1 < K; j += kMetaThreads) {
    const int a0 = sel_s[j], a1 = sel_s[j + 1];
    const int k0 = a0 < 0 ? INT_MAX : a0, k1 = a1 < 0 ? INT_MAX : a1;
    if (!(k0 < k1 || (k0 == INT_MAX && k1 == INT_MAX))) bad = true;
  }
  const bool fast = __syncthreads_or(bad) == 0;
  // Block-table entry of every selected page, gathered straight into LDS.
  const int32_t* bt = a.bt + a.bt_off[r];
  for (int c = wid * 64; c < K; c += kMetaThreads) {
    const int j = c + lane;
    if (j < K) {
      const int p = sel_s[j];
      __builtin_amdgcn_global_load_lds(bt + (p >= 0 ? (p >> page_shift) : 0), (lds_void*)(btv_s + c), 4, 0, 0);
    }
  }

  if (!fast) {
    // Repeated positions: keep the earliest entry (smallest j) of each.
    const int ES = 1 << seen_bits;
    for (int i = tid; i < ES; i += kMetaThreads) kv64_s[i] = ~0ull;
    __syncthreads();
    for (int j = tid; j < K; j += kMetaThreads) {
      const int p = sel_s[j];
      if (p < 0) continue;
      const unsigned long long ent = ((unsigned long long)(uint32_t)p << 32) | (uint32_t)j;
      uint32_t h = hash_pos(p, seen_bits);
      while (true) {
        const unsigned long long old = atomicCAS(&kv64_s[h], ~0ull, ent);
        if (old == ~0ull) break;
        if ((uint32_t)(old >> 32) == (uint32_t)p) {
          atomicMin(&kv64_s[h], ent);
          break;
        }
        h = (h + 1) & (ES - 1);
      }
    }
    __syncthreads();
    for (int j = tid; j < K; j += kMetaThreads) {
      const int p = sel_s[j];
      if (p < 0) continue;
      uint32_t h = hash_pos(p, seen_bits);
      while ((uint32_t)(kv64_s[h] >> 32) != (uint32_t)p) h = (h + 1) & (ES - 1);
      if ((uint32_t)kv64_s[h] != (uint32_t)j) {
        sel_s[j] = -1;
        errbits |= HISPARSE_ERR_DUP;
      }
    }
    __syncthreads();
  }

  // Page table: position -> slot, rebuilt from the owner array.
  const int HS = 1 << a.hash_bits;
  for (int i = tid; i < HS; i += kMetaThreads) hash_s[i] = -1;
  __syncthreads();
  for (int s0 = 0; s0 < B; s0 += 4 * kMetaThreads) {
    // four inserts per thread in flight at once
    int sl[4];
    uint32_t h[4];
    bool pend[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      sl[u] = s0 + kMetaThreads * u + tid;
      const int p = sl[u] < B ? owner_s[sl[u]] : -1;
      pend[u] = p >= 0;
      h[u] = pend[u] ? hash_pos(p, a.hash_bits) : 0u;
    }
    while (pend[0] || pend[1] || pend[2] || pend[3]) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        if (pend[u]) {
          if (atomicCAS(&hash_s[h[u]], -1, sl[u]) == -1) pend[u] = false;
          else h[u] = (h[u] + 1) & (HS - 1);
        }
      }
    }
  }
  wait_vmem_and_sync();  // also completes the block-table gather

  // Classify every entry: resident page, hot hit (stamp refresh + pin), miss.
  // Wave w takes entries [w Kq, (w+1) Kq), so wave order is input order.
  const int Kq = (K + kMetaThreads - 1) / kMetaThreads * 64;
  const int jb = wid * Kq, je = min(K, jb + Kq);
  int n_res = 0, n_hit = 0, mloc = 0;
  for (int j0 = jb; j0 < je; j0 += 64) {
    const int j = j0 + lane;
    bool miss = false;
    if (j < je) {
      const int p = sel_s[j];
      int row = -1;
      if (p >= 0) {
        const int blk = btv_s[j];
        if (blk >= 0) {
          row = (blk << page_shift) + (p & page_mask);
          ++n_res;
        } else {
          uint32_t h = hash_pos(p, a.hash_bits);
          int s;
          while ((s = hash_s[h]) >= 0 && owner_s[s] != p) h = (h + 1) & (HS - 1);
          if (s >= 0) {
            stamp_s[s] = t;
            stamp_g[s] = t;
            flag_s[s] = 1;
            row = (int)(hot_base + s);
            ++n_hit;
          } else {
            miss = true;
          }
        }
      }
      if (!miss) rows_out[j] = row;
      missf_s[j] = miss ? 1 : 0;
    }
    mloc += __popcll(__ballot(miss));
  }
  if (lane == 0) cnt_s[0][wid] = mloc;
  __syncthreads();
  int m;
  {
    int run = wave_base(cnt_s[0], wid, &m);
    for (int j0 = jb; j0 < je; j0 += 64) {
      const int j = j0 + lane;
      const bool miss = j < je && missf_s[j];
      const uint64_t bm = __ballot(miss);
      if (miss) {
        const int idx = run + __popcll(bm & lt);
        mpos_s[idx] = sel_s[j];
        mj_s[idx] = j;
      }
      run += __popcll(bm);
    }
  }
  __syncthreads();

  if (!fast && m > 1) {
    // Ascending position order of the misses: bitonic sort of (pos, j).
    int mp = 1;
    while (mp < m) mp <<= 1;
    for (int i = tid; i < mp; i += kMetaThreads)
      kv64_s[i] = i < m ? (((unsigned long long)(uint32_t)mpos_s[i] << 32) | (uint32_t)mj_s[i]) : ~0ull;
    __syncthreads();
    for (int k = 2; k <= mp; k <<= 1) {
      for (int jj = k >> 1; jj > 0; jj >>= 1) {
        for (int i = tid; i < mp; i += kMetaThreads) {
          const int ixj = i ^ jj;
          if (ixj > i) {
            const unsigned long long x = kv64_s[i], y = kv64_s[ixj];
            const bool up = (i & k) == 0;
            if ((x > y) == up) {
              kv64_s[i] = y;
              kv64_s[ixj] = x;
            }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < m; i += kMetaThreads) {
      mpos_s[i] = (int)(kv64_s[i] >> 32);
      mj_s[i] = (int)(uint32_t)kv64_s[i];
    }
    __syncthreads();
  }

  // Victims: the first m unpinned slots of the (stamp, slot) order array.
  // Wave w scans entries [w Bq, (w+1) Bq) of the array.
  const int Bq = (B + kMetaThreads - 1) / kMetaThreads * 64;
  const int ib = wid * Bq, ie = min(B, ib + Bq);
  {
    int uloc = 0;
    for (int i0 = ib; i0 < ie; i0 += 64) {
      const int i = i0 + lane;
      const bool cand = i < ie && flag_s[lru_s[i]] == 0;
      uloc += __popcll(__ballot(cand));
    }
    if (lane == 0) cnt_s[1][wid] = uloc;
  }
  __syncthreads();
  {
    int unpinned;
    int run = wave_base(cnt_s[1], wid, &unpinned);
    for (int i0 = ib; i0 < ie && run < m; i0 += 64) {
      const int i = i0 + lane;
      const int s = i < ie ? lru_s[i] : 0;
      const bool cand = i < ie && flag_s[s] == 0;
      const uint64_t bm = __ballot(cand);
      if (cand) {
        const int rank = run + __popcll(bm & lt);
        if (rank < m) vic_s[rank] = s;
      }
      run += __popcll(bm);
    }
  }
  __syncthreads();

  // Fill: i-th smallest missing position -> i-th victim.
  int2* fetch = a.fetch + cpair * K;
  for (int i = tid; i < m; i += kMetaThreads) {
    const int v = vic_s[i], p = mpos_s[i], j = mj_s[i];
    owner_s[v] = p;
    stamp_s[v] = t;
    flag_s[v] = 1;
    owner_g[v] = p;
    stamp_g[v] = t;
    rows_out[j] = (int)(hot_base + v);
    fetch[i] = make_int2(p, v);
  }
  __syncthreads();

  // New order: untouched slots older than t (old order), then every slot
  // stamped t, by slot index.  Both parts are counted in one pass.
  {
    int ca = 0, cb = 0;
    for (int i0 = ib; i0 < ie; i0 += 64) {
      const int i = i0 + lane;
      const bool keep = i < ie && stamp_s[lru_s[i]] < t;
      const bool inB = i < ie && stamp_s[i] == t;
      ca += __popcll(__ballot(keep));
      cb += __popcll(__ballot(inB));
    }
    if (lane == 0) {
      cnt_s[0][wid] = ca;
      cnt_s[1][wid] = cb;
    }
  }
  __syncthreads();
  {
    int nA, nB;
    int ra = wave_base(cnt_s[0], wid, &nA);
    int rb = nA + wave_base(cnt_s[1], wid, &nB);
    for (int i0 = ib; i0 < ie; i0 += 64) {
      const int i = i0 + lane;
      const int s = i < ie ? lru_s[i] : 0;
      const bool keep = i < ie && stamp_s[s] < t;
      const bool inB = i < ie && stamp_s[i] == t;
      const uint64_t ba = __ballot(keep), bb = __ballot(inB);
      if (keep) lru_g[ra + __popcll(ba & lt)] = s;
      if (inB) lru_g[rb + __popcll(bb & lt)] = i;
      ra += __popcll(ba);
      rb += __popcll(bb);
    }
  }

  n_res = wave_sum(n_res);
  n_hit = wave_sum(n_hit);
  if (errbits) atomicOr(a.err, errbits);
  if (lane == 0) {
    red_s[0][wid] = n_res;
    red_s[1][wid] = n_hit;
  }
  __syncthreads();
  if (tid == 0) {
    int tr = 0, th = 0;
#pragma unroll
    for (int w2 = 0; w2 < kMetaWaves; ++w2) {
      tr += red_s[0][w2];
      th += red_s[1][w2];
    }
    a.counts[cpair * 3 + 0] = tr;
    a.counts[cpair * 3 + 1] = th;
    a.counts[cpair * 3 + 2] = m;
    a.miss_count[cpair] = m;
    a.last_t[pair] = t;
  }
}

// 1024-thread workgroups (16 wavefronts) keep enough zero-copy loads in
// flight that a few dozen CUs saturate the host link.
constexpr int kFetchThreads = 1024;
constexpr int kFetchUnroll = 4;
constexpr int kCopyThreads = 256;
constexpr int kFetchMaxPairs = 8192;

__global__ __launch_bounds__(kFetchThreads) void fetch_rows(FetchArgs a, const int32_t* ctx) {
  extern __shared__ int32_t pre_s[];  // [n_pairs + 1] exclusive prefix of the miss counts
  __shared__ int32_t part_s[kFetchThreads];
  const int n = a.n_pairs, tid = threadIdx.x;
  const int per = (n + kFetchThreads - 1) / kFetchThreads;
  int sum = 0;
  for (int i = tid * per; i < n && i < (tid + 1) * per; ++i) sum += a.miss_count[i];
  part_s[tid] = sum;
  __syncthreads();
  // exclusive scan of part_s (Hillis-Steele, in place through a register)
  for (int off = 1; off < kFetchThreads; off <<= 1) {
    const int add = tid >= off ? part_s[tid - off] : 0;
    __syncthreads();
    part_s[tid] += add;
    __syncthreads();
  }
  const int excl = part_s[tid] - sum;
  __syncthreads();
  part_s[tid] = excl;
  __syncthreads();
  int acc = part_s[tid];
  for (int i = tid * per; i < n && i < (tid + 1) * per; ++i) {
    pre_s[i] = acc;
    acc += a.miss_count[i];
  }
  if (tid == kFetchThreads - 1) pre_s[n] = acc;
  __syncthreads();
  const int64_t total_chunks = (int64_t)pre_s[n] * kRowChunks;
  const int R = a.num_requests;

  for (int64_t base = (int64_t)blockIdx.x * kFetchThreads * kFetchUnroll; base < total_chunks;
       base += (int64_t)gridDim.x * kFetchThreads * kFetchUnroll) {
    u32x4 v[kFetchUnroll];
    u32x4* dst[kFetchUnroll];
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kFetchThreads + tid;
      dst[u] = nullptr;
      if (q < total_chunks) {
        const int gi = (int)(q / kRowChunks);
        const int c = (int)(q - (int64_t)gi * kRowChunks);
        int lo = 0, hi = n;  // largest pair with pre_s[pair] <= gi
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pre_s[mid] <= gi) lo = mid; else hi = mid;
        }
        const int pr = lo;
        const int i = gi - pre_s[pr];
        const int2 e = a.fetch[(size_t)pr * a.top_k + i];
        const int li = pr / R;
        const int r = pr - li * R;
        const int l = a.layer_begin + li;
        if ((unsigned)e.y < (unsigned)a.hot_slots && e.x >= 0 && e.x < ctx[r]) {
          const u32x4* src = reinterpret_cast<const u32x4*>(
              reinterpret_cast<const char*>(a.host_rows[(size_t)l * R + r]) + (size_t)e.x * kRowBytes) + c;
          const int64_t row = a.resident_rows + (int64_t)r * a.hot_slots + e.y;
          dst[u] = reinterpret_cast<u32x4*>(a.kv[l] + row * kLatent) + c;
          v[u] = __builtin_nontemporal_load(src);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u)
      if (dst[u]) *dst[u] = v[u];
  }
}

__global__ void iota_lru(int32_t* lru, int64_t n_pairs, int B) {
  const int64_t total = n_pairs * B;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x)
    lru[i] = (int32_t)(i % B);
}

__global__ __launch_bounds__(kCopyThreads) void copy16(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                      int64_t n) {
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads * kFetchUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kCopyThreads * kFetchUnroll; base < n; base += stride) {
    u32x4 v[kFetchUnroll];
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kCopyThreads + threadIdx.x;
      if (q < n) v[u] = __builtin_nontemporal_load(src + q);
    }
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kCopyThreads + threadIdx.x;
      if (q < n) dst[q] = v[u];
    }
  }
}

}  // namespace

size_t resolve_lds_bytes(int top_k, int hot_slots, int hash_bits) {
  return lds_map(top_k, hot_slots, hash_bits, ceil_log2(2 * (int64_t)top_k)).total;
}

hipError_t launch_state_reset(hisparse_pool* p, hipStream_t s) {
  const auto& c = p->cfg;
  const int64_t pairs = (int64_t)c.num_layers * c.num_requests;
  hipError_t e;
  if ((e = hipMemsetAsync(p->owner, 0xFF, pairs * c.hot_slots * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->stamp, 0xFF, pairs * c.hot_slots * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->last_t, 0xFF, pairs * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->miss_count, 0, pairs * 4, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(iota_lru, dim3(1024), dim3(256), 0, s, p->lru, pairs, c.hot_slots);
  return hipGetLastError();
}

hipError_t launch_workspace_init(hisparse_pool* p, hipStream_t s) {
  hipError_t e;
  if ((e = hipMemsetAsync(p->bt, 0xFF, p->lay.bt_entries * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->err, 0, 4, s)) != hipSuccess) return e;
  return launch_state_reset(p, s);
}

hipError_t launch_meta(hisparse_pool* p, const ResolveArgs& a, hipStream_t s) {
  const int seen_bits = ceil_log2(2 * (int64_t)a.top_k);
  const size_t lds = lds_map(a.top_k, a.hot_slots, a.hash_bits, seen_bits).total;
  prof_begin(p, kKMeta, s);
  hipLaunchKernelGGL(resolve_meta, dim3(a.n_layers * a.num_requests), dim3(kMetaThreads), lds, s, a, seen_bits);
  hipError_t e = hipGetLastError();
  prof_end(p, s);
  return e;
}

hipError_t launch_fetch(hisparse_pool* p, const FetchArgs& f, int grid, hipStream_t s) {
  if (f.n_pairs < 1 || f.n_pairs > kFetchMaxPairs || grid < 1) return hipErrorInvalidValue;
  prof_begin(p, kKFetch, s);
  hipLaunchKernelGGL(fetch_rows, dim3(grid), dim3(kFetchThreads), (f.n_pairs + 1) * sizeof(int32_t), s, f, p->ctx_d);
  hipError_t e = hipGetLastError();
  prof_end(p, s);
  return e;
}

hipError_t launch_stream_copy(void* dst, const void* src, size_t bytes, hipStream_t s) {
  const int64_t n = (int64_t)(bytes / 16);
  int64_t blocks = (n + kCopyThreads * kFetchUnroll - 1) / (kCopyThreads * kFetchUnroll);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(copy16, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, (u32x4*)dst, (const u32x4*)src, n);
  return hipGetLastError();
}

hipError_t set_resolve_lds_limit(size_t bytes) {
  return hipFuncSetAttribute((const void*)resolve_meta, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace hs
