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
//  * resolve_meta: one 16-wavefront workgroup per (request, layer).  The
//    position->slot page table is a persistent int16 map per (layer,
//    request) in device memory; the selection and the pin flags live in
//    LDS.  Misses are compacted with wavefront ballots in ascending position
//    order; victims are the first unpinned slots of a persistent array that
//    lists all slots in ascending (stamp, slot) order, so victim choice is a
//    ballot scan with no sort.  After the fills the order array is rebuilt
//    as [untouched slots with stamp < t, in old order] ++ [slots with stamp
//    == t, by slot index], which keeps it sorted.  Only the owner, stamp and
//    map entries that change are written.
//  * fetch_rows: a fan-out copy over the whole GPU.  Each workgroup scans
//    the per-(request, layer) miss counts in LDS, then the grid walks a flat
//    index of 16-byte chunks over every missed row (72 chunks per 1152-byte
//    bf16 row, 36 per 576-byte FP8 row), so a wavefront's loads cover 1 KiB
//    of contiguous host memory.
//    Loads are zero-copy reads of the pinned, device-mapped pool over the
//    host link.
#include "internal.h"

#include <climits>
#include <mutex>

namespace hs {
namespace {

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

[[maybe_unused]] int ceil_log2(int64_t v) {
  int b = 0;
  while ((int64_t{1} << b) < v) ++b;
  return b;
}

constexpr int kMetaThreads = 1024;  // 16 wavefronts per (request, layer)
constexpr int kMetaWaves = kMetaThreads / 64;
constexpr int kSelChunksMax = kMaxTopK / kMetaThreads;  // entries per thread of a one-token selection
constexpr int kRankSortMax = 128;  // misses ordered by a rank count up to this many, else by buckets
constexpr int kHashTokensMax = 8;  // several tokens: repeats found by a hash up to this many tokens, else a sort

// LDS of one metadata workgroup: the selection (W int32), the sort and
// miss-list region (W 64-bit keys, a power of two), the victims (W int32),
// one pin byte per slot, and an auxiliary region used at two different
// times: the hash table that finds repeated positions of a one-token
// selection in input order (2 W' int32 positions and 2 W' int32 earliest
// entries, W' = W rounded up to a power of two), and, for random
// replacement, B 64-bit keys (the misses stay in the key region while the
// victims are sorted).  Several tokens add the fill mask (W bits), which
// their cross-token copies extend before it is written out.
struct LdsMap {
  size_t sel, key, vic, tflag, aux, fm, total;
};

__host__ __device__ inline size_t round16(size_t v) { return (v + 15) & ~(size_t)15; }

__host__ __device__ inline int next_pow2(int v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

__host__ __device__ inline size_t hash_entries(int W) { return 2 * (size_t)next_pow2(W); }

__host__ __device__ inline LdsMap lds_map(int W, int B, bool random, bool one_token) {
  LdsMap m;
  m.sel = 0;
  m.key = round16(m.sel + 4 * (size_t)W);
  m.vic = m.key + 8 * (size_t)next_pow2(W);
  m.tflag = round16(m.vic + 4 * (size_t)W);
  m.aux = round16(m.tflag + (size_t)B);
  const size_t hash = one_token ? 8 * hash_entries(W) : 0;
  const size_t rkey = random ? 8 * (size_t)next_pow2(B) : 0;
  m.fm = round16(m.aux + (hash > rkey ? hash : rkey));
  m.total = m.fm + (one_token ? 0 : 8 * (size_t)((W + 63) / 64));
  return m;
}

// Direct-to-LDS copy of n int32 by one workgroup: wave w issues chunks
// w, w+16, ... of 64 dwords; lanes past n are masked off.
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

// Ascending bitonic sort of n (a power of two) 64-bit keys in LDS by the
// whole workgroup.
__device__ void bitonic_sort(unsigned long long* k, int n, int tid) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = tid; i < n; i += kMetaThreads) {
        const int ixj = i ^ stride;
        if (ixj > i) {
          const unsigned long long x = k[i], y = k[ixj];
          if ((x > y) == ((i & size) == 0)) {
            k[i] = y;
            k[ixj] = x;
          }
        }
      }
      __syncthreads();
    }
  }
}

// SplitMix64 (Steele, Lea, Flood, OOPSLA 2014): the generator's output for
// state x -- add the golden gamma, then the mixing function.
__device__ __forceinline__ uint64_t splitmix64(uint64_t x) {
  uint64_t z = x + 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

// One workgroup (16 wavefronts) per (request, layer).
//  * The position -> slot page table is a persistent int16 map over the
//    request's positions in device memory (exact: map[p] = s iff owner[s] =
//    p), so a lookup is one gather and a fill changes two entries.
//  * Pinning is a byte per slot in LDS (bit 0: hit or filled by this call;
//    bit 1: already stamped with this step by an earlier call of the same
//    step; bit 2: stamped by this call -- every fill, and hits except under
//    FIFO).  Stamps themselves are only written, except on that rare path.
//  * Replacement policy (the HiSparse summary article, section 04, compares
//    LRU with FIFO and random): LRU and FIFO take victims from the order
//    array (sorted by the stamp, which FIFO does not refresh on a hit);
//    random sorts (empty slots by index, then (31-bit SplitMix64 priority,
//    slot)) over the unpinned slots.
//  * Order-preserving compactions (misses in input order, victims in order
//    array order, the rebuilt order array) give each wave a contiguous range,
//    keep its ballots in registers, exchange the sixteen counts through LDS
//    and write at base + ballot prefix.  The order array is read once into
//    registers and rewritten at the end.
//  * The misses are kept as 64-bit keys (position << 32 | entry index), so
//    the unsorted path orders them in place (a rank count, or buckets of
//    positions).
// SC / BC: 64-entry chunks of the selection / of the order array per wave
// (the selection width W is at most 1024 SC, the slot count B at most 1024 BC).
template <int SC, int BC>
__global__ __launch_bounds__(kMetaThreads) void resolve_meta(ResolveArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ int cnt_s[2][kMetaWaves];
  __shared__ int red_s[2][kMetaWaves];
  __shared__ int scan_s[kMetaWaves];
  const int B = a.hot_slots, K = a.top_k, R = a.num_requests;
  const bool one_token = a.tok_k == K;
  const LdsMap M = lds_map(K, B, a.policy == HISPARSE_POLICY_RANDOM, one_token);
  int32_t* sel_s = (int32_t*)(smem + M.sel);
  unsigned long long* key_s = (unsigned long long*)(smem + M.key);  // sort region, then the miss list
  int32_t* vic_s = (int32_t*)(smem + M.vic);
  unsigned char* tflag_s = smem + M.tflag;
  unsigned long long* rkey_s = (unsigned long long*)(smem + M.aux);

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
  const int last = a.last_t[pair];
  const int ctx = a.ctx[r];
  const int64_t hot_base = a.resident_rows + (int64_t)r * B;
  const int page_shift = a.page_shift;
  const int page_mask = (1 << page_shift) - 1;

  if (t < 0 || t < last) {
    if (!a.prefetch)
      for (int j = tid; j < K; j += kMetaThreads) rows_out[j] = -1;
    if (a.fill_mask && !a.prefetch)
      for (int i = tid; i < (K + 63) / 64; i += kMetaThreads) a.fill_mask[cpair * ((K + 63) / 64) + i] = 0ull;
    if (tid == 0) {
      if (a.prefetch) {
        if (a.counts)
          for (int i = 0; i < 4; ++i) a.counts[cpair * 4 + i] = 0;
      } else {
        a.counts[cpair * 3 + 0] = 0;
        a.counts[cpair * 3 + 1] = 0;
        a.counts[cpair * 3 + 2] = 0;
      }
      a.miss_count[cpair] = 0;
      atomicOr(a.err, HISPARSE_ERR_STEP);
    }
    return;
  }
  const bool same_step = t == last;
  // A prefetch leaves every slot stamped t alone (the running step's
  // selection, and earlier fills of this step), as well as its own hits.
  const bool pf = a.prefetch != 0;
  const int pin_mask = pf ? 3 : 1;

  int32_t* owner_g = a.owner + pair * B;
  int32_t* stamp_g = a.stamp + pair * B;
  int32_t* lru_g = a.lru + pair * B;
  int16_t* map = a.posmap + (size_t)l * a.map_layer_stride + a.map_off[r];
  const int32_t* bt = a.bt + a.bt_off[r];  // read here, not at first use: one dependent round trip less

  // Wave ranges: selection entries [jb, je), order-array entries [ib, ie).
  const int Kq = (K + kMetaThreads - 1) / kMetaThreads * 64;
  const int jb = wid * Kq, je = min(K, jb + Kq);
  const int njc = Kq / 64;
  const int Bq = (B + kMetaThreads - 1) / kMetaThreads * 64;
  const int ib = wid * Bq, ie = min(B, ib + Bq);
  const int nsc = Bq / 64;

  g2l_block(sel_s, topk, K, wid, lane);
  int lv[BC];  // order-array entries of this wave
#pragma unroll
  for (int c = 0; c < BC; ++c) {
    const int i = ib + 64 * c + lane;
    lv[c] = (c < nsc && i < ie) ? lru_g[i] : 0;
  }
  for (int i = tid; i < (int)(round16(B) / 4); i += kMetaThreads) ((uint32_t*)tflag_s)[i] = 0u;
  wait_vmem_and_sync();
  if (same_step) {
    for (int s = tid; s < B; s += kMetaThreads)
      if (stamp_g[s] == t) tflag_s[s] = 2;
    __syncthreads();
  }

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
  const int KP = next_pow2(K);

  if (!fast && one_token) {
    // Repeated positions of a one-token selection: an LDS hash table keyed
    // by position (open addressing over twice the width, so every position
    // finds a slot) keeps the earliest entry of each position; every later
    // entry is an error and becomes padding.
    const int HN = (int)hash_entries(K);
    int* hpos = (int*)(smem + M.aux);
    int* hidx = hpos + HN;
    // cleared 16 bytes at a time (HN is a power of two, the region starts on 16 bytes)
    for (int i = tid; i < HN / 4; i += kMetaThreads) {
      ((int4*)hpos)[i] = make_int4(-1, -1, -1, -1);
      ((int4*)hidx)[i] = make_int4(INT_MAX, INT_MAX, INT_MAX, INT_MAX);
    }
    for (int i = HN / 4 * 4 + tid; i < HN; i += kMetaThreads) {
      hpos[i] = -1;
      hidx[i] = INT_MAX;
    }
    __syncthreads();
    int hs[kSelChunksMax];
#pragma unroll
    for (int c = 0; c < kSelChunksMax; ++c) {
      const int j = tid + c * kMetaThreads;
      hs[c] = -1;
      const int p = j < K ? sel_s[j] : -1;
      if (p >= 0) {
        int h = (int)(((uint32_t)p * 0x9E3779B1u) & (uint32_t)(HN - 1));
        for (int probe = 0; probe < HN; ++probe) {
          const int old = atomicCAS(&hpos[h], -1, p);
          if (old == -1 || old == p) break;
          h = (h + 1) & (HN - 1);
        }
        atomicMin(&hidx[h], j);
        hs[c] = h;
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < kSelChunksMax; ++c) {
      const int j = tid + c * kMetaThreads;
      if (hs[c] >= 0 && hidx[hs[c]] != j) {
        sel_s[j] = -1;
        errbits |= HISPARSE_ERR_DUP;
      }
    }
    __syncthreads();
  } else if (!fast && K / a.tok_k <= kHashTokensMax) {
    // Repeated positions of several tokens' selections: the earliest entry
    // of each position is the one resolved; a later entry of the same
    // token's list is an error (padding); an entry of a later token shares
    // the row of the earliest entry, which it names as sel = -2 - index
    // (padding to the classification below).  An LDS hash keyed by
    // position (linear probing over HN >= W slots in the key and victim
    // regions, unused until the classification) holds per position the
    // earliest entry overall (atomic minimum) and, one token after the
    // other, the earliest entry of the current token (atomic maximum of
    // (token << 16) | (65535 - entry), larger than every earlier token's).
    const int T = K / a.tok_k;
    const int HN = (int)((M.tflag - M.key) / 12);
    int* hpos = (int*)key_s;
    int* hfirst = hpos + HN;
    int* hcur = hfirst + HN;
    for (int i = tid; i < HN; i += kMetaThreads) {
      hpos[i] = -1;
      hfirst[i] = INT_MAX;
      hcur[i] = -1;
    }
    __syncthreads();
    for (int tk = 0; tk < T; ++tk) {
      int hs[kSelChunksMax];
#pragma unroll
      for (int c = 0; c < kSelChunksMax; ++c) {
        const int jt = tid + c * kMetaThreads;
        const int j = tk * a.tok_k + jt;
        hs[c] = -1;
        const int p = jt < a.tok_k ? sel_s[j] : -1;
        if (p >= 0) {
          int h = (int)(((uint64_t)((uint32_t)p * 0x9E3779B1u) * (uint32_t)HN) >> 32);
          int probe = 0;
          for (; probe < HN; ++probe) {  // HN >= W >= distinct positions: always ends on a break
            const int old = atomicCAS(&hpos[h], -1, p);
            if (old == -1 || old == p) break;
            if (++h == HN) h = 0;
          }
          if (probe < HN) {
            atomicMin(&hfirst[h], j);
            atomicMax(&hcur[h], (tk << 16) | (65535 - j));
            hs[c] = h;
          }
        }
      }
      __syncthreads();
#pragma unroll
      for (int c = 0; c < kSelChunksMax; ++c) {
        const int j = tk * a.tok_k + tid + c * kMetaThreads;
        if (hs[c] >= 0 && hcur[hs[c]] != ((tk << 16) | (65535 - j))) {
          sel_s[j] = -1;
          errbits |= HISPARSE_ERR_DUP;
          hs[c] = -1;
        }
      }
      __syncthreads();  // the token's checks read hcur before the next token raises it
#pragma unroll
      for (int c = 0; c < kSelChunksMax; ++c) {
        const int j = tk * a.tok_k + tid + c * kMetaThreads;
        if (hs[c] >= 0 && hfirst[hs[c]] != j) sel_s[j] = -2 - hfirst[hs[c]];
      }
    }
    __syncthreads();  // the key region is free again
  } else if (!fast) {
    // Repeated positions, many tokens: sort (position, index), with the
    // rules above.
    for (int i = tid; i < KP; i += kMetaThreads) {
      const int p = i < K ? sel_s[i] : -1;
      key_s[i] = p >= 0 ? (((unsigned long long)(uint32_t)p << 32) | (uint32_t)i) : ~0ull;
    }
    __syncthreads();
    bitonic_sort(key_s, KP, tid);
    for (int i = tid + 1; i < KP; i += kMetaThreads) {
      const unsigned long long x = key_s[i];
      if (x == ~0ull || (x >> 32) != (key_s[i - 1] >> 32)) continue;
      const int j = (int)(uint32_t)x, jp = (int)(uint32_t)key_s[i - 1];
      if (j / a.tok_k == jp / a.tok_k) {
        sel_s[j] = -1;
        errbits |= HISPARSE_ERR_DUP;
      } else {
        int f = i - 1;
        while (f > 0 && (key_s[f - 1] >> 32) == (x >> 32)) --f;
        sel_s[j] = -2 - (int)(uint32_t)key_s[f];
      }
    }
    __syncthreads();  // the key region is free again
  }

  // Classify every entry: resident page, hot hit (stamp refresh + pin), miss.
  // All gathers are consumed before the first store: a store issued between
  // two loads would make the wait for the later load wait for the store too.
  int pv[SC], bv[SC], sv[SC];
#pragma unroll
  for (int c = 0; c < SC; ++c) {
    const int j = jb + 64 * c + lane;
    const int p = (c < njc && j < je) ? sel_s[j] : -1;
    pv[c] = p;
    bv[c] = p >= 0 ? bt[p >> page_shift] : -1;
    sv[c] = p >= 0 ? (int)map[p] : -1;
  }
  int n_res = 0, n_hit = 0, mloc = 0;  // wave totals (uniform)
  uint64_t mb[SC], hb[SC];              // ballots: misses, hot hits
  int rowv[SC];                         // row id of a resident or hit entry, -1 for padding
#pragma unroll
  for (int c = 0; c < SC; ++c) {
    const int j = jb + 64 * c + lane;
    const int p = pv[c];
    const bool in = c < njc && j < je && p >= 0;
    const bool res = in && bv[c] >= 0;
    const bool hit = in && !res && sv[c] >= 0;
    const bool miss = in && !res && !hit;
    rowv[c] = res ? (bv[c] << page_shift) + (p & page_mask) : hit ? (int)(hot_base + sv[c]) : -1;
    mb[c] = __ballot(miss);
    hb[c] = __ballot(hit);
    mloc += __popcll(mb[c]);
    n_hit += __popcll(hb[c]);
    n_res += __popcll(__ballot(res));
  }
  // Pin and stamp the hits (LRU: refreshed to t; FIFO keeps the fill step
  // and a prefetch, a guess, refreshes nothing); write the rows of every
  // entry that is not a miss.  Before this call of the step no slot holds
  // a flag unless an earlier call of the same step stamped it.
  const unsigned char hit_flag = (pf || a.policy == HISPARSE_POLICY_FIFO) ? 1 : 5;
#pragma unroll
  for (int c = 0; c < SC; ++c) {
    const int j = jb + 64 * c + lane;
    if ((hb[c] >> lane) & 1) {
      const int s = sv[c];
      tflag_s[s] = same_step ? (unsigned char)(tflag_s[s] | hit_flag) : hit_flag;
      if (hit_flag == 5) stamp_g[s] = t;
    }
    if (c < njc && j < je && !((mb[c] >> lane) & 1) && !pf) rows_out[j] = rowv[c];
  }
  // The entries this call fills, one bit each (wave ranges start on 64);
  // with several tokens the mask goes through LDS first (see below).
  const bool fill_mask = a.fill_mask && !pf;
  uint64_t* fm_s = (uint64_t*)(smem + M.fm);
  if (fill_mask && lane == 0) {
    uint64_t* fm = one_token ? a.fill_mask + cpair * ((K + 63) / 64) : fm_s;
#pragma unroll
    for (int c = 0; c < SC; ++c)
      if (c < njc && jb + 64 * c < je) fm[(jb >> 6) + c] = mb[c];
  }
  if (lane == 0) {
    cnt_s[0][wid] = mloc;
    red_s[0][wid] = n_res;
    red_s[1][wid] = n_hit;
  }
  __syncthreads();
  int m;
  {
    int run = wave_base(cnt_s[0], wid, &m);
#pragma unroll
    for (int c = 0; c < SC; ++c) {
      if ((mb[c] >> lane) & 1) {
        const int idx = run + __popcll(mb[c] & lt);
        key_s[idx] = ((unsigned long long)(uint32_t)pv[c] << 32) | (uint32_t)(jb + 64 * c + lane);
      }
      run += __popcll(mb[c]);
    }
  }
  if (fill_mask && !one_token) {
    // An entry of a later token that repeats a filled position reads the
    // same row, which is being written in this step: it is marked as
    // filled too (the decode then reads it from the host pool as well).
    for (int j = tid; j < K; j += kMetaThreads) {
      const int p = sel_s[j];
      if (p <= -2) {
        const int e = -2 - p;
        if ((fm_s[e >> 6] >> (e & 63)) & 1ull) atomicOr((unsigned long long*)&fm_s[j >> 6], 1ull << (j & 63));
      }
    }
  }
  __syncthreads();
  if (fill_mask && !one_token)
    for (int i = tid; i < (K + 63) / 64; i += kMetaThreads) a.fill_mask[cpair * ((K + 63) / 64) + i] = fm_s[i];

  if (!fast && m > 1 && m <= kRankSortMax) {
    // Ascending position order of a few misses (their positions are
    // distinct: a repeat is padding or a copy by now): thread i counts the
    // misses at smaller positions than miss i (every thread reads the same
    // key at a time, an LDS broadcast), then writes it at that rank.
    const unsigned long long x = tid < m ? key_s[tid] : 0ull;
    const uint32_t xp = (uint32_t)(x >> 32);
    int rank = 0;
    if (tid < m)
      for (int i = 0; i < m; ++i) rank += (uint32_t)(key_s[i] >> 32) < xp ? 1 : 0;
    __syncthreads();
    if (tid < m) key_s[rank] = x;
    __syncthreads();
  } else if (!fast && m > 1) {
    // More misses: ascending position order by buckets of positions:
    // bucket b holds positions [b ctx / NB, (b + 1) ctx / NB).
    // Count the misses per bucket, take the exclusive prefix of the counts,
    // scatter the misses in bucket order, and place each miss by its rank
    // within its bucket (each thread counts the smaller positions there).
    const int NB = min(kMetaThreads, K / 2);
    int* bcnt = vic_s;  // the victims' region, unused until the victims are chosen
    int* bbase = vic_s + NB;
    for (int i = tid; i < NB; i += kMetaThreads) bcnt[i] = 0;
    __syncthreads();
    unsigned long long xk[SC];
    int bk[SC], lo[SC];
#pragma unroll
    for (int c = 0; c < SC; ++c) {
      const int i = tid + c * kMetaThreads;
      xk[c] = 0ull;
      bk[c] = 0;
      lo[c] = -1;
      if (i < m) {
        xk[c] = key_s[i];
        bk[c] = (int)(((uint64_t)(uint32_t)(xk[c] >> 32) * (uint32_t)NB) / (uint32_t)ctx);
        lo[c] = atomicAdd(&bcnt[bk[c]], 1);
      }
    }
    __syncthreads();
    const int v = tid < NB ? bcnt[tid] : 0;
    int incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int u = __shfl_up(incl, o, 64);
      if (lane >= o) incl += u;
    }
    if (lane == 63) scan_s[wid] = incl;
    __syncthreads();
    int wb = 0;
    for (int w2 = 0; w2 < wid; ++w2) wb += scan_s[w2];
    if (tid < NB) bbase[tid] = wb + incl - v;
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SC; ++c)
      if (lo[c] >= 0) key_s[bbase[bk[c]] + lo[c]] = xk[c];
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SC; ++c) {
      if (lo[c] >= 0) {
        const int s0 = bbase[bk[c]], n = bcnt[bk[c]];
        const uint32_t xp = (uint32_t)(xk[c] >> 32);
        int rk = 0;
        for (int q = 0; q < n; ++q) rk += (uint32_t)(key_s[s0 + q] >> 32) < xp ? 1 : 0;
        lo[c] = s0 + rk;  // from here on: the miss's place
      }
    }
    __syncthreads();
#pragma unroll
    for (int c = 0; c < SC; ++c)
      if (lo[c] >= 0) key_s[lo[c]] = xk[c];
    __syncthreads();
  }

  int unpinned = 0;  // slots a fill may take
  if (a.policy == HISPARSE_POLICY_RANDOM) {
    // Victims: empty slots by index, then ascending (priority, slot); the
    // priority of slot s is the top 31 bits of SplitMix64(k ^ s) with k
    // derived from (seed, t, layer, request).
    const uint64_t k = splitmix64(splitmix64(splitmix64(a.policy_seed) ^ (uint64_t)(uint32_t)t) ^
                                  (((uint64_t)(uint32_t)l << 32) | (uint32_t)r));
    const int BP = next_pow2(B);
    int uloc = 0;
    for (int i = tid; i < BP; i += kMetaThreads) {
      unsigned long long key = ~0ull;
      if (i < B && !(tflag_s[i] & pin_mask)) {
        ++uloc;
        key = owner_g[i] < 0 ? (unsigned long long)i
                             : ((1ull << 63) | ((splitmix64(k ^ (uint64_t)i) >> 33) << 32) | (uint32_t)i);
      }
      rkey_s[i] = key;
    }
    uloc = wave_sum(uloc);
    if (lane == 0) cnt_s[1][wid] = uloc;
    __syncthreads();
    wave_base(cnt_s[1], wid, &unpinned);
    bitonic_sort(rkey_s, BP, tid);
    for (int i = tid; i < m && i < unpinned; i += kMetaThreads) vic_s[i] = (int)(uint32_t)rkey_s[i];
  } else {
    // Victims: the first m unpinned slots of the (stamp, slot) order array.
    uint64_t vb[BC];
    int uloc = 0;
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const int i = ib + 64 * c + lane;
      const bool cand = c < nsc && i < ie && (tflag_s[lv[c]] & pin_mask) == 0;
      vb[c] = __ballot(cand);
      uloc += __popcll(vb[c]);
    }
    if (lane == 0) cnt_s[1][wid] = uloc;
    __syncthreads();
    int run = wave_base(cnt_s[1], wid, &unpinned);
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      if ((vb[c] >> lane) & 1) {
        const int rank = run + __popcll(vb[c] & lt);
        if (rank < m) vic_s[rank] = lv[c];
      }
      run += __popcll(vb[c]);
    }
  }
  __syncthreads();
  // A RESOLVE always has a victim per miss (B >= the selection width); a
  // prefetch fills what the free slots hold and drops the largest positions.
  const int m_all = m;
  m = min(m, unpinned);

  // Fill: i-th smallest missing position -> i-th victim.  The evicted
  // position cannot be in this selection (its slot would be pinned), so the
  // map entries cleared and set here are all distinct.
  // The victims' owners are all read before the first store (as in the
  // classification); m <= W <= SC * kMetaThreads.
  int2* fetch = a.fetch + cpair * K;
  int fv[SC], fold[SC];
#pragma unroll
  for (int c = 0; c < SC; ++c) {
    const int i = tid + c * kMetaThreads;
    fv[c] = i < m ? vic_s[i] : 0;
    fold[c] = i < m ? owner_g[fv[c]] : -1;
  }
#pragma unroll
  for (int c = 0; c < SC; ++c) {
    const int i = tid + c * kMetaThreads;
    if (i < m) {
      const unsigned long long x = key_s[i];
      const int v = fv[c], p = (int)(x >> 32), j = (int)(uint32_t)x;
      if (fold[c] >= 0) map[fold[c]] = -1;
      map[p] = (int16_t)v;
      owner_g[v] = p;
      stamp_g[v] = t;
      // a victim is unpinned: no flag but "stamped earlier this step"
      tflag_s[v] = same_step ? (unsigned char)(tflag_s[v] | 5) : 5;
      if (!pf) rows_out[j] = (int)(hot_base + v);
      fetch[i] = make_int2(p, v);
    }
  }
  __syncthreads();  // also makes every row id written above visible to the workgroup
  if (!fast && !pf) {
    // Entries that repeat a position of an earlier verify token take its row.
    for (int j = tid; j < K; j += kMetaThreads) {
      const int p = sel_s[j];
      if (p <= -2) rows_out[j] = rows_out[-2 - p];
    }
  }

  // New order: slots with stamp < t (untouched; old order), then every slot
  // stamped t, by slot index.
  {
    uint64_t ka[BC], kb[BC];
    int ca = 0, cb = 0;
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const int i = ib + 64 * c + lane;
      const bool in = c < nsc && i < ie;
      // stamp < t: neither stamped by this call nor earlier in this step
      ka[c] = __ballot(in && (tflag_s[lv[c]] & 6) == 0);
      kb[c] = __ballot(in && (tflag_s[i] & 6) != 0);
      ca += __popcll(ka[c]);
      cb += __popcll(kb[c]);
    }
    if (lane == 0) {
      cnt_s[0][wid] = ca;
      cnt_s[1][wid] = cb;
    }
    __syncthreads();
    int nA, nB;
    int ra = wave_base(cnt_s[0], wid, &nA);
    int rb = nA + wave_base(cnt_s[1], wid, &nB);
#pragma unroll
    for (int c = 0; c < BC; ++c) {
      const int i = ib + 64 * c + lane;
      if ((ka[c] >> lane) & 1) lru_g[ra + __popcll(ka[c] & lt)] = lv[c];
      if ((kb[c] >> lane) & 1) lru_g[rb + __popcll(kb[c] & lt)] = i;
      ra += __popcll(ka[c]);
      rb += __popcll(kb[c]);
    }
  }

  if (errbits) atomicOr(a.err, errbits);
  if (tid == 0) {  // red_s was written before the classification barrier
    int tr = 0, th = 0;
#pragma unroll
    for (int w2 = 0; w2 < kMetaWaves; ++w2) {
      tr += red_s[0][w2];
      th += red_s[1][w2];
    }
    if (pf) {
      if (a.counts) {
        a.counts[cpair * 4 + 0] = tr;
        a.counts[cpair * 4 + 1] = th;
        a.counts[cpair * 4 + 2] = m;
        a.counts[cpair * 4 + 3] = m_all - m;
      }
    } else {
      a.counts[cpair * 3 + 0] = tr;
      a.counts[cpair * 3 + 1] = th;
      a.counts[cpair * 3 + 2] = m;
    }
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
  const int rc = a.row_chunks;
  const int64_t total_chunks = (int64_t)pre_s[n] * rc;
  const int R = a.num_requests, RT = a.total_requests;

  for (int64_t base = (int64_t)blockIdx.x * kFetchThreads * kFetchUnroll; base < total_chunks;
       base += (int64_t)gridDim.x * kFetchThreads * kFetchUnroll) {
    u32x4 v[kFetchUnroll];
    u32x4* dst[kFetchUnroll];
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kFetchThreads + tid;
      dst[u] = nullptr;
      if (q < total_chunks) {
        const int gi = (int)(q / rc);
        const int c = (int)(q - (int64_t)gi * rc);
        int lo = 0, hi = n;  // largest pair with pre_s[pair] <= gi
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (pre_s[mid] <= gi) lo = mid; else hi = mid;
        }
        const int pr = lo;
        const int i = gi - pre_s[pr];
        const int2 e = a.fetch[(size_t)pr * a.top_k + i];
        const int li = pr / R;
        const int r = a.request_begin + (pr - li * R);
        const int l = a.layer_begin + li;
        const bool held = e.x < a.hv[(size_t)l * RT + r];  // the host pool holds this position
        if (!held && c == 0) atomicOr(a.err, HISPARSE_ERR_UNMATERIALIZED);
        if ((unsigned)e.y < (unsigned)a.hot_slots && e.x >= 0 && e.x < ctx[r] && held) {
          const u32x4* src = reinterpret_cast<const u32x4*>(
              reinterpret_cast<const char*>(a.host_rows[(size_t)l * RT + r]) + (size_t)e.x * rc * 16) + c;
          const int64_t row = a.resident_rows + (int64_t)r * a.hot_slots + e.y;
          dst[u] = reinterpret_cast<u32x4*>(a.kv[l] + row * rc * 16) + c;
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

// Rows of `rc` 16-byte chunks gathered by a list of row indices: the miss
// fetch's access pattern (one flat index over all chunks, nontemporal
// 16-byte loads, several in flight per thread) without its metadata.
__global__ __launch_bounds__(kCopyThreads) void gather16(u32x4* __restrict__ dst, const u32x4* __restrict__ src,
                                                        const int64_t* __restrict__ rows, int64_t n_chunks, int rc) {
  const int64_t stride = (int64_t)gridDim.x * kCopyThreads * kFetchUnroll;
  for (int64_t base = (int64_t)blockIdx.x * kCopyThreads * kFetchUnroll; base < n_chunks; base += stride) {
    u32x4 v[kFetchUnroll];
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kCopyThreads + threadIdx.x;
      if (q < n_chunks) {
        const int64_t i = q / rc;
        v[u] = __builtin_nontemporal_load(src + rows[i] * rc + (q - i * rc));
      }
    }
#pragma unroll
    for (int u = 0; u < kFetchUnroll; ++u) {
      const int64_t q = base + (int64_t)u * kCopyThreads + threadIdx.x;
      if (q < n_chunks) dst[q] = v[u];
    }
  }
}

}  // namespace

size_t resolve_lds_bytes(int width, int hot_slots, bool random, bool one_token) {
  return lds_map(width, hot_slots, random, one_token).total;
}

hipError_t launch_state_reset(hisparse_pool* p, hipStream_t s) {
  const auto& c = p->cfg;
  const int64_t pairs = (int64_t)c.num_layers * c.num_requests;
  hipError_t e;
  if ((e = hipMemsetAsync(p->owner, 0xFF, pairs * c.hot_slots * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->stamp, 0xFF, pairs * c.hot_slots * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->last_t, 0xFF, pairs * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->miss_count, 0, pairs * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->posmap, 0xFF, p->lay.posmap_entries * 2, s)) != hipSuccess) return e;
  if ((e = hipMemcpyAsync(p->ctx_d, p->init_ctx32.data(), c.num_requests * 4, hipMemcpyHostToDevice, s)) !=
      hipSuccess)
    return e;
  if ((e = hipMemcpyAsync(p->hv_d, p->init_hv32.data(), pairs * 4, hipMemcpyHostToDevice, s)) != hipSuccess) return e;
  hipLaunchKernelGGL(iota_lru, dim3(1024), dim3(256), 0, s, p->lru, pairs, c.hot_slots);
  return hipGetLastError();
}

hipError_t launch_workspace_init(hisparse_pool* p, hipStream_t s) {
  hipError_t e;
  if ((e = hipMemsetAsync(p->bt, 0xFF, p->lay.bt_entries * 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->err, 0, 4, s)) != hipSuccess) return e;
  if ((e = hipMemsetAsync(p->fallback_count, 0, 4, s)) != hipSuccess) return e;
  return launch_state_reset(p, s);
}

// Chunk counts of the metadata kernel: the common sizes (W <= 4096, B <=
// 8192) keep the per-wave register arrays of the first instance; larger
// selections (multi-token verification) and buffers take the second.
constexpr int kSelChunksSmall = 4, kSlotChunksSmall = 8;
constexpr int kSelChunksLarge = kMaxSelection / kMetaThreads;
constexpr int kSlotChunksLarge = kMaxHotSlots / kMetaThreads;
static_assert(kSelChunksLarge * kMetaThreads == kMaxSelection && kSlotChunksLarge * kMetaThreads == kMaxHotSlots,
              "whole chunks per wave");

hipError_t launch_meta(hisparse_pool* p, const ResolveArgs& a, hipStream_t s) {
  const size_t lds = lds_map(a.top_k, a.hot_slots, a.policy == HISPARSE_POLICY_RANDOM, a.tok_k == a.top_k).total;
  const dim3 grid(a.n_layers * a.num_requests), block(kMetaThreads);
  const bool small_sel = a.top_k <= kSelChunksSmall * kMetaThreads;
  const bool small_slots = a.hot_slots <= kSlotChunksSmall * kMetaThreads;
  prof_begin(p, kKMeta, s);
  if (small_sel && small_slots)
    hipLaunchKernelGGL((resolve_meta<kSelChunksSmall, kSlotChunksSmall>), grid, block, lds, s, a);
  else
    hipLaunchKernelGGL((resolve_meta<kSelChunksLarge, kSlotChunksLarge>), grid, block, lds, s, a);
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

hipError_t launch_row_gather(void* dst, const void* src, const int64_t* rows, int64_t n_rows, int row_bytes,
                             hipStream_t s) {
  const int rc = row_bytes / 16;
  const int64_t n = n_rows * rc;
  int64_t blocks = (n + kCopyThreads * kFetchUnroll - 1) / (kCopyThreads * kFetchUnroll);
  if (blocks > 2048) blocks = 2048;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(gather16, dim3((unsigned)blocks), dim3(kCopyThreads), 0, s, (u32x4*)dst, (const u32x4*)src,
                     rows, n, rc);
  return hipGetLastError();
}

// The dynamic-LDS limit is an attribute of the kernel, shared by every pool
// of the process, so it only ever grows (per device): a pool with a smaller
// selection must not lower the limit another pool's launches rely on.
hipError_t set_resolve_lds_limit(int device, size_t bytes) {
  static std::mutex mu;
  static size_t cur[64] = {};
  if (device < 0 || device >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (bytes <= cur[device]) return hipSuccess;
  hipError_t e = hipFuncSetAttribute((const void*)resolve_meta<kSelChunksSmall, kSlotChunksSmall>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e != hipSuccess) return e;
  e = hipFuncSetAttribute((const void*)resolve_meta<kSelChunksLarge, kSlotChunksLarge>,
                          hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) cur[device] = bytes;
  return e;
}

}  // namespace hs
