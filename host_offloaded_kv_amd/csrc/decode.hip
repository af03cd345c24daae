// Sparse MLA decode attention over resolved KV rows (gfx950).
//
// For every (layer, request) the K resolved row ids name 576-wide bf16
// latent rows of the layer's KV tensor (resident pages and hot rows share
// one row-id space, as in the vLLM Hybrid HiSparse blog, Fig. 1 text: hot
// pages and KV pages live in one KV-cache tensor, so the sparse MLA kernel
// sees ordinary pages).  Per head h:
//     s_j = scale * q_h . x_j          (576 dims)
//     O_h = sum_j softmax(s)_j x_j[0:512],  lse_h = logsumexp_j s_j
// The HiSparse summary article (section 02) fixes that these outputs are the
// same as attention over the full KV with the same selection.
//
// Work split: a workgroup handles (layer, request, group of up to 64 heads,
// K split) with 12 wavefronts, three per SIMD, specialised by role:
//  * score waves 0-3: wave w keeps the Q of heads 16w .. 16w+15 in
//    registers and scores all 32 rows of each tile on 16x16x32 bf16 MFMA;
//    it applies the softmax with a reference max per head and writes the
//    probabilities P to LDS;
//  * value waves 4-7: wave 4+c owns output columns 128c .. 128c+127 for
//    every head of the group (fp32 accumulators in registers); it multiplies
//    the transposed tile (read with ds_read_b64_tr_b16) by P;
//  * loader waves 8-11: gather the row tiles through registers, three tiles
//    ahead, and write them to LDS as bf16 (FP8 rows widened exactly).
// The value waves run one tile behind the score waves and the loaders one
// tile ahead, so each tile costs a single workgroup barrier, and no compute
// wave waits on a global load or an LDS store.  Split partials are merged by
// a second kernel.
//
// Precision.  The scores multiply the bf16 rows and queries as given (the
// products are exact, accumulation fp32).  For PV the value waves convert
// the row operands from bf16 to fp16, which is exact for magnitudes in
// [2^-14, 2^16); smaller ones become fp16 subnormals (absolute error below
// 2^-25).  P is one fp16 plane: 11 significant bits, a relative rounding
// error of at most 2^-11 per weight, while O and lse are normalised by the
// sum of the unrounded fp32 weights.  (A single bf16 plane, 8 bits, gave O
// errors above 2e-3 of max|O| for near-uniform weights.)  A V value of
// magnitude 2^16 or more becomes inf in fp16 and makes O inf or NaN (also
// where its weight is zero), and an inf or NaN input makes a score
// non-finite; either way the workgroup computes its result again in plain
// fp32 arithmetic on the values as given (exact_fallback), a slow path for
// inputs that KV caches do not hold.  FP8 rows always fit fp16.
#include "internal.h"

#include <algorithm>
#include <cmath>
#include <mutex>
#include <type_traits>

namespace hs {
namespace {

constexpr int kT = 32;                        // rows per tile
// LDS row pitch: 72 data + 2 pad chunks (1184 bytes).  With this pitch the
// score waves' 16-row b128 reads run at the contiguous-read rate on gfx950;
// a 1168-byte pitch costs them 1.5x and 1152 bytes 3x (measured).
constexpr int kPitchChunks = kRowChunks + 2;
constexpr int kPitch = kPitchChunks * 16;
constexpr int kTileBytes = kT * kPitch;       // 37888
constexpr int kNBuf = 3;                      // tiles in LDS: scored, multiplied, being stored
constexpr int kThreads = 768;                 // 12 wavefronts: 4 score, 4 value, 4 loader
constexpr int kPPitch = kT + 8;               // fp16 per P row (80 bytes)
constexpr float kMaxGrowLog2 = 15.f;          // P = 2^(s - m) <= 2^15 stays finite in fp16
constexpr int kMaxPasses = 2;
constexpr int kStage = kRowChunks / 8;        // 9 chunks per loading thread per tile
static_assert(kT * 8 == 256 && kRowChunks % 8 == 0, "8 loader threads per row, 256 loaders per tile");

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;
typedef const __attribute__((address_space(1))) u32x4 gu32x4;
typedef const __attribute__((address_space(1))) u32x2 gu32x2;
typedef const __attribute__((address_space(1))) uint32_t gu32;
typedef const __attribute__((address_space(1))) uint16_t gu16;

// Two fp32 values -> their fp16 pair, rounded to nearest even (overflow
// gives +-inf).
__device__ __forceinline__ uint32_t pack_f16(float lo, float hi) {
  const f16x2 v = {(_Float16)lo, (_Float16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Two fp32 values that bf16 holds exactly -> their bf16 pair.
__device__ __forceinline__ uint32_t pack_bf16_exact(float lo, float hi) {
  return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

// A bf16 pair -> the fp16 pair of the same values.
__device__ __forceinline__ uint32_t bf16x2_to_f16x2(uint32_t b) {
  return pack_f16(__uint_as_float(b << 16), __uint_as_float(b & 0xFFFF0000u));
}

__device__ __forceinline__ int load_row_id(const DecodeArgs& a, const int32_t* rows, int k, int k1) {
  if (k >= k1) return -1;
  const int r = rows[k];
  if (r < -1 || r >= a.kv_rows) {
    atomicOr(a.err, HISPARSE_ERR_ROW);
    return -1;
  }
  return r;
}

// Tile loads go through VGPRs: each loader thread fetches its part of a
// tile with ordinary global loads three tiles ahead and writes it to LDS
// one tile ahead of the score waves.  On MI355X this sustains ~7.3 TB/s for a
// random 1152-byte row gather, where direct-to-LDS loads stayed under
// 3 TB/s.  The loads use global-address-space pointers: flat loads would
// also count against the LDS wait counter and be drained by every
// lds_barrier().  Loader thread t (0..255) owns row t / 8 of the tile and
// its 8-value groups t % 8 + 8 k, k = 0..8 (LDS chunk t % 8 + 8 k of the
// row): eight threads cover contiguous bytes of a row per k, and every
// address is one base plus an immediate.
//
// The LDS tile is bf16.  FP8 E4M3 rows are widened while staging: every
// E4M3 value (at most 4 significant bits, magnitude at most 448, smallest
// 2^-9) converts to fp32 and then to bf16 exactly; the layer's scale is
// applied to the scores and to O instead.
template <bool FP8>
struct TileStage;

// A hot-row write of a fetched row goes through a buffer resource over
// the request's hot rows; threads with nothing to write pass an offset
// beyond its end, which the hardware drops.  The store is issued on every
// path, so the loads in flight stay the same on all of them.
constexpr int kNoHotWrite = 0x7FFF0000;

template <>
struct TileStage<false> {
  u32x4 v[kStage];
  // row: first byte of the row (a KV tensor row or a host pool row)
  __device__ __forceinline__ void load_row(const unsigned char* row, int t) {
    gu32x4* src = (gu32x4*)(row + (t & 7) * 16);
#pragma unroll
    for (int k = 0; k < kStage; ++k) v[k] = src[8 * k];
  }
  __device__ __forceinline__ void store_hot(__amdgpu_buffer_rsrc_t hot, int off, int t) const {
#pragma unroll
    for (int k = 0; k < kStage; ++k)
      __builtin_amdgcn_raw_buffer_store_b128(v[k], hot, off + ((t & 7) + 8 * k) * 16, 0, 0);
  }
  __device__ __forceinline__ void store(unsigned char* xs, int t) const {
    u32x4* dst = reinterpret_cast<u32x4*>(xs + (t >> 3) * kPitch + (t & 7) * 16);
#pragma unroll
    for (int k = 0; k < kStage; ++k) dst[8 * k] = v[k];
  }
};

template <>
struct TileStage<true> {
  u32x2 v[kStage];
  __device__ __forceinline__ void load_row(const unsigned char* row, int t) {
    gu32x2* src = (gu32x2*)(row + (t & 7) * 8);
#pragma unroll
    for (int k = 0; k < kStage; ++k) v[k] = src[8 * k];
  }
  __device__ __forceinline__ void store_hot(__amdgpu_buffer_rsrc_t hot, int off, int t) const {
#pragma unroll
    for (int k = 0; k < kStage; ++k)
      __builtin_amdgcn_raw_buffer_store_b64(v[k], hot, off + ((t & 7) + 8 * k) * 8, 0, 0);
  }
  __device__ __forceinline__ void store(unsigned char* xs, int t) const {
    u32x4* dst = reinterpret_cast<u32x4*>(xs + (t >> 3) * kPitch + (t & 7) * 16);
#pragma unroll
    for (int k = 0; k < kStage; ++k) {
      const f32x2 a0 = __builtin_amdgcn_cvt_pk_f32_fp8(v[k][0], false);
      const f32x2 a1 = __builtin_amdgcn_cvt_pk_f32_fp8(v[k][0], true);
      const f32x2 b0 = __builtin_amdgcn_cvt_pk_f32_fp8(v[k][1], false);
      const f32x2 b1 = __builtin_amdgcn_cvt_pk_f32_fp8(v[k][1], true);
      const u32x4 w = {pack_bf16_exact(a0[0], a0[1]), pack_bf16_exact(a1[0], a1[1]), pack_bf16_exact(b0[0], b0[1]),
                       pack_bf16_exact(b1[0], b1[1])};
      dst[8 * k] = w;
    }
  }
};

// Workgroup barrier for LDS traffic only: unlike __syncthreads() it does
// not wait for outstanding global loads, so tile loads stay in flight.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// All MFMAs are written as inline asm with every operand in VGPRs (the
// kernel uses no AGPRs, so every role may use all of a wave's 168 VGPRs at
// three waves per SIMD); with the builtin the register allocator moves
// accumulators between register files around the MFMAs.  The compiler does
// not see these as MFMAs, so the hazards they can meet are covered by hand:
//  * an operand written by a VALU instruction just before: two wait states
//    in front of the first MFMA that reads a freshly assembled operand;
//  * reading results afterwards: score_drain() and acc_drain() insert wait
//    states after the last MFMA;
//  * accumulators must never be copied or touched by other instructions
//    inside the loops (checked in the generated code), since such an
//    access could meet an MFMA still writing them.
// Back-to-back MFMAs that chain through srcC need no wait states.
__device__ __forceinline__ void mfma_acc(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_acc_after_valu(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void zero_acc(f32x4& d) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_f16 %0, %1, %1, 0" : "=&v"(d) : "v"(z));
}
// Score MFMAs: A (tile rows) and B (Q) in VGPRs; the first k-step starts
// from srcC = 0.
__device__ __forceinline__ void mfma_score_first(f32x4& d, const u32x4& a, const f32x4& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_score(f32x4& d, const u32x4& a, const f32x4& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
// The drains name the registers they protect as read-write operands of the
// wait-state asm itself, so the MFMAs writing them stay above it and no
// later read of them can be scheduled above it.
template <int N>
__device__ __forceinline__ void score_drain(f32x4 (&s)[N]) {
  static_assert(N == 1 || N == 2, "one or two score accumulators");
  if constexpr (N == 1)
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0])::"memory");
  else
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" : "+v"(s[0]), "+v"(s[1])::"memory");
}
// acc_drain() follows the loop that issues the accumulating MFMAs, which
// keeps them above it.
template <int N>
__device__ __forceinline__ void acc_drain(f32x4 (&acc)[N]) {
  asm volatile(
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\t"
      "s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; i += 2) asm volatile("" : "+v"(acc[i]), "+v"(acc[i + 1]));
}

template <int HG>
struct DecodeSmem {
  unsigned char xs[kNBuf][kTileBytes];  // row tiles: scored, multiplied, being stored
  uint16_t ps[2][HG][kPPitch];          // P by tile parity: [head][row], fp16
  int rowid[kMaxTopK];                  // row ids of the workgroup's K range
  int rowpos[kMaxTopK];                 // fetch in the decode: host pool position of row k (-1: the KV tensor)
  float lexact[HG], mfin[HG];           // weight sum and reference max per head
  int overflow[kMaxPasses];             // a tile exceeded the reference max
  int nonfinite;                        // a score was inf or NaN: exact_fallback takes over
  int vbad;                             // an O accumulator is inf or NaN (read after the last barrier)
  int cnt[kThreads / 64];               // per-wave counts of the row-id compaction
  // merging an earlier launch's partials: factors per head (see merge_prepare)
  float mown[HG], minv[HG], mlse[HG], mf[HG][kMaxMergeSlots];
};

// Passes over the K range: the first uses the reference max of the first
// tile with a valid row; if a later tile exceeds it by more than 2^15 (the
// range of an fp16 weight), the range is recomputed once with the true
// maximum of every head, which no tile can exceed.  Read by every role after
// the same barrier, so all take the same branch.
template <int HG>
__device__ __forceinline__ bool again(const DecodeSmem<HG>& sm, int p) {
  return p + 1 < kMaxPasses && sm.overflow[p] && !sm.nonfinite;
}

// One pass of a score wave over the tiles (see score_role).
template <int HG>
__device__ __forceinline__ void score_tiles(DecodeSmem<HG>& sm, const f32x4 (&q)[kLatent / 32], float score_scale,
                                            int n_tiles, int p, int w, int g, int i16, float& m_run, float& m_seen,
                                            float& l_exact) {
  const bool active = 16 * w < HG;
  constexpr int GS = 3;                 // k-steps per operand group
  constexpr int NG = kLatent / 32 / GS;  // 6 groups
  for (int it = 0; it <= n_tiles; ++it) {
    if (active && it < n_tiles) {
      const unsigned char* xb = sm.xs[it % kNBuf];
      f32x4 sacc[2];
      // A operands: lane (g, i16) reads rows i16 and 16 + i16, dims 32 s + 8 g .. +7;
      // the group after the one being multiplied is already loading.
      const unsigned char* xrow = xb + i16 * kPitch + 16 * g;
      u32x4 A[2][GS][2];
#pragma unroll
      for (int s = 0; s < GS; ++s) {
        A[0][s][0] = *reinterpret_cast<const u32x4*>(xrow + 64 * s);
        A[0][s][1] = *reinterpret_cast<const u32x4*>(xrow + 16 * kPitch + 64 * s);
      }
#pragma unroll
      for (int gi = 0; gi < NG; ++gi) {
        if (gi + 1 < NG) {
#pragma unroll
          for (int s = 0; s < GS; ++s) {
            const int ks = GS * (gi + 1) + s;
            A[(gi + 1) & 1][s][0] = *reinterpret_cast<const u32x4*>(xrow + 64 * ks);
            A[(gi + 1) & 1][s][1] = *reinterpret_cast<const u32x4*>(xrow + 16 * kPitch + 64 * ks);
          }
        }
#pragma unroll
        for (int s = 0; s < GS; ++s) {
          const int ks = GS * gi + s;
          if (ks == 0) {
            mfma_score_first(sacc[0], A[gi & 1][s][0], q[0]);
            mfma_score_first(sacc[1], A[gi & 1][s][1], q[0]);
          } else {
            mfma_score(sacc[0], A[gi & 1][s][0], q[ks]);
            mfma_score(sacc[1], A[gi & 1][s][1], q[ks]);
          }
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      score_drain(sacc);
      // lane (g, i16): head 16 w + i16, rows 16 rb + 4 g + v
      bool valid[2][4];
      bool finite = true;
      float mx = -INFINITY;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        const int4 rid = *reinterpret_cast<const int4*>(sm.rowid + it * kT + 16 * rb + 4 * g);
        valid[rb][0] = rid.x >= 0;
        valid[rb][1] = rid.y >= 0;
        valid[rb][2] = rid.z >= 0;
        valid[rb][3] = rid.w >= 0;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          // Every staged row counts, the filler rows of padding entries too:
          // their zero weights must not meet an inf in the PV product.
          finite = finite && __builtin_fabsf(sacc[rb][v]) <= 3.0e38f;
          sacc[rb][v] = valid[rb][v] ? sacc[rb][v] * score_scale : -INFINITY;
          mx = fmaxf(mx, sacc[rb][v]);
        }
      }
      if (!finite) sm.nonfinite = 1;  // the fast-path result is discarded
      m_seen = fmaxf(m_seen, mx);  // this lane's rows only; reduced when needed
      if (__builtin_amdgcn_readfirstlane(m_run == -INFINITY ? 1 : 0)) {
        // first tile with a valid row (the same tile for every head)
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        m_run = mx;
      } else if (mx > m_run + kMaxGrowLog2) {
        sm.overflow[p] = 1;  // this pass is discarded
      }
      const int head = 16 * w + i16;
#pragma unroll
      for (int rb = 0; rb < 2; ++rb) {
        float pr[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) pr[v] = valid[rb][v] ? __builtin_amdgcn_exp2f(sacc[rb][v] - m_run) : 0.f;
        l_exact += (pr[0] + pr[1]) + (pr[2] + pr[3]);
        const u32x2 pw = {pack_f16(pr[0], pr[1]), pack_f16(pr[2], pr[3])};
        *reinterpret_cast<u32x2*>(&sm.ps[it & 1][head][16 * rb + 4 * g]) = pw;
      }
    }
    lds_barrier();
  }
}

// Score waves 0-3: wave w scores all 32 rows of each tile against heads
// 16w .. 16w+15 (waves past the group's heads idle through the barriers).
// The A operand (16 rows x 32 dims) comes from LDS, the B operand (Q) from
// registers, and the two 16-row blocks of a tile give two accumulators, so
// each wave sees every row of its heads and needs no exchange with another.
//
// Softmax with a fixed reference max per head: the first tile with a valid
// row sets m, and P = 2^(s*scale*log2e - m) accumulates unnormalised, so
// the O accumulators are never rescaled inside the loop.  Both passes give
// the exact softmax.
template <int HG>
__device__ __forceinline__ void merge_prepare(const DecodeArgs& a, DecodeSmem<HG>& sm, float kvs, int pair, int hg,
                                              int h, float mo, float lo);

template <int HG, bool FP8>
__device__ __forceinline__ void score_role(const DecodeArgs& a, DecodeSmem<HG>& sm, float kvs, size_t head0,
                                           int pair, int hg, int n_tiles, int w, int g, int i16) {
  const bool active = 16 * w < HG;
  // Q as MFMA B operands: lane (g, i16) holds dims 32 s + 8 g .. +7 of
  // head 16 w + i16, in bf16.
  f32x4 q[kLatent / 32];
  if (active) {
    gu32x4* qp = (gu32x4*)(a.q + (head0 + 16 * w + i16) * kLatent + 8 * g);
#pragma unroll
    for (int s = 0; s < kLatent / 32; ++s) {
      q[s] = __builtin_bit_cast(f32x4, qp[4 * s]);
    }
#pragma unroll
    for (int s = 0; s < kLatent / 32; s += 2) asm volatile("" : "+v"(q[s]), "+v"(q[s + 1]));
  }
  // Scores in log2 units; FP8 rows carry the layer's scale.
  const float score_scale = a.scale_log2 * kvs;
  // m_run: reference max of this lane's head; m_seen: the largest score
  // seen; l_exact: sum of the unrounded weights.
  float m_run = -INFINITY, m_seen = -INFINITY, l_exact = 0.f;
  for (int p = 0; p < kMaxPasses; ++p) {
    l_exact = 0.f;
    lds_barrier();  // tile 0 is in LDS
    score_tiles<HG>(sm, q, score_scale, n_tiles, p, w, g, i16, m_run, m_seen, l_exact);
    if (!again(sm, p)) break;
    // recompute with the true maximum of the head over all its lanes' rows
    m_seen = fmaxf(m_seen, __shfl_xor(m_seen, 16, 64));
    m_seen = fmaxf(m_seen, __shfl_xor(m_seen, 32, 64));
    m_run = m_seen;
    lds_barrier();
  }

  // Reference max and weight sum per head for the value waves.
  if (active) {
    float le = l_exact;
    le += __shfl_xor(le, 16, 64);
    le += __shfl_xor(le, 32, 64);
    if (g == 0) {
      sm.lexact[16 * w + i16] = le;
      sm.mfin[16 * w + i16] = m_run;
      if (a.merge_from > 0) merge_prepare<HG>(a, sm, kvs, pair, hg, 16 * w + i16, m_run, le);
    }
  }
  __syncthreads();
}

// Where the output of head h of the group goes, from column c0 on: the O
// row (scaled by kvs / l) or a split partial for combine_splits (scaled by
// kvs, with m and l beside it).  The writer also stores lse or (m, l).
struct OutSlot {
  float scale;  // 0 when the head has no valid row
  float* dst;
};
template <int HG>
__device__ __forceinline__ OutSlot out_slot(const DecodeArgs& a, const DecodeSmem<HG>& sm, float kvs, size_t head0,
                                            int pair, int split, int hg, int h, int c0, bool writer) {
  // O and lse are normalised by the sum of the unrounded weights.
  const float lsum = sm.lexact[h];
  const float m = sm.mfin[h];
  if (!a.out_partial) {
    if (writer)
      a.lse[head0 + h] = lsum > 0.f ? (m + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    return {lsum > 0.f ? kvs / lsum : 0.f, a.out + (head0 + h) * kVDim + c0};
  }
  float* part =
      a.partial + (((size_t)pair * a.split_total + a.split_base + split) * a.num_heads + hg * HG + h) * kPartW;
  if (writer) {
    part[kVDim] = m;
    part[kVDim + 1] = lsum;
    part[kVDim + 2] = lsum;
  }
  return {kvs, part + c0};
}

// The output of head h of the group when the launch merges the partials of
// an earlier launch over the other entries of the same query sets (slots
// 0 .. merge_from-1): O = (sum_s f_s O_s + f O_own) / L and lse = m +
// log2(L) (in log2 units, then ln), where m is the largest reference max
// among the parts with weight and each part's sums are rescaled to it.
// Called by one thread per head with this workgroup's reference max and
// weight sum of the head; the factors go to LDS.
template <int HG>
__device__ __forceinline__ void merge_prepare(const DecodeArgs& a, DecodeSmem<HG>& sm, float kvs, int pair, int hg,
                                              int h, float mo, float lo) {
  const size_t stride = (size_t)a.num_heads * kPartW;
  const float* part = a.partial + ((size_t)pair * a.merge_from * a.num_heads + hg * HG + h) * kPartW;
  float m = lo > 0.f ? mo : -INFINITY;
#pragma unroll
  for (int q = 0; q < kMaxMergeSlots; ++q)
    if (q < a.merge_from && part[q * stride + kVDim + 1] > 0.f) m = fmaxf(m, part[q * stride + kVDim]);
  float own = 0.f, inv = 0.f, lse = -INFINITY, L = 0.f, LE = 0.f;
  if (m != -INFINITY) {
    const float fo = lo > 0.f ? exp2f(mo - m) : 0.f;
    L = lo * fo;
    LE = lo * fo;
    own = kvs * fo;
  }
#pragma unroll
  for (int q = 0; q < kMaxMergeSlots; ++q) {
    float f = 0.f;
    if (q < a.merge_from && m != -INFINITY) {
      const float ls = part[q * stride + kVDim + 1];
      if (ls > 0.f) {
        f = exp2f(part[q * stride + kVDim] - m);
        L += ls * f;
        LE += part[q * stride + kVDim + 2] * f;
      }
    }
    sm.mf[h][q] = f;
  }
  if (m != -INFINITY) {
    inv = 1.f / L;
    lse = (m + log2f(LE)) * 0.69314718055994531f;
  }
  sm.mown[h] = own;
  sm.minv[h] = inv;
  sm.mlse[h] = lse;
}

// Partial row of slot q of head h for the merge.
__device__ __forceinline__ const float* merge_part(const DecodeArgs& a, int pair, int head_in_layer, int q) {
  return a.partial + (((size_t)pair * a.merge_from + q) * a.num_heads + head_in_layer) * kPartW;
}

// One pass of a value wave over the tiles (see value_role).  The P
// operands of all head blocks are in registers, so the tile's columns are
// read once per tile.
template <int HG>
__device__ __forceinline__ void value_tiles(DecodeSmem<HG>& sm, f32x4 (&acc)[HG / 2], int n_tiles, int cw, int g,
                                            int i16) {
  constexpr int NBP = HG / 16;  // 16-head blocks
  for (int it = 0; it <= n_tiles; ++it) {
    if (it >= 1) {
      const int tp = it - 1;
      const unsigned char* xb = sm.xs[tp % kNBuf];
      // B operands: P of rows 8 g .. 8 g + 7, head 16 nb + i16.
      u32x4 bp[NBP];
#pragma unroll
      for (int nb = 0; nb < NBP; ++nb) bp[nb] = *reinterpret_cast<const u32x4*>(&sm.ps[tp & 1][16 * nb + i16][8 * g]);
      // A operand (X^T, 16 cols x 32 rows) by two transposed reads: lane
      // (g, i16) addresses row 8 g + i16 / 4 (+4), columns 128 cw + 16 mb +
      // 4 (i16 % 4) .. +3, and receives column 128 cw + 16 mb + i16 of rows
      // 8 g .. 8 g + 7 (bf16, converted to fp16 for the MFMA).
      uint32_t xoff = (8 * g + (i16 >> 2)) * kPitch + (128 * cw + 4 * (i16 & 3)) * 2;
      asm volatile("" : "+v"(xoff));
      const lds_u8* xl = (const lds_u8*)xb + xoff;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
        const s16x4 lo =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(xl + 32 * mb));
        const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(xl + 32 * mb + 4 * kPitch));
        const u32x4 raw = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        const u32x4 av = {bf16x2_to_f16x2(raw[0]), bf16x2_to_f16x2(raw[1]), bf16x2_to_f16x2(raw[2]),
                          bf16x2_to_f16x2(raw[3])};
        mfma_acc_after_valu(acc[mb * NBP], av, bp[0]);
#pragma unroll
        for (int nb = 1; nb < NBP; ++nb) mfma_acc(acc[mb * NBP + nb], av, bp[nb]);
        if (mb & 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
    lds_barrier();
  }
}

// Value waves 4-7: wave 4+cw owns output columns 128cw .. 128cw+127 of every
// head of the group, O^T[128 cols x HG heads] += X^T[cols x 32 rows] P^T.
// Writes nothing when the fast-path result is discarded.
template <int HG, bool FP8>
__device__ __forceinline__ void value_role(const DecodeArgs& a, DecodeSmem<HG>& sm, float kvs, size_t head0,
                                           int pair, int split, int hg, int n_tiles, int cw, int g, int i16) {
  constexpr int NBP = HG / 16;  // 16-head blocks
  // acc[mb * NBP + nb]: columns 128 cw + 16 mb + 4 g + v, head 16 nb + i16
  f32x4 acc[8 * NBP];
  for (int p = 0; p < kMaxPasses; ++p) {
#pragma unroll
    for (int mb = 0; mb < 8; ++mb)
#pragma unroll
      for (int nb = 0; nb < NBP; ++nb) zero_acc(acc[mb * NBP + nb]);
    lds_barrier();
    value_tiles<HG>(sm, acc, n_tiles, cw, g, i16);
    if (!again(sm, p)) break;
    lds_barrier();
  }
  acc_drain(acc);
  // A V value beyond fp16 became inf in the operand and shows up in O.
  bool bad = false;
#pragma unroll
  for (int i = 0; i < 8 * NBP; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) bad = bad || !(__builtin_fabsf(acc[i][v]) <= 3.0e38f);
  if (bad) sm.vbad = 1;
  __syncthreads();  // the score waves' normalisers are in LDS
  if (sm.nonfinite || sm.vbad) return;

  if (a.merge_from > 0) {
    // per head block: this workgroup's sums rescaled in place, then each
    // earlier slot's 8 column groups loaded four at a time and added
#pragma unroll
    for (int nb = 0; nb < NBP; ++nb) {
      const int h = nb * 16 + i16;
      if (cw == 0 && g == 0) a.lse[head0 + h] = sm.mlse[h];
      const float own = sm.mown[h], inv = sm.minv[h];
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) acc[mb * NBP + nb] *= own;
#pragma unroll
      for (int q = 0; q < kMaxMergeSlots; ++q) {
        if (q >= a.merge_from) break;
        const float* src = merge_part(a, pair, hg * HG + h, q) + 128 * cw + 4 * g;
        const float f = sm.mf[h][q];
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          f32x4 pa[4];
#pragma unroll
          for (int i = 0; i < 4; ++i) pa[i] = *reinterpret_cast<const f32x4*>(src + 16 * (4 * half + i));
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[(4 * half + i) * NBP + nb] += pa[i] * f;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      float* dst = a.out + (head0 + h) * kVDim + 128 * cw + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(dst + 16 * mb) = acc[mb * NBP + nb] * inv;
      __builtin_amdgcn_sched_barrier(0);  // one head block's loads in flight at a time
    }
    return;
  }

#pragma unroll
  for (int nb = 0; nb < NBP; ++nb) {
    const OutSlot o =
        out_slot(a, sm, kvs, head0, pair, split, hg, nb * 16 + i16, 128 * cw + 4 * g, cw == 0 && g == 0);
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      *reinterpret_cast<f32x4*>(o.dst + 16 * mb) = acc[mb * NBP + nb] * o.scale;
      __builtin_amdgcn_sched_barrier(0);  // few accumulators in VGPRs at a time
    }
  }
}

// Loader waves 8-11: tile n is held in register set n % kLoadSets from
// kLoadSets iterations before it is needed.  Iteration it writes tile it+1
// to its LDS slot (last read in iteration it-2) and starts the load of tile
// it+1+kLoadSets into the registers just freed, so three tiles' loads are in
// flight while the compute waves work on tiles it and it-1 (two sets left
// the gather waiting on HBM latency: 119 us instead of 102 us for one
// launch over 4 layers of 32 requests; four sets gained nothing more).
// For the wait before a store to name exactly that set's loads, the set
// index must be a constant and every path must issue the same loads: the
// loop runs three iterations per trip, and tiles past the range load row 0.
constexpr int kLoadSets = 3;

// Where the loader reads the rows of a workgroup's tiles: the layer's KV
// tensor, or, for rows this step fills when the decode fetches them, the
// request's host pool rows; each such row is also written to its hot row,
// by one of the head groups that read it (row i of the key range by head
// group hg when i mod nhg == hg).  Where most rows are filled, sharing the
// writes keeps the head groups of a key range at the same pace, so the
// later one still finds the host rows in their XCD's L2: with all the
// writes in head group 0 it fell behind, and a step of nothing but misses
// moved every row over the link twice.  Where few are, head group 0 writes
// them all (sharing measured up to 1% slower per step there, and 1-4% with
// several verify tokens).
struct RowSource {
  const unsigned char* kv;
  const unsigned char* host;       // the request's host pool rows (fetch in the decode)
  __amdgpu_buffer_rsrc_t hot;      // the request's hot rows
  int64_t hot_base;                // row id of the request's first hot row
  int hg, nhg;                     // this workgroup's head group, and the request's head groups
};

template <int HG, bool FP8, bool FETCH>
__device__ __forceinline__ void loader_role(DecodeSmem<HG>& sm, const RowSource& rs, int n_tiles, int lt) {
  static_assert(kLoadSets == 3, "the loop below is unrolled for three register sets");
  constexpr int RB = FP8 ? kRowBytesFp8 : kRowBytes;
  TileStage<FP8> st[kLoadSets];
  int hoff[kLoadSets];  // hot-row write offset of each set's row (kNoHotWrite: none)
  const int row = lt >> 3;
  const int n_ids = n_tiles * kT;
  // Source of this thread's row of tile n; tiles past the range stage row 0
  // (their loads are issued anyway, so that every path has the same loads
  // in flight and the wait before a store names exactly its set's loads).
  struct Ref {
    const unsigned char* src;
    int hoff;
  };
  auto ref_of = [&](int n) {
    const int i = n * kT + row;
    const bool in = i < n_ids;
    const int r = sm.rowid[in ? i : 0];
    const int rid = in ? r : -1;
    Ref x;
    x.src = rs.kv + (size_t)(rid < 0 ? 0 : rid) * RB;
    x.hoff = kNoHotWrite;
    if constexpr (FETCH) {
      const int pr = sm.rowpos[in ? i : 0];
      const int pos = in ? pr : -1;
      x.src = pos >= 0 ? rs.host + (size_t)pos * RB : x.src;
      x.hoff = pos >= 0 && i % rs.nhg == rs.hg ? (int)((rid - rs.hot_base) * RB) : kNoHotWrite;
    }
    return x;
  };
  int it = 0;
  Ref nxt;
  // Iteration it stores tile it + 1 (from set (it + 1) % 3) and loads tile
  // it + 4 into the same set; stores past the range land in a buffer
  // nobody reads.
  auto step = [&](auto u) {
    constexpr int U = decltype(u)::value;
    constexpr int S = (U + 1) % kLoadSets;
    const int nx = it + U + 1;
    st[S].store(sm.xs[nx % kNBuf], lt);
    if constexpr (FETCH) st[S].store_hot(rs.hot, hoff[S], lt);
    st[S].load_row(nxt.src, lt);
    hoff[S] = nxt.hoff;
    nxt = ref_of(nx + kLoadSets + 1);
    lds_barrier();
  };
  for (int p = 0; p < kMaxPasses; ++p) {
#pragma unroll
    for (int j = 0; j < kLoadSets; ++j) {
      const Ref x = ref_of(j);
      st[j].load_row(x.src, lt);
      hoff[j] = x.hoff;
    }
    nxt = ref_of(kLoadSets);
    st[0].store(sm.xs[0], lt);
    if constexpr (FETCH) st[0].store_hot(rs.hot, hoff[0], lt);
    st[0].load_row(nxt.src, lt);
    hoff[0] = nxt.hoff;
    nxt = ref_of(kLoadSets + 1);
    lds_barrier();
    // iterations 0 .. n_tiles, three per trip so that each step's register
    // set is a constant, then the remaining one or two
    for (it = 0; it + kLoadSets <= n_tiles + 1; it += kLoadSets) {
      step(std::integral_constant<int, 0>{});
      step(std::integral_constant<int, 1>{});
      step(std::integral_constant<int, 2>{});
    }
    if (it <= n_tiles) step(std::integral_constant<int, 0>{});
    if (it + 1 <= n_tiles) step(std::integral_constant<int, 1>{});
    if (!again(sm, p)) break;
    lds_barrier();
  }
  __syncthreads();
}

// The result of a workgroup whose fast path met a value beyond fp16 or a
// non-finite input, in plain fp32 arithmetic on the values as given: a
// first sweep over the rows finds each head's maximum score, a second forms
// the weights and O.
// Rows are staged 16 at a time as fp32 in the tile buffers (with Q as
// bf16); thread t < 8 HG owns O of head t / 8, columns 64 (t % 8) .. +63.
constexpr int kFbRows = 16;
constexpr int kFbPitch = kLatent + 4;  // floats per staged row

template <int HG, bool FP8, bool FETCH>
__device__ __forceinline__ void exact_fallback(const DecodeArgs& a, DecodeSmem<HG>& sm, const RowSource& rs,
                                               float kvs, size_t head0, int pair, int split, int hg, int n_rows,
                                               int tid) {
  static_assert(HG * kLatent * 2 + kFbRows * kFbPitch * 4 <= kNBuf * kTileBytes, "fallback staging fits the tiles");
  static_assert(HG * kFbRows * 4 <= sizeof(DecodeSmem<HG>::ps), "fallback scores fit the P buffers");
  uint32_t* qs = reinterpret_cast<uint32_t*>(&sm.xs[0][0]);              // [HG][288] bf16 pairs
  float* xf = reinterpret_cast<float*>(&sm.xs[0][0] + HG * kLatent * 2);  // [16][kFbPitch]
  float* sp = reinterpret_cast<float*>(&sm.ps[0][0][0]);                   // [HG][16]
  const float score_scale = a.scale_log2 * kvs;
  __syncthreads();  // every role is done with the tile buffers
  const uint32_t* qg = reinterpret_cast<const uint32_t*>(a.q + head0 * kLatent);
  for (int i = tid; i < HG * kLatent / 2; i += kThreads) qs[i] = qg[i];
  const int oh = tid >> 3, oc = (tid & 7) * 64;
  const bool owner = tid < 8 * HG;
  float acc[64];
#pragma unroll
  for (int c = 0; c < 64; ++c) acc[c] = 0.f;
  float m = -INFINITY, l = 0.f;  // of head tid, in threads tid < HG
  for (int pass = 0; pass < 2; ++pass) {
    for (int c0 = 0; c0 < n_rows; c0 += kFbRows) {
      __syncthreads();  // the previous chunk is consumed
      for (int i = tid; i < kFbRows * kLatent / 2; i += kThreads) {
        const int j = i / (kLatent / 2), d2 = i % (kLatent / 2);
        const int rid = c0 + j < n_rows ? sm.rowid[c0 + j] : -1;
        float x0 = 0.f, x1 = 0.f;
        if (rid >= 0) {
          // a row this step fills is read where the fast path read it
          const int pos = FETCH ? sm.rowpos[c0 + j] : -1;
          const unsigned char* row = pos >= 0 ? rs.host + (size_t)pos * (FP8 ? kRowBytesFp8 : kRowBytes)
                                              : rs.kv + (size_t)rid * (FP8 ? kRowBytesFp8 : kRowBytes);
          if constexpr (FP8) {
            const uint32_t w = *(gu16*)(row + 2 * d2);
            const f32x2 v = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
            x0 = v[0];
            x1 = v[1];
          } else {
            const uint32_t w = *(gu32*)(row + 4 * d2);
            x0 = __uint_as_float(w << 16);
            x1 = __uint_as_float(w & 0xFFFF0000u);
          }
        }
        xf[j * kFbPitch + 2 * d2] = x0;
        xf[j * kFbPitch + 2 * d2 + 1] = x1;
      }
      __syncthreads();
      for (int pr = tid; pr < HG * kFbRows; pr += kThreads) {
        const int h = pr / kFbRows, j = pr % kFbRows;
        const bool valid = c0 + j < n_rows && sm.rowid[c0 + j] >= 0;
        const uint32_t* qh = qs + h * (kLatent / 2);
        const float* xj = xf + j * kFbPitch;
        float dot = 0.f;
        for (int d2 = 0; d2 < kLatent / 2; ++d2) {
          const uint32_t w = qh[d2];
          dot = fmaf(__uint_as_float(w << 16), xj[2 * d2], dot);
          dot = fmaf(__uint_as_float(w & 0xFFFF0000u), xj[2 * d2 + 1], dot);
        }
        sp[h * kFbRows + j] = valid ? dot * score_scale : -INFINITY;
      }
      __syncthreads();
      if (tid < HG) {
        for (int j = 0; j < kFbRows; ++j) {
          const float s = sp[tid * kFbRows + j];
          if (pass == 0) {
            m = fmaxf(m, s);
          } else {
            const float pw = s == -INFINITY ? 0.f : exp2f(s - m);
            sp[tid * kFbRows + j] = pw;
            l += pw;
          }
        }
      }
      if (pass == 1) {
        __syncthreads();
        if (owner) {
          for (int j = 0; j < kFbRows; ++j) {
            const float pw = sp[oh * kFbRows + j];
            const float* xj = xf + j * kFbPitch + oc;
#pragma unroll
            for (int c = 0; c < 64; ++c) acc[c] = fmaf(pw, xj[c], acc[c]);
          }
        }
      }
    }
  }
  if (tid < HG) {
    sm.lexact[tid] = l;
    sm.mfin[tid] = m;
    if (a.merge_from > 0) merge_prepare<HG>(a, sm, kvs, pair, hg, tid, m, l);
  }
  __syncthreads();
  if (!owner) return;
  if (a.merge_from > 0) {
    if ((tid & 7) == 0) a.lse[head0 + oh] = sm.mlse[oh];
    const float own = sm.mown[oh], inv = sm.minv[oh];
    float* dst = a.out + (head0 + oh) * kVDim + oc;
#pragma unroll
    for (int c = 0; c < 64; ++c) acc[c] *= own;
#pragma unroll
    for (int q = 0; q < kMaxMergeSlots; ++q) {
      if (q >= a.merge_from) break;
      const float* pq = merge_part(a, pair, hg * HG + oh, q) + oc;
      const float fq = sm.mf[oh][q];
#pragma unroll
      for (int c = 0; c < 64; ++c) acc[c] += pq[c] * fq;
    }
#pragma unroll
    for (int c = 0; c < 64; ++c) dst[c] = acc[c] * inv;
    return;
  }
  const OutSlot o = out_slot(a, sm, kvs, head0, pair, split, hg, oh, oc, (tid & 7) == 0);
#pragma unroll
  for (int c = 0; c < 64; ++c) o.dst[c] = acc[c] * o.scale;
}

// Every role passes the same barriers: per pass one before the loop and one
// per iteration (n_tiles + 1), one between passes, and the final
// __syncthreads().
// FETCH: the decode reads the rows this step fills from the host pool (and
// writes them to their hot rows): the miss fetch and the decode in one pass
// over the rows.
template <int HG, bool FP8, bool FETCH>
__global__ __launch_bounds__(kThreads, 1) void decode_ws(DecodeArgs a, int nhg) {
  __shared__ __align__(16) DecodeSmem<HG> sm;
  const int H = a.num_heads, R = a.num_requests, K = a.top_k;
  // XCD-aware order: consecutive logical blocks share blockIdx % 8, i.e.
  // one XCD and its L2, and the head groups of one key range are
  // consecutive: they read the same rows (from HBM, or from the host pool
  // when the decode fetches), which the second one finds in that L2.
  int li = blockIdx.x;
  if (gridDim.x % 8 == 0) li = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int hg = li % nhg;
  li /= nhg;
  const int split = li % a.splits;
  const int pair = li / a.splits;
  const int l = a.layer_begin + pair / R;
  const unsigned char* kv = a.kv[l];
  const float kvs = FP8 ? a.kv_scale[l] : 1.f;  // x = decode(code) * kvs for FP8 rows
  const int32_t* rows = a.rows + (size_t)pair * K;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, g = lane >> 4, i16 = lane & 15;

  int per = (K + a.splits - 1) / a.splits;
  per = (per + kT - 1) / kT * kT;
  const int k0 = split * per;
  const int k1 = min(K, k0 + per);

  // Row ids of the K range, validated once.  A part launch keeps only the
  // entries of its part, in order (ballot compaction over the range).
  if (tid < kMaxPasses) sm.overflow[tid] = 0;
  if (tid == 0) {
    sm.nonfinite = 0;
    sm.vbad = 0;
  }
  constexpr int RB = FP8 ? kRowBytesFp8 : kRowBytes;
  RowSource rs;
  rs.kv = kv;
  rs.host = nullptr;
  rs.hot_base = 0;
  int held = 0;
  int q = 0;             // query set within its layer: token q % tokens of request q / tokens
  size_t mask_bit0 = 0;  // fill-mask bit of this query set's entry 0
  if constexpr (FETCH) {
    q = pair % R;
    const int r = q / a.tokens;
    mask_bit0 = ((size_t)(pair / R) * (R / a.tokens) + r) * a.mask_words * 64 + (size_t)(q - r * a.tokens) * K;
    held = a.hv[(size_t)l * a.total_requests + r];
    rs.host = reinterpret_cast<const unsigned char*>(a.host_rows[(size_t)l * a.total_requests + r]);
    rs.hot_base = a.resident_rows + (int64_t)r * a.hot_slots;
    rs.hot = __builtin_amdgcn_make_buffer_rsrc(const_cast<unsigned char*>(kv) + rs.hot_base * RB, 0,
                                               a.hot_slots * RB, 0x00020000);
  } else {
    rs.hot = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0x00020000);
  }
  int n_rows = k1 > k0 ? k1 - k0 : 0;
  if (a.part == 0) {
    const int n_pad = (n_rows + kT - 1) / kT * kT;
    int nf = 0;  // filled rows this wave saw
    for (int k = tid; k < n_pad; k += kThreads) {
      if constexpr (FETCH) {
        // The row id, its fill-mask word and its position are independent
        // loads: issued together and unconditionally (entries past the range
        // read entry k0 and are dropped), so that none waits for another.
        const int kk = k0 + k;
        const bool in = kk < k1;
        const int kc = in ? kk : k0;
        const size_t bit = mask_bit0 + kc;
        const int r_in = rows[kc];
        const uint64_t word = a.fill_mask[bit >> 6];
        const int p_in = a.sel[(size_t)q * K + kc];
        const bool rbad = in & ((r_in < -1) | (r_in >= a.kv_rows));
        const int rid = (in & !rbad) ? r_in : -1;
        const bool filled = (rid >= 0) & (((word >> (bit & 63)) & 1ull) != 0);
        const bool pbad = filled & ((p_in < 0) | (p_in >= held));
        sm.rowid[k] = rid;
        sm.rowpos[k] = (filled & !pbad) ? p_in : -1;
        nf += __popcll(__ballot(filled & !pbad));
        if (rbad) atomicOr(a.err, HISPARSE_ERR_ROW);
        if (pbad) atomicOr(a.err, HISPARSE_ERR_UNMATERIALIZED);
      } else {
        sm.rowid[k] = load_row_id(a, rows, k0 + k, k1);
      }
    }
    if (FETCH && lane == 0) sm.cnt[w] = nf;
  } else {
    const uint64_t* mask = a.fill_mask + (size_t)pair * a.mask_words;
    const bool want_filled = a.part == 2;
    int base = 0;
    for (int c0 = k0; c0 < k1; c0 += kThreads) {
      const int k = c0 + tid;
      const bool in = k < k1 && (((mask[k >> 6] >> (k & 63)) & 1ull) != 0) == want_filled;
      const uint64_t b = __ballot(in);
      if (lane == 0) sm.cnt[w] = __popcll(b);
      __syncthreads();
      int off = base, tot = 0;
#pragma unroll
      for (int i = 0; i < kThreads / 64; ++i) {
        const int n = sm.cnt[i];
        off += i < w ? n : 0;
        tot += n;
      }
      if (in) sm.rowid[off + __popcll(b & ((1ull << lane) - 1))] = load_row_id(a, rows, k, k1);
      base += tot;
      __syncthreads();  // cnt is rewritten by the next chunk
    }
    n_rows = base;
    for (int k = n_rows + tid; k < (n_rows + kT - 1) / kT * kT; k += kThreads) sm.rowid[k] = -1;
  }
  const int n_tiles = (n_rows + kT - 1) / kT;
  __syncthreads();
  if constexpr (FETCH) {
    // Who writes the filled rows to their hot rows.  With one verify token
    // and more than half of the key range filled (a step of misses), row i
    // by head group i mod nhg; otherwise head group 0 writes them all.  The
    // head groups of a key range count the same rows, so each row is
    // written once either way.
    int nfilled = 0;
#pragma unroll
    for (int i = 0; i < kThreads / 64; ++i) nfilled += sm.cnt[i];
    const bool share = a.tokens == 1 && 2 * nfilled > n_rows;
    rs.hg = share ? hg : (hg == 0 ? 0 : -1);
    rs.nhg = share ? nhg : 1;
  }

  const size_t head0 = (size_t)pair * H + hg * HG;
  if (w < 4)
    score_role<HG, FP8>(a, sm, kvs, head0, pair, hg, n_tiles, w, g, i16);
  else if (w < 8)
    value_role<HG, FP8>(a, sm, kvs, head0, pair, split, hg, n_tiles, w - 4, g, i16);
  else
    loader_role<HG, FP8, FETCH>(sm, rs, n_tiles, tid - 512);
  // nonfinite is final after every role's last barrier.
  if (sm.nonfinite || sm.vbad) {
    exact_fallback<HG, FP8, FETCH>(a, sm, rs, kvs, head0, pair, split, hg, n_rows, tid);
    if (tid == 0) atomicAdd(a.fallback_count, 1u);
  }
}

// Merge the split partials of one (layer, request, head) per wavefront.
// The per-split (m, l, l_exact) triples are read by lanes in parallel and
// reduced across the wave; the weights go through LDS, and the O rows are
// then accumulated with the loads of several splits in flight.  Lane i
// owns output columns [4i, 4i+4) and [256+4i, 256+4i+4).
constexpr int kCombineThreads = 256;
constexpr int kMaxSplits = kMaxTopK / kT;

__global__ __launch_bounds__(kCombineThreads) void combine_splits(DecodeArgs a) {
  __shared__ float f_s[kCombineThreads / 64][kMaxSplits];
  const int H = a.num_heads, S = a.split_total;
  const int wv = threadIdx.x >> 6;
  const size_t ph = (size_t)blockIdx.x * (kCombineThreads / 64) + wv;  // pair * H + head
  const int lane = threadIdx.x & 63;
  const size_t pair = ph / H;
  const int head = (int)(ph % H);
  const size_t sstride = (size_t)H * kPartW;  // floats between splits of one head
  const float* part0 = a.partial + (pair * S * H + head) * kPartW;
  float mloc = -INFINITY;
  for (int s = lane; s < S; s += 64) {
    const float* part = part0 + s * sstride;
    if (part[kVDim + 1] > 0.f) mloc = fmaxf(mloc, part[kVDim]);
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o, 64));
  const float mmax = mloc;
  float4* out = reinterpret_cast<float4*>(a.out + ph * kVDim);
  if (mmax == -INFINITY) {
    out[lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    out[64 + lane] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (lane == 0) a.lse[ph] = -INFINITY;
    return;
  }
  float L = 0.f, LE = 0.f;
  for (int s = lane; s < S; s += 64) {
    const float* part = part0 + s * sstride;
    const float ls = part[kVDim + 1];
    float f = 0.f;
    if (ls > 0.f) {
      f = exp2f(part[kVDim] - mmax);
      L += ls * f;
      LE += part[kVDim + 2] * f;
    }
    f_s[wv][s] = f;
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    L += __shfl_xor(L, o, 64);
    LE += __shfl_xor(LE, o, 64);
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  float4 o0 = make_float4(0.f, 0.f, 0.f, 0.f), o1 = o0;
#pragma unroll 8
  for (int s = 0; s < S; ++s) {
    const float f = f_s[wv][s];
    const float4* part = reinterpret_cast<const float4*>(part0 + s * sstride);
    const float4 x0 = part[lane], x1 = part[64 + lane];
    o0.x += x0.x * f; o0.y += x0.y * f; o0.z += x0.z * f; o0.w += x0.w * f;
    o1.x += x1.x * f; o1.y += x1.y * f; o1.z += x1.z * f; o1.w += x1.w * f;
  }
  const float inv = 1.f / L;
  out[lane] = make_float4(o0.x * inv, o0.y * inv, o0.z * inv, o0.w * inv);
  out[64 + lane] = make_float4(o1.x * inv, o1.y * inv, o1.z * inv, o1.w * inv);
  if (lane == 0) a.lse[ph] = (mmax + log2f(LE)) * 0.69314718055994531f;
}

}  // namespace

// Split partials of hisparse_sparse_mla_decode_layers_static, for callers
// that cannot allocate: a fixed array that every GPU the library runs on
// holds until the process ends.  Host code never passes `scratch` itself
// (its name is a host-side stand-in, not a device address); it looks up the
// device address once per device and passes that to the kernels.
static __device__ __align__(256) float scratch[HISPARSE_STATIC_SCRATCH_BYTES / sizeof(float)];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex scratch_mu;
float* scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t static_scratch_address(int device, float** out) {
  if (device < 0 || device >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(scratch_mu);
  if (!scratch_ptr[device]) {
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    scratch_ptr[device] = static_cast<float*>(ptr);
  }
  *out = scratch_ptr[device];
  return hipSuccess;
}

int head_group(int num_heads) { return num_heads % 64 == 0 ? 64 : (num_heads % 32 == 0 ? 32 : 16); }

int layer_workgroups(int num_requests, int num_heads) { return num_requests * (num_heads / head_group(num_heads)); }

// Key splits per (layer, query set, head group): enough workgroups to fill
// the 256 CUs, but at least two tiles each, since a workgroup's fixed costs
// (row ids, Q, the loader's first tiles, the partial write) outweigh a
// single tile (1M-token, 1-request workload: 89 us per step instead of 95).
constexpr int kMinTilesPerSplit = 2;

int decode_splits(int n_layers, int num_requests, int num_heads, int top_k) {
  const int base = n_layers * num_requests * (num_heads / head_group(num_heads));
  int splits = (256 + base - 1) / base;
  const int max_splits = (top_k + kMinTilesPerSplit * kT - 1) / (kMinTilesPerSplit * kT);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

// A decode that fetches is bound by the host link, not by the workgroup
// count: at least 8 tiles per key split keep each workgroup's loads
// streaming and halve the partials to merge (r8_ctx32k: 117 against 128 us
// per step with the 2-tile minimum; miss_1m 88 against 90).
constexpr int kMinTilesPerFetchSplit = 8;

int fetch_decode_splits(int n_layers, int num_requests, int num_heads, int top_k) {
  const int s = decode_splits(n_layers, num_requests, num_heads, top_k);
  return std::max(1, std::min(s, top_k / (kMinTilesPerFetchSplit * kT)));
}

// With at least 32 (request, head group) workgroups, the part beside the
// fetches runs without key splits (a whole fetch to hide under) and the
// part after the fetch is one launch without key splits that merges it, on
// workgroups of 16 heads: that part holds only the misses, so a workgroup
// has few tiles, and 16-head workgroups spread them over more CUs (the rows
// re-read by a request's head groups come from its XCD's L2) and merge
// fewer heads each.
// With fewer, the first part takes about 128 workgroups (at most
// kMaxMergeSlots key splits), leaving the other CUs to the fetch, and the
// second is split to fill the GPU and merged by combine_splits.
constexpr int kMergeMinWorkgroups = 32;

bool resident_first_pays(int num_requests, int num_heads) {
  return num_requests * (num_heads / head_group(num_heads)) >= kMergeMinWorkgroups;
}

void resident_first_splits(int num_requests, int num_heads, int top_k, int* before, int* after) {
  const int base = num_requests * (num_heads / head_group(num_heads));
  const int max_splits = (top_k + kMinTilesPerSplit * kT - 1) / (kMinTilesPerSplit * kT);
  if (base >= kMergeMinWorkgroups) {
    *before = 1;
    *after = 0;
  } else {
    *before = std::max(1, std::min({max_splits, kMaxMergeSlots, 128 / base}));
    *after = decode_splits(1, num_requests, num_heads, top_k);
  }
}

hipError_t launch_decode(hisparse_pool* p, const DecodeArgs& a, hipStream_t s, bool combine) {
  const int hgs = a.head_group > 0 ? a.head_group : head_group(a.num_heads);
  const int nhg = a.num_heads / hgs;
  const int grid = a.n_layers * a.num_requests * nhg * a.splits;
  prof_begin(p, a.fetch ? kKDecodeFetch : kKDecode, s);
  const bool fp8 = a.kv_dtype == HISPARSE_KV_FP8_E4M3;
  const dim3 gd(grid), bd(kThreads);
#define HS_DECODE(HG_, FP8_)                                                          \
  do {                                                                                \
    if (a.fetch) hipLaunchKernelGGL((decode_ws<HG_, FP8_, true>), gd, bd, 0, s, a, nhg); \
    else hipLaunchKernelGGL((decode_ws<HG_, FP8_, false>), gd, bd, 0, s, a, nhg);      \
  } while (0)
  if (hgs == 64) {
    if (fp8) HS_DECODE(64, true);
    else HS_DECODE(64, false);
  } else if (hgs == 32) {
    if (fp8) HS_DECODE(32, true);
    else HS_DECODE(32, false);
  } else {
    if (fp8) HS_DECODE(16, true);
    else HS_DECODE(16, false);
  }
#undef HS_DECODE
  hipError_t e = hipGetLastError();
  prof_end(p, s);
  if (e != hipSuccess || a.split_total == 1 || !combine) return e;
  prof_begin(p, kKCombine, s);
  // num_heads is a multiple of 16, so the (pair, head) count divides by 4
  hipLaunchKernelGGL(combine_splits, dim3(a.n_layers * a.num_requests * a.num_heads / (kCombineThreads / 64)),
                     dim3(kCombineThreads), 0, s, a);
  e = hipGetLastError();
  prof_end(p, s);
  return e;
}

}  // namespace hs
