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
// K split); 32-row tiles are gathered into LDS with direct-to-LDS loads
// (double-buffered), QK^T and PV run on 16x16x32 bf16 MFMA with fp32
// accumulation, and split partials are merged by a second kernel.
#include "internal.h"

#include <cmath>

namespace hs {
namespace {

constexpr int kT = 32;                        // rows per tile
constexpr int kPitchChunks = kRowChunks + 2;  // LDS row pitch: 72 data + 2 pad chunks (1184 bytes)
constexpr int kPitch = kPitchChunks * 16;
constexpr int kTileBytes = kT * kPitch;       // 37888 = 37 KiB
constexpr int kTileBlocks = kTileBytes / 1024; // 1 KiB direct-to-LDS blocks per tile
constexpr int kThreads = 256;                 // 4 wavefronts
constexpr int kPPitch = kT + 8;               // bf16 per P row (80 bytes)
constexpr int kPartW = kVDim + 2;             // partial record: o[512], m, l
constexpr float kMaxGrowLog2 = 64.f;          // P = 2^(s - m) may reach 2^64 before a restart

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) unsigned char lds_u8;

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
  const uint32_t a = __builtin_bit_cast(uint16_t, (__bf16)lo);
  const uint32_t b = __builtin_bit_cast(uint16_t, (__bf16)hi);
  return a | (b << 16);
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

// Issue the direct-to-LDS loads of one tile.  The tile is kT rows of
// kPitch bytes; block b (1 KiB) is written by one wavefront instruction,
// lane l landing at byte 16 (64 b + l).  Slot s = 64 b + l is chunk
// s % kPitchChunks of row s / kPitchChunks; the two pad chunks of a row
// re-read its first chunk (an L1 hit) and are never used.
__device__ __forceinline__ void issue_tile(const uint16_t* kv, unsigned char* xs, const int* rowid, int w, int lane) {
  for (int blk = w; blk < kTileBlocks; blk += 4) {
    const int slot = blk * 64 + lane;
    const int j = slot / kPitchChunks;
    int c = slot - j * kPitchChunks;
    c = c < kRowChunks ? c : 0;
    const int rid = rowid[j];
    const uint16_t* src = kv + (size_t)(rid < 0 ? 0 : rid) * kLatent + c * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_u8*)(xs + blk * 1024), 16, 0, 0);
  }
}

// D += A * B on a 16x16x32 bf16 MFMA (fp32 accumulate), compiler-scheduled.
__device__ __forceinline__ void mfma16(f32x4& d, const u32x4& a, const u32x4& b) {
  d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), d, 0, 0, 0);
}

// The PV accumulators are pinned to AGPRs with inline asm ("a" constraint):
// with the builtin the register allocator keeps them in VGPRs next to the
// 144-register Q operand and copies them through AGPRs around every MFMA.
// The compiler does not see these as MFMAs, so the two hazards they can
// meet are covered by hand:
//  * an operand written by a VALU instruction just before: two wait states
//    in front of the first MFMA that reads a freshly assembled operand;
//  * reading the accumulators afterwards (v_accvgpr_read): agpr_drain()
//    inserts 24 wait states, more than an 8-pass MFMA needs.
// Back-to-back MFMAs that chain through srcC need no wait states.
__device__ __forceinline__ void mfma16_agpr(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma16_agpr_after_valu(f32x4& d, const u32x4& a, const u32x4& b) {
  asm("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void zero_agpr(f32x4& d) {
  const u32x4 z = {0u, 0u, 0u, 0u};
  asm volatile("s_nop 1\n\tv_mfma_f32_16x16x32_bf16 %0, %1, %1, 0" : "=a"(d) : "v"(z));
}
__device__ __forceinline__ void agpr_drain() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory"); }

// One workgroup = (layer, request, group of HG heads, K split).  Wave w:
//  * QK^T: rows 16*(w%2) .. +15 of the tile against heads
//    (w/2)*SH .. +SH-1 of the group (SH = max(16, HG/2)), Q in registers;
//  * PV: output columns 128 w .. 128 w + 127 for all HG heads.
template <int HG>
__global__ __launch_bounds__(kThreads, 1) void decode_mfma(DecodeArgs a, int nhg) {
  constexpr int SH = HG / 2 < 16 ? 16 : HG / 2;  // heads per wave in QK^T
  constexpr int NBW = SH / 16;                    // 16-head blocks per wave in QK^T
  constexpr int NBP = HG / 16;                    // 16-head blocks in PV
  __shared__ __align__(16) unsigned char xs[2][kTileBytes];
  __shared__ __align__(16) uint16_t ps[HG][kPPitch];
  __shared__ float mred[2][HG];
  __shared__ float lred[2][HG];
  __shared__ float mfin_s[HG];
  __shared__ int rowid_s[2][kT];
  __shared__ int restart_s;

  const int H = a.num_heads, R = a.num_requests, K = a.top_k;
  // XCD-aware order: consecutive logical blocks (the head groups and splits
  // of one request) share blockIdx % 8, i.e. one XCD and its L2.
  int li = blockIdx.x;
  if (gridDim.x % 8 == 0) li = (blockIdx.x % 8) * (gridDim.x / 8) + blockIdx.x / 8;
  const int split = li % a.splits;
  li /= a.splits;
  const int hg = li % nhg;
  const int pair = li / nhg;
  const int l = a.layer_begin + pair / R;
  const uint16_t* kv = a.kv[l];
  const int32_t* rows = a.rows + (size_t)pair * K;

  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63, g = lane >> 4, i16 = lane & 15;
  const int rb = w & 1, hw = w >> 1;
  const bool s_active = hw * SH < HG;

  int per = (K + a.splits - 1) / a.splits;
  per = (per + kT - 1) / kT * kT;
  const int k0 = split * per;
  const int k1 = min(K, k0 + per);
  const int n_tiles = k1 > k0 ? (k1 - k0 + kT - 1) / kT : 0;

  // Q of this wave's QK^T heads, in the MFMA B-operand layout:
  // lane (g, i16) holds dims 32 s + 8 g .. +7 of head (block nb, i16).
  u32x4 qreg[NBW][kLatent / 32];
  if (s_active) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      const int head = hg * HG + hw * SH + nb * 16 + i16;
      const u32x4* qp = reinterpret_cast<const u32x4*>(a.q + ((size_t)pair * H + head) * kLatent + 8 * g);
#pragma unroll
      for (int s = 0; s < kLatent / 32; ++s) qreg[nb][s] = qp[4 * s];
    }
  }
  float m_run[NBW], l_run[NBW];
#pragma unroll
  for (int nb = 0; nb < NBW; ++nb) {
    m_run[nb] = -INFINITY;
    l_run[nb] = 0.f;
  }
  f32x4 o[8][NBP];
#pragma unroll
  for (int mb = 0; mb < 8; ++mb)
#pragma unroll
    for (int nb = 0; nb < NBP; ++nb) zero_agpr(o[mb][nb]);

  if (tid < kT) {
    rowid_s[0][tid] = load_row_id(a, rows, k0 + tid, k1);
    rowid_s[1][tid] = load_row_id(a, rows, k0 + kT + tid, k1);
  }
  __syncthreads();
  if (n_tiles > 0) issue_tile(kv, xs[0], rowid_s[0], w, lane);

  // Softmax with a fixed reference max per head: the first valid tile sets
  // m, and P = 2^(s*scale*log2e - m) accumulates unnormalised.  If a later
  // tile exceeds m by more than 2^64, every wave restarts from tile 0 with
  // the larger m (exact either way; never taken unless scores jump that
  // far), so the O accumulators never need rescaling inside the loop.
  for (int it = 0; it < n_tiles; ++it) {
    const int buf = it & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (tid == 0) restart_s = 0;
    if (it + 1 < n_tiles) issue_tile(kv, xs[buf ^ 1], rowid_s[buf ^ 1], w, lane);
    const unsigned char* xb = xs[buf];

    // ---- QK^T and the tile max -------------------------------------------
    f32x4 sacc[NBW];
    bool valid[4];
    if (s_active) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) sacc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
      // A operand: lane (g, i16) reads row 16 rb + i16, dims 32 s + 8 g .. +7.
      const unsigned char* xrow = xb + (16 * rb + i16) * kPitch + 16 * g;
#pragma unroll
      for (int s = 0; s < kLatent / 32; ++s) {
        const u32x4 av = *reinterpret_cast<const u32x4*>(xrow + 64 * s);
#pragma unroll
        for (int nb = 0; nb < NBW; ++nb) mfma16(sacc[nb], av, qreg[nb][s]);
        if ((s & 3) == 3) __builtin_amdgcn_sched_barrier(0);  // bound operand prefetch (registers)
      }
#pragma unroll
      for (int v = 0; v < 4; ++v) valid[v] = rowid_s[buf][16 * rb + 4 * g + v] >= 0;
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          sacc[nb][v] = valid[v] ? sacc[nb][v] * a.scale_log2 : -INFINITY;
          mx = fmaxf(mx, sacc[nb][v]);
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
        mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
        if (g == 0) mred[rb][hw * SH + nb * 16 + i16] = mx;
      }
    }
    __syncthreads();
    // ---- softmax against the reference max, P to LDS -----------------------
    if (s_active) {
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) {
        const int hs = hw * SH + nb * 16 + i16;
        const float mt = fmaxf(mred[0][hs], mred[1][hs]);
        if (m_run[nb] == -INFINITY) {
          m_run[nb] = mt;  // first valid rows of this head: O and l are still zero
        } else if (mt > m_run[nb] + kMaxGrowLog2) {
          m_run[nb] = mt;
          restart_s = 1;
        }
        const float m = m_run[nb];
        float p[4], sum = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          p[v] = valid[v] ? __builtin_amdgcn_exp2f(sacc[nb][v] - m) : 0.f;
          sum += p[v];
        }
        l_run[nb] += sum;
        u32x2 pk = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
        *reinterpret_cast<u32x2*>(&ps[hs][16 * rb + 4 * g]) = pk;
      }
    }
    __syncthreads();
    if (__builtin_expect(restart_s != 0, 0)) {
      // Rare path: drop everything accumulated and start over from tile 0.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int mb = 0; mb < 8; ++mb)
#pragma unroll
        for (int nb = 0; nb < NBP; ++nb) zero_agpr(o[mb][nb]);
#pragma unroll
      for (int nb = 0; nb < NBW; ++nb) l_run[nb] = 0.f;
      __syncthreads();
      if (tid < kT) {
        rowid_s[0][tid] = load_row_id(a, rows, k0 + tid, k1);
        rowid_s[1][tid] = load_row_id(a, rows, k0 + kT + tid, k1);
      }
      __syncthreads();
      issue_tile(kv, xs[0], rowid_s[0], w, lane);
      it = -1;
      continue;
    }
    if (tid < kT) rowid_s[buf][tid] = load_row_id(a, rows, k0 + (it + 2) * kT + tid, k1);
    // ---- PV: O^T[128 cols x HG heads] += X^T[cols x 32 rows] P^T[32 x HG] ---
    u32x4 bp[NBP];
#pragma unroll
    for (int nb = 0; nb < NBP; ++nb) bp[nb] = *reinterpret_cast<const u32x4*>(&ps[nb * 16 + i16][8 * g]);
    // Transposed A operand: lane i16 of each 16-lane group supplies row
    // j0 + i16/4, columns c0 + 4 (i16 % 4) .. +3, and receives column
    // c0 + i16 of rows j0 .. j0+3 (j0 = 8 g, then 8 g + 4).
    const lds_u8* xl = (const lds_u8*)xb + (8 * g + (i16 >> 2)) * kPitch + (128 * w + 4 * (i16 & 3)) * 2;
#pragma unroll
    for (int mb = 0; mb < 8; ++mb) {
      const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(xl + 32 * mb));
      const s16x4 hi =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(xl + 32 * mb + 4 * kPitch));
      const u32x4 av = __builtin_bit_cast(u32x4, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
      mfma16_agpr_after_valu(o[mb][0], av, bp[0]);
#pragma unroll
      for (int nb = 1; nb < NBP; ++nb) mfma16_agpr(o[mb][nb], av, bp[nb]);
      if (mb & 1) __builtin_amdgcn_sched_barrier(0);
    }
  }

  agpr_drain();
  // ---- epilogue: combine the row-half sums, normalise, write --------------
  if (s_active) {
#pragma unroll
    for (int nb = 0; nb < NBW; ++nb) {
      float ls = l_run[nb];
      ls += __shfl_xor(ls, 16, 64);
      ls += __shfl_xor(ls, 32, 64);
      const int hs = hw * SH + nb * 16 + i16;
      if (g == 0) {
        lred[rb][hs] = ls;
        if (rb == 0) mfin_s[hs] = m_run[nb];
      }
    }
  }
  __syncthreads();
  const size_t head0 = (size_t)pair * H + hg * HG;
#pragma unroll
  for (int nb = 0; nb < NBP; ++nb) {
    const int h = nb * 16 + i16;
    const float lsum = lred[0][h] + lred[1][h];
    const float m = mfin_s[h];
    if (a.splits == 1) {
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      float* out = a.out + (head0 + h) * kVDim + 128 * w + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) *reinterpret_cast<f32x4*>(out + 16 * mb) = o[mb][nb] * inv;
      if (w == 0 && g == 0) a.lse[head0 + h] = lsum > 0.f ? (m + __builtin_amdgcn_logf(lsum)) * 0.69314718055994531f : -INFINITY;
    } else {
      float* part = a.partial + (((size_t)pair * a.splits + split) * H + hg * HG + h) * kPartW;
      float* po = part + 128 * w + 4 * g;
#pragma unroll
      for (int mb = 0; mb < 8; ++mb) {
#pragma unroll
        for (int v = 0; v < 4; ++v) po[16 * mb + v] = o[mb][nb][v];
      }
      if (w == 0 && g == 0) {
        part[kVDim] = m;
        part[kVDim + 1] = lsum;
      }
    }
  }
}

__global__ __launch_bounds__(256) void combine_splits(DecodeArgs a) {
  const int H = a.num_heads;
  const size_t ph = blockIdx.x;  // pair * H + head
  const size_t pair = ph / H;
  const int head = (int)(ph % H);
  float mmax = -INFINITY;
  for (int s = 0; s < a.splits; ++s) {
    const float* part = a.partial + ((pair * a.splits + s) * H + head) * kPartW;
    if (part[kVDim + 1] > 0.f) mmax = fmaxf(mmax, part[kVDim]);
  }
  float* out = a.out + ph * kVDim;
  if (mmax == -INFINITY) {
    for (int c = threadIdx.x; c < kVDim; c += 256) out[c] = 0.f;
    if (threadIdx.x == 0) a.lse[ph] = -INFINITY;
    return;
  }
  float L = 0.f;
  for (int s = 0; s < a.splits; ++s) {
    const float* part = a.partial + ((pair * a.splits + s) * H + head) * kPartW;
    const float ls = part[kVDim + 1];
    if (ls > 0.f) L += ls * exp2f(part[kVDim] - mmax);
  }
  const float inv = 1.f / L;
  for (int c = threadIdx.x; c < kVDim; c += 256) {
    float acc = 0.f;
    for (int s = 0; s < a.splits; ++s) {
      const float* part = a.partial + ((pair * a.splits + s) * H + head) * kPartW;
      const float ls = part[kVDim + 1];
      if (ls > 0.f) acc += part[c] * exp2f(part[kVDim] - mmax);
    }
    out[c] = acc * inv;
  }
  if (threadIdx.x == 0) a.lse[ph] = (mmax + log2f(L)) * 0.69314718055994531f;
}

}  // namespace

int head_group(int num_heads) { return num_heads % 64 == 0 ? 64 : (num_heads % 32 == 0 ? 32 : 16); }

int decode_splits(int n_layers, int num_requests, int num_heads, int top_k) {
  const int base = n_layers * num_requests * (num_heads / head_group(num_heads));
  int splits = (256 + base - 1) / base;
  const int max_splits = (top_k + kT - 1) / kT;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

hipError_t launch_decode(hisparse_pool* p, const DecodeArgs& a, hipStream_t s) {
  const int hgs = head_group(a.num_heads);
  const int nhg = a.num_heads / hgs;
  const int grid = a.n_layers * a.num_requests * nhg * a.splits;
  prof_begin(p, kKDecode, s);
  if (hgs == 64)
    hipLaunchKernelGGL(decode_mfma<64>, dim3(grid), dim3(kThreads), 0, s, a, nhg);
  else if (hgs == 32)
    hipLaunchKernelGGL(decode_mfma<32>, dim3(grid), dim3(kThreads), 0, s, a, nhg);
  else
    hipLaunchKernelGGL(decode_mfma<16>, dim3(grid), dim3(kThreads), 0, s, a, nhg);
  hipError_t e = hipGetLastError();
  prof_end(p, s);
  if (e != hipSuccess || a.splits == 1) return e;
  prof_begin(p, kKCombine, s);
  hipLaunchKernelGGL(combine_splits, dim3(a.n_layers * a.num_requests * a.num_heads), dim3(256), 0, s, a);
  e = hipGetLastError();
  prof_end(p, s);
  return e;
}

}  // namespace hs
