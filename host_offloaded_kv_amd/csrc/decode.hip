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
// Work split: a workgroup handles (layer, request, 16-head group, K-split);
// rows are gathered tile by tile into LDS; the softmax is online (running
// max and sum in log2 units); split partials are merged by a second kernel.
#include "internal.h"

#include <cmath>

namespace hs {
namespace {

constexpr int kHG = 16;   // heads per workgroup
constexpr int kTR = 32;   // rows per tile
constexpr int kThreads = 256;
constexpr int kXPitch = kLatent + 8;  // bf16 elements per LDS row (16-byte multiple)
constexpr int kPartW = kVDim + 2;     // partial record: o[512], m, l

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__global__ __launch_bounds__(kThreads) void decode_tile(DecodeArgs a) {
  __shared__ float q_s[kHG][kLatent];
  __shared__ __align__(16) uint16_t x_s[kTR][kXPitch];
  __shared__ float p_s[kHG][kTR + 1];
  __shared__ float m_s[kHG], l_s[kHG], alpha_s[kHG];
  __shared__ int rowid_s[kTR];

  const int H = a.num_heads, R = a.num_requests, K = a.top_k;
  const int hgn = H / kHG;
  int bid = blockIdx.x;
  const int sp = bid % a.splits;
  bid /= a.splits;
  const int hg = bid % hgn;
  bid /= hgn;
  const int pair = bid;  // li * R + r
  const int li = pair / R;
  const int l = a.layer_begin + li;
  const int tid = threadIdx.x;
  const uint16_t* kv = a.kv[l];

  const int per = (K + a.splits - 1) / a.splits;
  const int k0 = sp * per;
  const int k1 = min(K, k0 + per);

  const uint16_t* q = a.q + ((size_t)pair * H + hg * kHG) * kLatent;
  for (int i = tid; i < kHG * kLatent; i += kThreads) q_s[i / kLatent][i % kLatent] = bf16_to_f32(q[i]) * a.scale_log2;
  if (tid < kHG) {
    m_s[tid] = -INFINITY;
    l_s[tid] = 0.f;
  }
  const int hh = tid / 16;       // head of this thread in the PV phase
  const int c0 = tid % 16;       // columns c0 + 16 i
  float o[kVDim / 16];
#pragma unroll
  for (int i = 0; i < kVDim / 16; ++i) o[i] = 0.f;
  const int32_t* rows = a.rows + (size_t)pair * K;

  for (int kb = k0; kb < k1; kb += kTR) {
    const int n = min(kTR, k1 - kb);
    __syncthreads();
    if (tid < kTR) {
      int row = tid < n ? rows[kb + tid] : -1;
      if (row < -1 || row >= a.kv_rows) {
        atomicOr(a.err, HISPARSE_ERR_ROW);
        row = -1;
      }
      rowid_s[tid] = row;
    }
    __syncthreads();
    for (int qc = tid; qc < kTR * kRowChunks; qc += kThreads) {
      const int j = qc / kRowChunks, c = qc % kRowChunks;
      const int row = rowid_s[j];
      uint4 v = make_uint4(0, 0, 0, 0);
      if (row >= 0) v = *(reinterpret_cast<const uint4*>(kv + (size_t)row * kLatent) + c);
      *reinterpret_cast<uint4*>(&x_s[j][c * 8]) = v;
    }
    __syncthreads();
    {
      const int h = tid / 16;
      const int j0 = (tid % 16) * 2;
#pragma unroll
      for (int jj = 0; jj < 2; ++jj) {
        const int j = j0 + jj;
        float acc = 0.f;
        for (int d = 0; d < kLatent; ++d) acc += q_s[h][d] * bf16_to_f32(x_s[j][d]);
        p_s[h][j] = rowid_s[j] >= 0 ? acc : -INFINITY;
      }
    }
    __syncthreads();
    if (tid < kHG) {
      float mx = -INFINITY;
      for (int j = 0; j < kTR; ++j) mx = fmaxf(mx, p_s[tid][j]);
      const float m_old = m_s[tid];
      const float m_new = fmaxf(m_old, mx);
      float alpha = 1.f, sum = 0.f;
      if (m_new != -INFINITY) {
        alpha = exp2f(m_old - m_new);
        for (int j = 0; j < kTR; ++j) {
          const float e = exp2f(p_s[tid][j] - m_new);
          p_s[tid][j] = e;
          sum += e;
        }
      } else {
        for (int j = 0; j < kTR; ++j) p_s[tid][j] = 0.f;
      }
      l_s[tid] = l_s[tid] * alpha + sum;
      m_s[tid] = m_new;
      alpha_s[tid] = alpha;
    }
    __syncthreads();
    const float al = alpha_s[hh];
#pragma unroll
    for (int i = 0; i < kVDim / 16; ++i) {
      const int c = c0 + 16 * i;
      float acc = o[i] * al;
      for (int j = 0; j < n; ++j) acc += p_s[hh][j] * bf16_to_f32(x_s[j][c]);
      o[i] = acc;
    }
  }
  __syncthreads();
  const int head = hg * kHG + hh;
  const float m = m_s[hh], lsum = l_s[hh];
  if (a.splits == 1) {
    float* out = a.out + ((size_t)pair * H + head) * kVDim;
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
    for (int i = 0; i < kVDim / 16; ++i) out[c0 + 16 * i] = o[i] * inv;
    if (c0 == 0) a.lse[(size_t)pair * H + head] = lsum > 0.f ? (m + log2f(lsum)) * 0.69314718055994531f : -INFINITY;
  } else {
    float* part = a.partial + (((size_t)pair * a.splits + sp) * H + head) * kPartW;
#pragma unroll
    for (int i = 0; i < kVDim / 16; ++i) part[c0 + 16 * i] = o[i];
    if (c0 == 0) {
      part[kVDim] = m;
      part[kVDim + 1] = lsum;
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

int decode_splits(int n_layers, int num_requests, int num_heads, int top_k) {
  const int base = n_layers * num_requests * (num_heads / kHG);
  int splits = (1024 + base - 1) / base;
  const int max_splits = (top_k + kTR - 1) / kTR;
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  return splits;
}

hipError_t launch_decode(hisparse_pool* p, const DecodeArgs& a, hipStream_t s) {
  const int grid = a.n_layers * a.num_requests * (a.num_heads / kHG) * a.splits;
  prof_begin(p, kKDecode, s);
  hipLaunchKernelGGL(decode_tile, dim3(grid), dim3(kThreads), 0, s, a);
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
