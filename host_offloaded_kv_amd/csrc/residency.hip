// Residency transitions around the decode step (gfx950): appending each
// request's new token to its GPU-resident tail page, and materialising
// completed pages in the pinned host pool.
//
// The vLLM Hybrid HiSparse blog (section "工作原理") describes the states a
// request moves through: fully resident, mixed (the tail stays on the GPU,
// older pages only in host memory, a block table of real blocks and
// placeholders), and none.  Two mechanisms keep those transitions cheap:
//  * when a page of the context completes, a copy of it to host memory is
//    queued while the GPU keeps serving it, so the page can later give up
//    its GPU block without another copy;
//  * the copy of all sparse-MLA layers is one launch after the forward
//    pass, ordered on the model's stream.
// Here:
//  * append_rows: one workgroup per request writes the new token's row of
//    every layer into the row of its tail page (block bt[r][ctx_r / page]),
//    then advances ctx_r.  A tail page that is not resident, or a full
//    context, sets HISPARSE_ERR_APPEND and leaves that request unchanged.
//  * writeback_rows: one workgroup per (layer, request) copies the rows
//    [hv, floor(ctx / page) * page) -- every page completed since the last
//    write-back, from the first position the host pool does not hold yet --
//    from their resident blocks to the host pool with zero-copy 16-byte
//    stores, then advances hv.  A completed page that is not resident
//    (dropped before being copied) sets HISPARSE_ERR_UNMATERIALIZED.
#include "internal.h"

namespace hs {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kAppendThreads = 256;
constexpr int kWritebackThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void append_rows(AppendArgs a) {
  const int r = blockIdx.x;
  const int R = a.num_requests;
  const int pos = a.ctx[r];
  const int page = pos >> a.page_shift;
  const int blk = pos < a.capacity[r] ? a.bt[a.bt_off[r] + page] : -1;
  if (blk < 0) {
    if (threadIdx.x == 0) atomicOr(a.err, HISPARSE_ERR_APPEND);
    return;
  }
  const int64_t row = ((int64_t)blk << a.page_shift) + (pos & ((1 << a.page_shift) - 1));
  const int rc = a.row_chunks;
  for (int i = threadIdx.x; i < a.num_layers * rc; i += kAppendThreads) {
    const int l = i / rc, c = i - l * rc;
    const u32x4* src = reinterpret_cast<const u32x4*>(a.rows + ((size_t)l * R + r) * rc * 16) + c;
    u32x4* dst = reinterpret_cast<u32x4*>(a.kv[l] + row * rc * 16) + c;
    *dst = *src;
  }
  __syncthreads();
  if (threadIdx.x == 0) a.ctx[r] = pos + 1;
}

__global__ __launch_bounds__(kWritebackThreads) void writeback_rows(WritebackArgs a) {
  const int R = a.num_requests;
  const int l = blockIdx.x / R;
  const int r = blockIdx.x - l * R;
  const int pshift = a.page_shift;
  const int pmask = (1 << pshift) - 1;
  const int from = a.hv[(size_t)l * R + r];
  const int to = (a.ctx[r] >> pshift) << pshift;  // complete pages only
  if (to <= from) return;
  const int32_t* bt = a.bt + a.bt_off[r];
  u32x4* host = reinterpret_cast<u32x4*>(a.host_rows[(size_t)l * R + r]);
  const unsigned char* kv = a.kv[l];
  const int rc = a.row_chunks;
  bool bad = false;
  const int64_t n = (int64_t)(to - from) * rc;
  for (int64_t i = threadIdx.x; i < n; i += kWritebackThreads) {
    const int p = from + (int)(i / rc);
    const int c = (int)(i - (int64_t)(p - from) * rc);
    const int blk = bt[p >> pshift];
    if (blk < 0) {
      bad = true;
      continue;
    }
    const u32x4 v = reinterpret_cast<const u32x4*>(kv + (((int64_t)blk << pshift) + (p & pmask)) * rc * 16)[c];
    __builtin_nontemporal_store(v, host + (size_t)p * rc + c);
  }
  if (__syncthreads_or(bad)) {
    if (threadIdx.x == 0) atomicOr(a.err, HISPARSE_ERR_UNMATERIALIZED);
    return;  // hv stays: the host pool does not hold these rows
  }
  if (threadIdx.x == 0) a.hv[(size_t)l * R + r] = to;
}

}  // namespace

hipError_t launch_append(hisparse_pool* p, const AppendArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(append_rows, dim3(a.num_requests), dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_writeback(hisparse_pool* p, const WritebackArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(writeback_rows, dim3(a.num_layers * a.num_requests), dim3(kWritebackThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace hs
