// Token-level sparse decode (library card page "FlashMLA: Efficient Multi-head Latent Attention
// Kernels": sparse attention over selected tokens in decoding, with an FP8 cache): each query
// token (sequence i, token j) attends to its own list of top-k token positions. This pre-pass
// turns every list into the cache rows the decode kernel gathers: entry u of the list is a key
// when 0 <= u < min(t_i, max_pages * 64) (others are padding and dropped), its row is
// block_table[i, u / 64] * 64 + u % 64, stored + 1 (0 = a key whose page id is outside
// [0, num_pages), which reads as zeros, as in the dense decode, and is reported in the status word). The kept entries are packed
// to the front of the query token's row list, in list order, the rest filled with 0, and their
// count becomes that query token's visible length for the split plan, which then treats each
// query token as a sequence of one query row per head.
//
// One 256-thread work-group per query token. The list is taken in blocks of 2,048 entries, 8
// consecutive ones per thread, so that a block's index loads and then its block-table loads
// are all in flight at once; a work-group prefix sum over the per-thread key counts (a shuffle
// scan within each wave, then the four wave totals through LDS) places every thread's keys,
// which keeps list order.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kSrThreads = 256;
constexpr int kSrPer = 8;   // consecutive entries per thread and block

__global__ __launch_bounds__(kSrThreads) void sparse_rows_kernel(const int32_t* __restrict__ indices, int topk,
                                                                 const int32_t* __restrict__ block_table,
                                                                 int max_pages, const int32_t* __restrict__ seqlens,
                                                                 int s_q, int64_t num_pages, int32_t* __restrict__ rows,
                                                                 int stride, int32_t* __restrict__ vis,
                                                                 int32_t* __restrict__ status) {
  __shared__ int wave_tot[4];
  const int v = blockIdx.x, i = v / s_q, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int t = seqlens[i];
  const int cap = max_pages * kPage;
  t = t < cap ? t : cap;
  const int32_t* src = indices + (int64_t)v * topk;
  int32_t* dst = rows + (int64_t)v * stride;
  int kept = 0;   // keys placed by the earlier blocks (the same in every thread)
  bool bad_page = false;
  for (int e0 = 0; e0 < topk; e0 += kSrThreads * kSrPer) {
    int u[kSrPer], stored[kSrPer];
#pragma unroll
    for (int r = 0; r < kSrPer; ++r) {
      const int e = e0 + kSrPer * tid + r;
      u[r] = e < topk ? src[e] : -1;
    }
    int mine = 0;
#pragma unroll
    for (int r = 0; r < kSrPer; ++r) {
      const bool key = u[r] >= 0 && u[r] < t;
      stored[r] = -1;   // (not a key)
      if (key) {
        const int pid = block_table[(int64_t)i * max_pages + (u[r] >> 6)];
        const bool in_range = pid >= 0 && (int64_t)pid < num_pages;
        stored[r] = in_range ? pid * kPage + (u[r] & (kPage - 1)) + 1 : 0;
        bad_page = bad_page || !in_range;
        ++mine;
      }
    }
    // exclusive prefix of `mine` over the work-group
    int incl = mine;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(incl, d, 64);
      if (lane >= d) incl += y;
    }
    if (lane == 63) wave_tot[wave] = incl;
    __syncthreads();
    int before = incl - mine;
    for (int w = 0; w < wave; ++w) before += wave_tot[w];
    const int block_tot = wave_tot[0] + wave_tot[1] + wave_tot[2] + wave_tot[3];
    __syncthreads();   // (wave_tot is rewritten by the next block)
    int pos = kept + before;
#pragma unroll
    for (int r = 0; r < kSrPer; ++r)
      if (stored[r] >= 0) dst[pos++] = stored[r];
    kept += block_tot;
  }
  for (int e = kept + tid; e < stride; e += kSrThreads) dst[e] = 0;
  if (tid == 0) vis[v] = kept;
  if (status != nullptr && bad_page)
    __hip_atomic_fetch_or(status, (int)kDevPageOutOfRange, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t launch_sparse_rows(const int32_t* indices, int topk, const int32_t* block_table, int max_pages,
                              const int32_t* seqlens, int batch, int s_q, int64_t num_pages, int32_t* rows,
                              int stride, int32_t* vis, int32_t* status, hipStream_t stream) {
  hipLaunchKernelGGL(sparse_rows_kernel, dim3(batch * s_q), dim3(kSrThreads), 0, stream, indices, topk, block_table,
                     max_pages, seqlens, s_q, num_pages, rows, stride, vis, status);
  return hipGetLastError();
}

}  // namespace mla
