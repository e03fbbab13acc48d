// Token-level sparse decode (library card page "FlashMLA: Efficient Multi-head Latent Attention
// Kernels": sparse attention over selected tokens in decoding, with an FP8 cache): each query
// token (sequence i, token j) attends to its own list of top-k token positions. This pre-pass
// turns every list into the cache rows the decode kernel gathers: entry u of the list is a key
// when 0 <= u < min(t_i, max_pages * 64) (others are padding and dropped), its row is
// block_table[i, u / 64] * 64 + u % 64, stored + 1 (0 = a key whose page id is outside
// [0, num_pages), which reads as zeros, as in the dense decode). The kept entries are packed
// to the front of the query token's row list, in list order, the rest filled with 0, and their
// count becomes that query token's visible length for the split plan, which then treats each
// query token as a sequence of one query row per head.
//
// One wave per query token; 64 entries per pass, packed with a ballot and a lane prefix count.
#include "mla_device.h"

namespace mla {
namespace {

__global__ __launch_bounds__(64) void sparse_rows_kernel(const int32_t* __restrict__ indices, int topk,
                                                         const int32_t* __restrict__ block_table, int max_pages,
                                                         const int32_t* __restrict__ seqlens, int s_q,
                                                         int64_t num_pages, int32_t* __restrict__ rows, int stride,
                                                         int32_t* __restrict__ vis) {
  const int v = blockIdx.x, i = v / s_q, lane = threadIdx.x;
  int t = seqlens[i];
  const int cap = max_pages * kPage;
  t = t < cap ? t : cap;
  const int32_t* src = indices + (int64_t)v * topk;
  int32_t* dst = rows + (int64_t)v * stride;
  int kept = 0;
  for (int e0 = 0; e0 < topk; e0 += 64) {
    const int e = e0 + lane;
    const int u = e < topk ? src[e] : -1;
    const bool key = u >= 0 && u < t;
    int32_t stored = 0;
    if (key) {
      const int pid = block_table[(int64_t)i * max_pages + (u >> 6)];
      if (pid >= 0 && (int64_t)pid < num_pages) stored = pid * kPage + (u & (kPage - 1)) + 1;
    }
    const uint64_t mask = __ballot(key);
    const int before = __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0));
    if (key) dst[kept + before] = stored;
    kept += __popcll(mask);
  }
  for (int e = kept + lane; e < stride; e += 64) dst[e] = 0;
  if (lane == 0) vis[v] = kept;
}

}  // namespace

hipError_t launch_sparse_rows(const int32_t* indices, int topk, const int32_t* block_table, int max_pages,
                              const int32_t* seqlens, int batch, int s_q, int64_t num_pages, int32_t* rows,
                              int stride, int32_t* vis, hipStream_t stream) {
  hipLaunchKernelGGL(sparse_rows_kernel, dim3(batch * s_q), dim3(64), 0, stream, indices, topk, block_table,
                     max_pages, seqlens, s_q, num_pages, rows, stride, vis);
  return hipGetLastError();
}

}  // namespace mla
