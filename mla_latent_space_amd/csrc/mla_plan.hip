// Split-KV planner: one 1024-thread work-group builds the whole plan on the device.
//
// FlashMLA-2 newsletter page, section "Architectural Analysis": a radix-sorted block
// scheduler balances sequence partitions across compute units so that 128-token and
// 128k-token sequences in one batch leave no stragglers. This kernel is that idea on
// gfx950: items (sequence, 128-row tile) are keyed by page count, sorted longest first
// (up to 1024 items by a rank sort, beyond that by a two-pass LSD radix sort in LDS with
// 8-bit digits and wave ballots for the stable rank),
// costed as overhead + pages, prefix-summed, and cut into equal-cost contiguous runs,
// one per worker (one persistent decode work-group per compute unit). An item's overhead
// is spread evenly over its pages (page j of item k starts at C_k + j (overhead + pages) /
// pages), so equal items cut into equal page counts.
#include "mla_internal.h"

namespace mla {
namespace {

constexpr int kThreads = 1024;         // block size for batches of more than 256 items
constexpr int kThreadsSmall = 256;     // ... and up to 256 items (cheaper barriers)
constexpr int kWaves = kThreads / 64;

__device__ inline void item_shape(const int32_t* seqlens, int idx, int tiles, int s_q, int heads, int causal,
                                  int* seq, int* tile, int* vis, int* pages) {
  const int sq = idx / tiles, tl = idx - sq * tiles;
  int t = seqlens[sq];
  t = t < 0 ? 0 : t;
  const int cap = kMaxPagesPerSeq * kPage;
  t = t > cap ? cap : t;
  int v = t;
  if (causal) {
    const int rows = s_q * heads;
    int last_row = (tl + 1) * kRowsPerTile;
    last_row = (last_row < rows ? last_row : rows) - 1;
    const int j_last = last_row / heads;
    v = t - s_q + 1 + j_last;
    v = v < 0 ? 0 : (v > t ? t : v);
  }
  int p = (v + kPage - 1) / kPage;
  *seq = sq; *tile = tl; *vis = v; *pages = p < 1 ? 1 : p;
}

// Exclusive scan over the block: each thread contributes `x`, returns its exclusive prefix,
// `total` gets the block sum. `scratch` holds >= blockDim.x / 64 ints.
__device__ inline int block_exclusive_scan(int x, int* scratch, int* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const int y = __shfl_up(incl, d, 64);
    if (lane >= d) incl += y;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  int wave_off = 0, tot = 0;
  const int nwaves = blockDim.x >> 6;
  for (int w = 0; w < nwaves; ++w) {
    const int s = scratch[w];
    wave_off += (w < wave) ? s : 0;
    tot += s;
  }
  __syncthreads();
  *total = tot;
  return wave_off + incl - x;
}

// Worker of page j of an item with cost prefix ck and `pages` pages: floor(x W / C) for the
// page's start x = ck + j (overhead + pages) / pages, in integers.
__device__ inline int page_worker(int64_t ck, int64_t pages, int64_t j, int64_t total, int64_t W) {
  return (int)(((ck * pages + j * (kPlanOverhead + pages)) * W) / (total * pages));
}

// First (item, page) of worker w: the first page whose start position is >= w C / Weff, or
// (n, 0) past the active workers. `cost` holds the cost prefixes of the sorted keys `keys`.
__device__ inline void worker_start(int64_t w, int n, int64_t Weff, int64_t C, const int* cost, const uint32_t* keys,
                                    int* sk, int* sp) {
  if (w >= Weff) { *sk = n; *sp = 0; return; }
  const int64_t b = w * C;   // position w C / Weff, times Weff
  int l = 0, r = n - 1;      // largest k with cost[k] Weff <= b
  while (l < r) {
    const int m = (l + r + 1) >> 1;
    if ((int64_t)cost[m] * Weff <= b) l = m; else r = m - 1;
  }
  const int64_t pages = 0xFFFF - (int64_t)(keys[l] >> 16);
  const int64_t num = (b - (int64_t)cost[l] * Weff) * pages;
  const int64_t den = Weff * (kPlanOverhead + pages);
  const int64_t j = (num + den - 1) / den;   // smallest j whose start is >= w C / Weff
  *sk = j < pages ? l : l + 1;
  *sp = j < pages ? (int)j : 0;
}

__global__ __launch_bounds__(kThreads) void plan_kernel(const int32_t* __restrict__ seqlens, int batch, int s_q,
                                                         int heads, int causal, int W, int32_t* __restrict__ plan) {
  extern __shared__ __attribute__((aligned(16))) uint32_t sm[];
  uint32_t* keys_a = sm;
  uint32_t* keys_b = sm + kMaxItems;
  int* wave_cnt = reinterpret_cast<int*>(keys_b + kMaxItems);   // [kWaves][256]
  int* digit_base = wave_cnt + kWaves * 256;                    // [256]
  int* tile_tot = digit_base + 256;                             // [256]
  int* scratch = tile_tot + 256;                                // [kWaves]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nthreads = blockDim.x;
  const int tiles = tiles_per_seq(s_q, heads);
  const int n = batch * tiles;

  // keys: (0xFFFF - pages) in the high half sorts longest first; the item index in the
  // low half is already ascending, and the LSD passes are stable.
  // (all page counts equal -- e.g. one length for the whole batch -- means the item order
  // is already sorted)
  int first_pages;
  {
    int sq0, tl0, vis0;
    item_shape(seqlens, 0, tiles, s_q, heads, causal, &sq0, &tl0, &vis0, &first_pages);
  }
  // Batches of at most one item per thread keep each item's visible length in the upper
  // half of keys_b (free in both of their paths), so the items pass reads no seqlens again.
  const bool one_each = n <= nthreads;
  int* vis_of = reinterpret_cast<int*>(keys_b + kMaxItems / 2);
  bool same = true;
  for (int i = tid; i < n; i += nthreads) {
    int sq, tl, vis, pages;
    item_shape(seqlens, i, tiles, s_q, heads, causal, &sq, &tl, &vis, &pages);
    keys_a[i] = ((uint32_t)(0xFFFF - pages) << 16) | (uint32_t)i;
    if (one_each) vis_of[i] = vis;
    same = same && pages == first_pages;
  }
  const bool uniform = __syncthreads_and(same);

  uint32_t* src = keys_a;
  uint32_t* dst = keys_b;
  if (uniform) {
    // nothing to sort
  } else if (n <= nthreads) {
    // Small batches: the packed keys are unique, so each item's position is the number of
    // smaller keys (a rank sort; same order as the radix sort below).
    const int n4 = (n + 3) & ~3;
    if (tid >= n && tid < n4) keys_a[tid] = 0xFFFFFFFFu;   // pads compare greater than every key
    __syncthreads();
    const uint32_t mine = tid < n ? keys_a[tid] : 0u;
    int rank = 0;
    for (int j = 0; j < n4; j += 4) {
      const uint4 v = *reinterpret_cast<const uint4*>(keys_a + j);
      rank += (v.x < mine) + (v.y < mine) + (v.z < mine) + (v.w < mine);
    }
    if (tid < n) keys_b[rank] = mine;
    __syncthreads();
    src = keys_b;
    dst = keys_a;
  } else {
    // Two stable LSD passes over the 16-bit page key (8-bit digits). Within a tile of 1024
    // items, the rank among equal digits comes from wave ballots; waves and tiles are
    // ordered through per-digit counters.
    for (int shift = 16; shift < 32; shift += 8) {
      if (tid < 256) digit_base[tid] = 0;
      for (int i = tid; i < kWaves * 256; i += nthreads) wave_cnt[i] = 0;
      __syncthreads();
      for (int i = tid; i < n; i += nthreads) atomicAdd(&digit_base[(src[i] >> shift) & 255], 1);
      __syncthreads();
      {
        int tot_unused = 0;
        const int cnt = tid < 256 ? digit_base[tid] : 0;
        const int excl = block_exclusive_scan(cnt, scratch, &tot_unused);
        if (tid < 256) digit_base[tid] = excl;
        __syncthreads();
      }
      for (int t0 = 0; t0 < n; t0 += nthreads) {
        const int i = t0 + tid;
        const bool valid = i < n;
        const uint32_t v = valid ? src[i] : 0u;
        const int d = (int)((v >> shift) & 255);
        uint64_t peers = __ballot(valid);
#pragma unroll
        for (int b = 0; b < 8; ++b) {
          const uint64_t bb = __ballot((d >> b) & 1);
          peers &= ((d >> b) & 1) ? bb : ~bb;
        }
        const int rank = __popcll(peers & ((1ull << lane) - 1ull));
        if (valid && rank == 0) wave_cnt[wave * 256 + d] = __popcll(peers);
        __syncthreads();
        if (tid < 256) {
          int run = 0;
          for (int w = 0; w < (nthreads >> 6); ++w) {
            const int c = wave_cnt[w * 256 + tid];
            wave_cnt[w * 256 + tid] = run;
            run += c;
          }
          tile_tot[tid] = run;
        }
        __syncthreads();
        if (valid) dst[digit_base[d] + wave_cnt[wave * 256 + d] + rank] = v;
        __syncthreads();
        if (tid < 256) {
          digit_base[tid] += tile_tot[tid];
          for (int w = 0; w < (nthreads >> 6); ++w) wave_cnt[w * 256 + tid] = 0;
        }
        __syncthreads();
      }
      uint32_t* tmp = src; src = dst; dst = tmp;
    }
  }
  // src holds the sorted keys; dst becomes the cost prefix C_k.
  int* cost = reinterpret_cast<int*>(dst);
  const int per = (n + nthreads - 1) / nthreads;
  const int lo = tid * per;
  const int hi = lo + per < n ? lo + per : n;
  int local = 0;
  for (int k = lo; k < hi; ++k) local += kPlanOverhead + (0xFFFF - (int)(src[k] >> 16));
  int total = 0;
  int run = block_exclusive_scan(local, scratch, &total);
  for (int k = lo; k < hi; ++k) {
    cost[k] = run;
    run += kPlanOverhead + (0xFFFF - (int)(src[k] >> 16));
  }
  __syncthreads();
  const int64_t C = total;
  // fewer workers than cost units / (1 + overhead / 2): every worker interval is at least
  // as long as one page of an item of two or more pages
  const int64_t Wcap = (2 * C) / (2 + kPlanOverhead);
  const int64_t Weff = (int64_t)W < Wcap ? (int64_t)W : Wcap;

  // owners, splits; slots and split-list positions by one packed scan
  int local_pack = 0;
  int first1 = 0, ns1 = 0;   // the thread's item when it holds one (one_each)
  for (int k = lo; k < hi; ++k) {
    const int pages = 0xFFFF - (int)(src[k] >> 16);
    const int first = page_worker(cost[k], pages, 0, C, Weff);
    const int last = page_worker(cost[k], pages, pages - 1, C, Weff);
    const int ns = last - first + 1;
    local_pack += ns > 1 ? ((ns << 16) | 1) : 0;
    first1 = first;
    ns1 = ns;
  }
  // Worker starts, each found once: entry w of `bound` (in the free tail of the cost array)
  // is worker w's first (item, page) packed as item << 16 | page, read by workers w - 1 and w.
  int* bound = cost + n;
  const bool shared_bounds = n + W + 1 <= kMaxItems;
  if (shared_bounds) {
    for (int w = tid; w <= W; w += nthreads) {
      int sk, sp;
      worker_start(w, n, Weff, C, cost, src, &sk, &sp);
      bound[w] = (sk << 16) | sp;
    }
  }
  int pack_total = 0;
  int pack_run = block_exclusive_scan(local_pack, scratch, &pack_total);
  int32_t* items = plan + plan_items_off();
  int32_t* split_list = plan + plan_split_off(n, W);
  for (int k = lo; k < hi; ++k) {
    const uint32_t key = src[k];
    const int idx = (int)(key & 0xFFFF);
    int sq, tl, vis, pages, first, ns;
    if (one_each) {
      sq = idx / tiles;
      tl = idx - sq * tiles;
      vis = vis_of[idx];
      pages = 0xFFFF - (int)(key >> 16);
      first = first1;
      ns = ns1;
    } else {
      item_shape(seqlens, idx, tiles, s_q, heads, causal, &sq, &tl, &vis, &pages);
      first = page_worker(cost[k], pages, 0, C, Weff);
      ns = page_worker(cost[k], pages, pages - 1, C, Weff) - first + 1;
    }
    int32_t* it = items + kItemWords * k;
    it[kISeq] = sq;
    it[kITile] = tl;
    it[kIVis] = vis;
    it[kIPages] = pages;
    it[kICost] = cost[k];
    it[kIOwner] = first;
    it[kINsplits] = ns;
    it[kISlot] = ns > 1 ? (pack_run >> 16) : -1;
    if (ns > 1) {
      int32_t* sr = split_list + kSplitWords * (pack_run & 0xFFFF);
      sr[kSSeq] = sq;
      sr[kSTile] = tl;
      sr[kSNsplits] = ns;
      sr[kSSlot] = pack_run >> 16;
    }
    pack_run += ns > 1 ? ((ns << 16) | 1) : 0;
  }
  // workers: start(w) = the first page whose start position is >= w C / Weff
  int32_t* workers = plan + plan_workers_off(n);
  if (shared_bounds) __syncthreads();
  for (int w = tid; w < W; w += nthreads) {
    int sk[2], sp[2];
    if (shared_bounds) {
      const int b0 = bound[w], b1 = bound[w + 1];
      sk[0] = b0 >> 16; sp[0] = b0 & 0xFFFF;
      sk[1] = b1 >> 16; sp[1] = b1 & 0xFFFF;
    } else {
      worker_start(w, n, Weff, C, cost, src, &sk[0], &sp[0]);
      worker_start(w + 1, n, Weff, C, cost, src, &sk[1], &sp[1]);
    }
    int32_t* wr = workers + kWorkerWords * w;
    wr[0] = sk[0]; wr[1] = sp[0]; wr[2] = sk[1]; wr[3] = sp[1];
  }
  if (tid == 0) {
    plan[kHMagic] = kPlanMagic;
    plan[kHVersion] = kPlanVersion;
    plan[kHBatch] = batch;
    plan[kHSq] = s_q;
    plan[kHHeads] = heads;
    plan[kHCausal] = causal;
    plan[kHWorkers] = W;
    plan[kHTiles] = tiles;
    plan[kHItems] = n;
    plan[kHOverhead] = kPlanOverhead;
    plan[kHTotalCost] = total;
    plan[kHActiveWorkers] = (int)Weff;
    plan[kHSplitItems] = pack_total & 0xFFFF;
    plan[kHSlots] = pack_total >> 16;
    plan[kHReserved0] = 0;
    plan[kHReserved1] = 0;
  }
}

constexpr size_t kPlanLds = (size_t)2 * kMaxItems * 4 + (size_t)(kWaves * 256 + 256 + 256 + kWaves) * 4;

}  // namespace

hipError_t launch_plan(const int32_t* seqlens, int batch, int s_q, int heads, int causal, int workers,
                       int32_t* plan, hipStream_t stream) {
  static_assert(kPlanLds <= 160 * 1024, "plan LDS");
  static thread_local int configured = -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)plan_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)kPlanLds);
    if (e != hipSuccess) return e;
    configured = dev;
  }
  const int n_items = batch * tiles_per_seq(s_q, heads);
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(n_items <= kThreadsSmall ? kThreadsSmall : kThreads), kPlanLds, stream,
                     seqlens, batch, s_q, heads, causal,
                     workers, plan);
  return hipGetLastError();
}

}  // namespace mla
