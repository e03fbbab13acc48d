// Internal constants and device-plan layout shared by the libmla host code and kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mla {

constexpr int kPage = 64;          // tokens per cache page
constexpr int kLat = 512;          // latent (c_KV) channels, the value width
constexpr int kRope = 64;          // shared rope key channels
constexpr int kDqk = kLat + kRope; // 576: absorbed query / cached row width
constexpr int kNope = 128;         // per-head query channels before absorption
constexpr int kDv = 128;           // per-head value channels after decompression
constexpr int kRowsPerTile = 128;  // query rows (token, head) per work item

// Planner limits.
constexpr int kMaxItems = 16384;
constexpr int kMaxWorkers = 4096;
constexpr int kMaxPagesPerSeq = 65535;
// Per-item cost in page units (queries in, rows out, and for a split item its partial rows and
// their merge). Swept on the jagged mix of 96 short and 32 long sequences (b=128, h=128):
// 1 -> 880 us, 2 -> 846, 3 -> 822, 4 -> 788, 6 -> 766, 8 -> 768, 12 -> 771, 24 -> 780 per
// decode call; batches of equal lengths cut the same way at any value.
constexpr int kPlanOverhead = 6;

// Plan buffer (int32 words).
constexpr int kPlanMagic = 0x4D4C4150;  // 'MLAP'
enum PlanHeader {
  kHMagic = 0, kHVersion, kHBatch, kHSq, kHHeads, kHCausal, kHWorkers, kHTiles, kHItems,
  kHOverhead, kHTotalCost, kHActiveWorkers, kHSplitItems, kHSlots, kHReserved0, kHReserved1,
  kHeaderWords = 16
};
// item record (sorted order): seq, tile, vis, pages, cost_begin, owner, nsplits, slot_base
constexpr int kItemWords = 8;
enum ItemField { kISeq = 0, kITile, kIVis, kIPages, kICost, kIOwner, kINsplits, kISlot };
// worker record: item_begin, page_begin, item_end, page_end (end exclusive)
constexpr int kWorkerWords = 4;
// split record (one per split item, in sorted order): seq, tile, nsplits, slot_base
constexpr int kSplitWords = 4;
enum SplitField { kSSeq = 0, kSTile, kSNsplits, kSSlot };
constexpr int kPlanVersion = 2;

__host__ __device__ inline int plan_items_off() { return kHeaderWords; }
__host__ __device__ inline int plan_workers_off(int n_items) { return kHeaderWords + kItemWords * n_items; }
__host__ __device__ inline int plan_split_off(int n_items, int workers) {
  return plan_workers_off(n_items) + kWorkerWords * workers;
}
__host__ __device__ inline int64_t plan_words(int n_items, int workers) {
  return (int64_t)plan_split_off(n_items, workers) + (int64_t)kSplitWords * n_items;
}

// Device-side precondition violations, OR-ed into the caller's status word (libmla.h).
enum DeviceStatus {
  kDevPlanMismatch = 1,      // the plan header does not match the call
  kDevPageOutOfRange = 2,    // a needed block-table entry is outside [0, num_pages)
  kDevLengthOverCap = 4,     // a length above max_pages * 64
};
__host__ __device__ inline int tiles_per_seq(int s_q, int heads) {
  return (s_q * heads + kRowsPerTile - 1) / kRowsPerTile;
}

// Workspace: per partial slot (one split part of a 128-row item), the unnormalised partial out
// as bf16 in the value MFMAs' register order (128 x 512 values, see the decode kernel's
// finalize), then two fp32 per row: its reference max (log2 units) and its softmax
// denominator.
constexpr int64_t kSlotPartBytes = (int64_t)kRowsPerTile * kLat * 2;
constexpr int64_t kSlotBytes = kSlotPartBytes + (int64_t)kRowsPerTile * 8;

hipError_t launch_plan(const int32_t* seqlens, int batch, int s_q, int heads, int causal, int workers,
                       int32_t* plan, hipStream_t stream);

struct DecodeArgs {
  const void* q;
  const void* kv;
  const float* kv_scales;
  int64_t num_pages;
  const int32_t* block_table;
  int max_pages;
  const int32_t* seqlens;
  int batch, s_q, heads, causal;
  float scale_log2;   // softmax_scale * log2(e)
  const int32_t* plan;
  int workers;
  float* ws;          // partial slots
  float* out;
  float* lse;
  int32_t* status;    // device status word (may be null)
};

hipError_t launch_decode_rows32(const DecodeArgs& a, bool fp8, hipStream_t stream);
hipError_t launch_decode_sparse_fp8(const DecodeArgs& a, const int32_t* rows, int row_stride, hipStream_t stream);
hipError_t launch_sparse_rows(const int32_t* indices, int topk, const int32_t* block_table, int max_pages,
                              const int32_t* seqlens, int batch, int s_q, int64_t num_pages, int32_t* rows,
                              int stride, int32_t* vis, int32_t* status, hipStream_t stream);
// token-sparse decode: row lists [batch * s_q, stride] (stride = topk rounded up to 32), then
// the visible counts [batch * s_q]
inline int sparse_stride(int topk) { return (topk + 31) / 32 * 32; }
constexpr int kSparseHeads = 128;   // one 128-row tile per query token
constexpr int kSparseMaxTopk = 1 << 20;
hipError_t launch_combine_rows32(const DecodeArgs& a, hipStream_t stream);
struct HybridArgs {
  const void *q_nope, *q_rope, *k_new, *kr_new, *v_new;
  const float *out_old, *lse_old;
  float *out, *lse;
  int batch, s_q, heads, n_new, causal;
  float scale_log2;   // softmax_scale * log2(e)
};
hipError_t launch_hybrid_merge(const HybridArgs& a, hipStream_t stream);
hipError_t launch_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int tokens, int heads,
                               void* qz, hipStream_t stream);
hipError_t launch_decompress_output(const float* out_latent, const void* w_v, int tokens, int heads, float* out,
                                    hipStream_t stream);

}  // namespace mla
