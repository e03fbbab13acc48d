// libmla C ABI: host-side validation, sizing and dispatch. Every check here happens before
// any work is enqueued; the library allocates nothing and keeps no pointer across calls.
#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "libmla.h"
#include "mla_internal.h"

// Library-owned device word (one copy per GPU, alive until the process ends): the status word
// of calls validated without a caller status word.
static __device__ int32_t g_validate_status;

// Split-partial scratch of mla_decode_fwd_noalloc: one copy per GPU, held until the process
// ends. Its device address is taken once per device (hipGetSymbolAddress, with that device
// current) and that address, never the symbol, is what host code passes to the kernels.
static __device__ __align__(256) char scratch[MLA_NOALLOC_SCRATCH_BYTES];

namespace {

__global__ void clear_word_kernel(int32_t* w) { *w = 0; }

thread_local char g_err[512] = "";

int32_t fail(int32_t status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int32_t ok() {
  g_err[0] = '\0';
  return MLA_OK;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Device address of `scratch` per device, taken at the first mla_decode_fwd_noalloc call on
// that device.
constexpr int kMaxDevices = 64;
void* g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;

hipError_t scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

bool env_flag(const char* name) {
  const char* e = std::getenv(name);
  return e != nullptr && e[0] != '\0' && std::strcmp(e, "0") != 0;
}

std::string describe_status(int32_t bits) {
  std::string m;
  auto add = [&](int32_t b, const char* what) {
    if (bits & b) m += std::string(m.empty() ? "" : "; ") + what;
  };
  add(mla::kDevPlanMismatch, "the plan was built for other arguments (batch, s_q, heads, causal or num_workers)");
  add(mla::kDevPageOutOfRange, "a block-table entry a sequence needs is outside [0, num_pages)");
  add(mla::kDevLengthOverCap, "a sequence length exceeds max_pages * 64");
  return m;
}

// MLA_VALIDATE=1: the device status word of the call (the caller's, or the library's own
// word cleared first) is read after a stream synchronisation, and any bit set turns the call
// into MLA_ERR_INVALID_ARG. Returns the status pointer the kernels should use.
int32_t* validate_begin(int32_t* status, hipStream_t stream, bool* on) {
  *on = false;
  if (!env_flag("MLA_VALIDATE")) return status;
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cs) != hipSuccess || cs != hipStreamCaptureStatusNone) return status;
  *on = true;
  if (status != nullptr) return status;
  int32_t* w = nullptr;
  if (hipGetSymbolAddress(reinterpret_cast<void**>(&w), HIP_SYMBOL(g_validate_status)) != hipSuccess) {
    *on = false;
    return nullptr;
  }
  hipLaunchKernelGGL(clear_word_kernel, dim3(1), dim3(1), 0, stream, w);
  return w;
}

int32_t validate_end(int32_t* word, hipStream_t stream, const char* call) {
  int32_t bits = 0;
  hipError_t e = hipStreamSynchronize(stream);
  if (e == hipSuccess) e = hipMemcpy(&bits, word, sizeof(bits), hipMemcpyDeviceToHost);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "%s: validation read-back: %s", call, hipGetErrorString(e));
  if (bits != 0)
    return fail(MLA_ERR_INVALID_ARG, "%s: device-side check failed (status 0x%x): %s", call, (unsigned)bits,
                describe_status(bits).c_str());
  return ok();
}

// Shape checks shared by the plan and the decode call.
int32_t check_shape(int32_t batch, int32_t s_q, int32_t heads, int32_t causal, int32_t num_workers) {
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (s_q < 1) return fail(MLA_ERR_INVALID_ARG, "s_q must be >= 1 (got %d)", s_q);
  if (heads < 1) return fail(MLA_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", heads);
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (num_workers < 1) return fail(MLA_ERR_INVALID_ARG, "num_workers must be >= 1 (got %d)", num_workers);
  if (s_q > 64) return fail(MLA_ERR_UNSUPPORTED, "s_q must be <= 64 (got %d)", s_q);
  if (heads != 16 && heads != 32 && heads != 64 && heads != 128)
    return fail(MLA_ERR_UNSUPPORTED, "heads must be 16, 32, 64 or 128 (got %d)", heads);
  if (batch > mla::kMaxItems) return fail(MLA_ERR_UNSUPPORTED, "batch must be <= %d (got %d)", mla::kMaxItems, batch);
  const int64_t items = (int64_t)batch * mla::tiles_per_seq(s_q, heads);
  if (items > mla::kMaxItems)
    return fail(MLA_ERR_UNSUPPORTED, "batch * ceil(s_q*heads/128) must be <= %d (got %lld)", mla::kMaxItems,
                (long long)items);
  if (num_workers > mla::kMaxWorkers)
    return fail(MLA_ERR_UNSUPPORTED, "num_workers must be <= %d (got %d)", mla::kMaxWorkers, num_workers);
  return MLA_OK;
}

size_t plan_bytes_of(int32_t batch, int32_t s_q, int32_t heads, int32_t workers) {
  const int n = batch * mla::tiles_per_seq(s_q, heads);
  return (size_t)mla::plan_words(n, workers) * 4;
}

size_t workspace_bytes_of(int32_t batch, int32_t s_q, int32_t heads, int32_t workers) {
  const int64_t n = (int64_t)batch * mla::tiles_per_seq(s_q, heads);
  // split slots <= 2 * (active workers - 1); a split item needs >= 2 workers
  int64_t slots = 2 * ((int64_t)workers - 1);
  if (slots > 2 * n * workers) slots = 2 * n * workers;
  if (slots < 0) slots = 0;
  return (size_t)slots * (size_t)mla::kSlotBytes;
}

// Host checks of a decode call beyond its shape; `need` is the workspace the shape requires.
int32_t check_decode_args(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                          int64_t num_pages, const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                          float softmax_scale, const void* plan, const void* workspace, size_t workspace_bytes,
                          const float* out, const float* lse, const int32_t* status, size_t need) {
  if (!q || !kv_cache || !block_table || !seqlens || !plan || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (q, kv_cache, block_table, seqlens, plan, out, lse)");
  if (kv_dtype != MLA_KV_BF16 && kv_dtype != MLA_KV_FP8_E4M3)
    return fail(MLA_ERR_INVALID_ARG, "kv_dtype must be MLA_KV_BF16 or MLA_KV_FP8_E4M3 (got %d)", kv_dtype);
  if (kv_dtype == MLA_KV_FP8_E4M3 && !kv_scales)
    return fail(MLA_ERR_INVALID_ARG, "kv_scales is required for an fp8 cache");
  if (kv_dtype == MLA_KV_BF16 && kv_scales)
    return fail(MLA_ERR_INVALID_ARG, "kv_scales must be NULL for a bf16 cache");
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %lld)", (long long)num_pages);
  if (max_pages < 1 || max_pages > mla::kMaxPagesPerSeq)
    return fail(max_pages < 1 ? MLA_ERR_INVALID_ARG : MLA_ERR_UNSUPPORTED, "max_pages must be in 1..%d (got %d)",
                mla::kMaxPagesPerSeq, max_pages);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(out) || !aligned16(plan) ||
      (kv_scales && !aligned16(kv_scales)) || (workspace && !aligned16(workspace)))
    return fail(MLA_ERR_INVALID_ARG, "q, kv_cache, kv_scales, out, plan and workspace must be 16-byte aligned");
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace ? workspace_bytes : 0,
                need);
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "status must be 4-byte aligned");
  return MLA_OK;
}

// Enqueue the decode kernel and the split combine of a checked call (workspace: the split
// partials' device memory, caller-owned or the library's scratch).
int32_t decode_launch(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype, int64_t num_pages,
                      const int32_t* block_table, int32_t max_pages, const int32_t* seqlens, int32_t batch,
                      int32_t s_q, int32_t heads, float softmax_scale, int32_t causal, const void* plan,
                      int32_t num_workers, void* workspace, float* out, float* lse, int32_t* status, void* stream,
                      const char* call) {
  mla::DecodeArgs a;
  a.q = q;
  a.kv = kv_cache;
  a.kv_scales = kv_scales;
  a.num_pages = num_pages;
  a.block_table = block_table;
  a.max_pages = max_pages;
  a.seqlens = seqlens;
  a.batch = batch;
  a.s_q = s_q;
  a.heads = heads;
  a.causal = causal;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.plan = static_cast<const int32_t*>(plan);
  a.workers = num_workers;
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  bool validating = false;
  a.status = validate_begin(status, s, &validating);
  hipError_t e = mla::launch_decode_rows32(a, kv_dtype == MLA_KV_FP8_E4M3, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
  e = mla::launch_combine_rows32(a, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  if (validating) return validate_end(a.status, s, call);
  return ok();
}

}  // namespace

extern "C" {

int32_t mla_abi_version(void) { return MLA_ABI_VERSION; }

const char* mla_status_string(int32_t s) {
  switch (s) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_INVALID_ARG: return "MLA_ERR_INVALID_ARG";
    case MLA_ERR_UNSUPPORTED: return "MLA_ERR_UNSUPPORTED";
    case MLA_ERR_WORKSPACE_TOO_SMALL: return "MLA_ERR_WORKSPACE_TOO_SMALL";
    case MLA_ERR_HIP: return "MLA_ERR_HIP";
    case MLA_ERR_INTERNAL: return "MLA_ERR_INTERNAL";
    default: return "unknown status";
  }
}

const char* mla_last_error_message(void) { return g_err; }

int32_t mla_default_num_workers(int32_t device) {
  int count = 0;
  hipError_t e = hipDeviceGetAttribute(&count, hipDeviceAttributeMultiprocessorCount, device);
  if (e != hipSuccess) {
    fail(MLA_ERR_HIP, "hipDeviceGetAttribute(MultiprocessorCount, %d): %s", device, hipGetErrorString(e));
    return -1;
  }
  ok();
  return count;
}

size_t mla_plan_bytes(int32_t batch, int32_t s_q, int32_t heads, int32_t num_workers) {
  if (check_shape(batch, s_q, heads, 0, num_workers) != MLA_OK) return 0;
  return plan_bytes_of(batch, s_q, heads, num_workers);
}

size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t heads, int32_t num_workers) {
  if (check_shape(batch, s_q, heads, 0, num_workers) != MLA_OK) return 0;
  return workspace_bytes_of(batch, s_q, heads, num_workers);
}

int32_t mla_get_split_plan(const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads, int32_t causal,
                           int32_t num_workers, void* plan, size_t plan_bytes, void* stream) {
  int32_t st = check_shape(batch, s_q, heads, causal, num_workers);
  if (st != MLA_OK) return st;
  if (!seqlens) return fail(MLA_ERR_INVALID_ARG, "seqlens is NULL");
  if (!plan) return fail(MLA_ERR_INVALID_ARG, "plan is NULL");
  if (!aligned16(plan)) return fail(MLA_ERR_INVALID_ARG, "plan must be 16-byte aligned");
  const size_t need = plan_bytes_of(batch, s_q, heads, num_workers);
  if (plan_bytes < need)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "plan_bytes %zu < required %zu", plan_bytes, need);
  hipError_t e = mla::launch_plan(seqlens, batch, s_q, heads, causal, num_workers, static_cast<int32_t*>(plan),
                                  static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t mla_decode_fwd(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                       int64_t num_pages, const int32_t* block_table, int32_t max_pages, const int32_t* seqlens,
                       int32_t batch, int32_t s_q, int32_t heads, float softmax_scale, int32_t causal,
                       const void* plan, int32_t num_workers, void* workspace, size_t workspace_bytes, float* out,
                       float* lse, int32_t* status, void* stream) {
  int32_t st = check_shape(batch, s_q, heads, causal, num_workers);
  if (st != MLA_OK) return st;
  st = check_decode_args(q, kv_cache, kv_scales, kv_dtype, num_pages, block_table, max_pages, seqlens, softmax_scale,
                         plan, workspace, workspace_bytes, out, lse, status,
                         workspace_bytes_of(batch, s_q, heads, num_workers));
  if (st != MLA_OK) return st;
  return decode_launch(q, kv_cache, kv_scales, kv_dtype, num_pages, block_table, max_pages, seqlens, batch, s_q,
                       heads, softmax_scale, causal, plan, num_workers, workspace, out, lse, status, stream,
                       "mla_decode_fwd");
}

int32_t mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                               int64_t num_pages, const int32_t* block_table, int32_t max_pages,
                               const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads,
                               float softmax_scale, int32_t causal, const void* plan, int32_t num_workers,
                               float* out, float* lse, int32_t* status, void* stream) {
  int32_t st = check_shape(batch, s_q, heads, causal, num_workers);
  if (st != MLA_OK) return st;
  const size_t need = workspace_bytes_of(batch, s_q, heads, num_workers);
  if (need > (size_t)MLA_NOALLOC_SCRATCH_BYTES)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL,
                "mla_decode_fwd_noalloc: this shape needs %zu bytes of split scratch, more than the library's "
                "%zu (use fewer workers, or mla_decode_fwd with a workspace)",
                need, (size_t)MLA_NOALLOC_SCRATCH_BYTES);
  // every argument check of mla_decode_fwd before the scratch address is taken (a stand-in
  // workspace pointer; nothing is launched when a check fails)
  void* ws = need > 0 ? reinterpret_cast<void*>(static_cast<uintptr_t>(256)) : nullptr;
  st = check_decode_args(q, kv_cache, kv_scales, kv_dtype, num_pages, block_table, max_pages, seqlens, softmax_scale,
                         plan, ws, need, out, lse, status, need);
  if (st != MLA_OK) return st;
  if (need > 0) {
    hipError_t e = scratch_ptr(&ws);
    if (e != hipSuccess) return fail(MLA_ERR_HIP, "scratch address: %s", hipGetErrorString(e));
  }
  return decode_launch(q, kv_cache, kv_scales, kv_dtype, num_pages, block_table, max_pages, seqlens, batch, s_q,
                       heads, softmax_scale, causal, plan, num_workers, ws, out, lse, status, stream,
                       "mla_decode_fwd_noalloc");
}

int32_t mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int32_t tokens, int32_t heads,
                         void* qz, void* stream) {
  if (!q_nope || !q_rope || !w_k || !qz)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (q_nope, q_rope, w_k, qz)");
  if (tokens < 1) return fail(MLA_ERR_INVALID_ARG, "tokens must be >= 1 (got %d)", tokens);
  if (heads < 1) return fail(MLA_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", heads);
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "heads must be <= 65535 (got %d)", heads);
  if ((int64_t)tokens > 32LL * 65535) return fail(MLA_ERR_UNSUPPORTED, "tokens must be <= %d", 32 * 65535);
  if ((int64_t)tokens * heads * mla::kNope * 2 > 0xFFFFFFFFLL)
    return fail(MLA_ERR_UNSUPPORTED, "tokens * heads must be below 2^24 (got %lld)", (long long)tokens * heads);
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(w_k) || !aligned16(qz))
    return fail(MLA_ERR_INVALID_ARG, "q_nope, q_rope, w_k and qz must be 16-byte aligned");
  hipError_t e = mla::launch_absorb_query(q_nope, q_rope, w_k, tokens, heads, qz, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "absorption kernel launch: %s", hipGetErrorString(e));
  return ok();
}

int32_t mla_decompress_output(const float* out_latent, const void* w_v, int32_t tokens, int32_t heads, float* out,
                              void* stream) {
  if (!out_latent || !w_v || !out)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (out_latent, w_v, out)");
  if (tokens < 1) return fail(MLA_ERR_INVALID_ARG, "tokens must be >= 1 (got %d)", tokens);
  if (heads < 1) return fail(MLA_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", heads);
  if (heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "heads must be <= 65535 (got %d)", heads);
  if ((int64_t)tokens > 32LL * 65535) return fail(MLA_ERR_UNSUPPORTED, "tokens must be <= %d", 32 * 65535);
  if ((int64_t)tokens * heads * mla::kLat * 4 > 0xFFFFFFFFLL)
    return fail(MLA_ERR_UNSUPPORTED, "tokens * heads must be below 2^21 (got %lld)", (long long)tokens * heads);
  if (!aligned16(out_latent) || !aligned16(w_v) || !aligned16(out))
    return fail(MLA_ERR_INVALID_ARG, "out_latent, w_v and out must be 16-byte aligned");
  hipError_t e = mla::launch_decompress_output(out_latent, w_v, tokens, heads, out, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decompression kernel launch: %s", hipGetErrorString(e));
  return ok();
}

size_t mla_sparse_rows_bytes(int32_t batch, int32_t s_q, int32_t topk) {
  if (batch < 1 || s_q < 1 || topk < 1 || topk > mla::kSparseMaxTopk || (int64_t)batch * s_q > mla::kMaxItems)
    return 0;
  const int64_t n = (int64_t)batch * s_q;
  return (size_t)((n * mla::sparse_stride(topk) + n) * 4 + 15) / 16 * 16;
}

// Shape checks of the token-sparse calls; the plan and decode shapes are those of batch * s_q
// sequences of one query token.
static int32_t check_sparse(int32_t batch, int32_t s_q, int32_t heads, int32_t topk, int64_t num_pages,
                            int32_t num_workers) {
  if (batch < 1 || s_q < 1) return fail(MLA_ERR_INVALID_ARG, "batch and s_q must be >= 1 (got %d, %d)", batch, s_q);
  if (topk < 1) return fail(MLA_ERR_INVALID_ARG, "topk must be >= 1 (got %d)", topk);
  if (num_pages < 1) return fail(MLA_ERR_INVALID_ARG, "num_pages must be >= 1 (got %lld)", (long long)num_pages);
  if (heads != mla::kSparseHeads)
    return fail(MLA_ERR_UNSUPPORTED, "the token-sparse decode needs heads = %d (got %d)", mla::kSparseHeads, heads);
  if (topk > mla::kSparseMaxTopk) return fail(MLA_ERR_UNSUPPORTED, "topk must be <= %d", mla::kSparseMaxTopk);
  if (s_q > 64) return fail(MLA_ERR_UNSUPPORTED, "s_q must be <= 64 (got %d)", s_q);
  if (num_pages * mla::kPage * (mla::kLat + 2 * mla::kRope) >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "the token-sparse decode addresses the cache with 31-bit offsets: num_pages "
                "must be below %lld", (long long)((1LL << 31) / (mla::kPage * (mla::kLat + 2 * mla::kRope))));
  return check_shape((int32_t)std::min<int64_t>((int64_t)batch * s_q, 1LL << 30), 1, heads, 0, num_workers);
}

int32_t mla_get_sparse_plan(const int32_t* indices, int32_t topk, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads, int64_t num_pages,
                            int32_t num_workers, void* rows, size_t rows_bytes, void* plan, size_t plan_bytes,
                            int32_t* status, void* stream) {
  int32_t st = check_sparse(batch, s_q, heads, topk, num_pages, num_workers);
  if (st != MLA_OK) return st;
  if (!indices || !block_table || !seqlens || !rows || !plan)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (indices, block_table, seqlens, rows, plan)");
  if (max_pages < 1 || max_pages > mla::kMaxPagesPerSeq)
    return fail(max_pages < 1 ? MLA_ERR_INVALID_ARG : MLA_ERR_UNSUPPORTED, "max_pages must be in 1..%d (got %d)",
                mla::kMaxPagesPerSeq, max_pages);
  if (!aligned16(rows) || !aligned16(plan)) return fail(MLA_ERR_INVALID_ARG, "rows and plan must be 16-byte aligned");
  const int32_t n = batch * s_q;
  const size_t need_rows = mla_sparse_rows_bytes(batch, s_q, topk);
  if (rows_bytes < need_rows)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "rows_bytes %zu < required %zu", rows_bytes, need_rows);
  const size_t need_plan = plan_bytes_of(n, 1, heads, num_workers);
  if (plan_bytes < need_plan)
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "plan_bytes %zu < required %zu", plan_bytes, need_plan);
  const int stride = mla::sparse_stride(topk);
  int32_t* rows32 = static_cast<int32_t*>(rows);
  int32_t* vis = rows32 + (int64_t)n * stride;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "status must be 4-byte aligned");
  bool validating = false;
  int32_t* sw = validate_begin(status, s, &validating);
  hipError_t e = mla::launch_sparse_rows(indices, topk, block_table, max_pages, seqlens, batch, s_q, num_pages,
                                         rows32, stride, vis, sw, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "row-list kernel launch: %s", hipGetErrorString(e));
  e = mla::launch_plan(vis, n, 1, heads, 0, num_workers, static_cast<int32_t*>(plan), s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "plan kernel launch: %s", hipGetErrorString(e));
  if (validating) return validate_end(sw, s, "mla_get_sparse_plan");
  return ok();
}

int32_t mla_sparse_decode_fwd(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                              int64_t num_pages, int32_t batch, int32_t s_q, int32_t heads, int32_t topk,
                              float softmax_scale, const void* rows, const void* plan, int32_t num_workers,
                              void* workspace, size_t workspace_bytes, float* out, float* lse, int32_t* status,
                              void* stream) {
  int32_t st = check_sparse(batch, s_q, heads, topk, num_pages, num_workers);
  if (st != MLA_OK) return st;
  if (!q || !kv_cache || !kv_scales || !rows || !plan || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (q, kv_cache, kv_scales, rows, plan, out, lse)");
  if (kv_dtype != MLA_KV_FP8_E4M3)
    return fail(kv_dtype == MLA_KV_BF16 ? MLA_ERR_UNSUPPORTED : MLA_ERR_INVALID_ARG,
                "the token-sparse decode reads an fp8 e4m3 cache (kv_dtype %d)", kv_dtype);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (!aligned16(q) || !aligned16(kv_cache) || !aligned16(kv_scales) || !aligned16(out) || !aligned16(plan) ||
      !aligned16(rows) || (workspace && !aligned16(workspace)))
    return fail(MLA_ERR_INVALID_ARG, "q, kv_cache, kv_scales, rows, out, plan and workspace must be 16-byte aligned");
  const int32_t n = batch * s_q;
  const size_t need = workspace_bytes_of(n, 1, heads, num_workers);
  if (need > 0 && (!workspace || workspace_bytes < need))
    return fail(MLA_ERR_WORKSPACE_TOO_SMALL, "workspace_bytes %zu < required %zu", workspace ? workspace_bytes : 0,
                need);
  const int stride = mla::sparse_stride(topk);
  mla::DecodeArgs a;
  a.q = q;
  a.kv = kv_cache;
  a.kv_scales = kv_scales;
  a.num_pages = num_pages;
  a.block_table = nullptr;
  a.max_pages = (stride + mla::kPage - 1) / mla::kPage;   // caps no list: vis <= topk <= stride
  a.seqlens = static_cast<const int32_t*>(rows) + (int64_t)n * stride;
  a.batch = n;
  a.s_q = 1;
  a.heads = heads;
  a.causal = 0;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.plan = static_cast<const int32_t*>(plan);
  a.workers = num_workers;
  a.ws = static_cast<float*>(workspace);
  a.out = out;
  a.lse = lse;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (status && (reinterpret_cast<uintptr_t>(status) & 3u))
    return fail(MLA_ERR_INVALID_ARG, "status must be 4-byte aligned");
  bool validating = false;
  a.status = validate_begin(status, s, &validating);
  hipError_t e = mla::launch_decode_sparse_fp8(a, static_cast<const int32_t*>(rows), stride, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "decode kernel launch: %s", hipGetErrorString(e));
  e = mla::launch_combine_rows32(a, s);
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "combine kernel launch: %s", hipGetErrorString(e));
  if (validating) return validate_end(a.status, s, "mla_sparse_decode_fwd");
  return ok();
}

int32_t mla_hybrid_merge(const void* q_nope, const void* q_rope, const void* k_new, const void* kr_new,
                         const void* v_new, int32_t n_new, const float* out_old, const float* lse_old, int32_t batch,
                         int32_t s_q, int32_t heads, float softmax_scale, int32_t causal, float* out, float* lse,
                         void* stream) {
  if (!q_nope || !q_rope || !out_old || !lse_old || !out || !lse)
    return fail(MLA_ERR_INVALID_ARG, "a required pointer is NULL (q_nope, q_rope, out_old, lse_old, out, lse)");
  if (n_new < 0) return fail(MLA_ERR_INVALID_ARG, "n_new must be >= 0 (got %d)", n_new);
  if (n_new > 0 && (!k_new || !kr_new || !v_new))
    return fail(MLA_ERR_INVALID_ARG, "k_new, kr_new and v_new are required when n_new > 0");
  if (batch < 1) return fail(MLA_ERR_INVALID_ARG, "batch must be >= 1 (got %d)", batch);
  if (s_q < 1) return fail(MLA_ERR_INVALID_ARG, "s_q must be >= 1 (got %d)", s_q);
  if (heads < 1) return fail(MLA_ERR_INVALID_ARG, "heads must be >= 1 (got %d)", heads);
  if (causal != 0 && causal != 1) return fail(MLA_ERR_INVALID_ARG, "causal must be 0 or 1 (got %d)", causal);
  if (!(softmax_scale > 0.f) || !std::isfinite(softmax_scale))
    return fail(MLA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  if (s_q > 32) return fail(MLA_ERR_UNSUPPORTED, "s_q must be <= 32 (got %d)", s_q);
  if (batch > 65535 || heads > 65535) return fail(MLA_ERR_UNSUPPORTED, "batch and heads must be <= 65535");
  if (n_new > (1 << 24)) return fail(MLA_ERR_UNSUPPORTED, "n_new must be <= 2^24 (got %d)", n_new);
  if ((int64_t)(n_new + 32) * heads * 256 >= (1LL << 31))
    return fail(MLA_ERR_UNSUPPORTED, "(n_new + 32) * heads * 256 must be below 2^31 (31-bit offsets into k_new, v_new)");
  if (causal && n_new < s_q)
    return fail(MLA_ERR_UNSUPPORTED, "causal needs n_new >= s_q (got n_new %d, s_q %d): the old tokens must all "
                "be visible", n_new, s_q);
  if (!aligned16(q_nope) || !aligned16(q_rope) || !aligned16(out_old) || !aligned16(out) ||
      (n_new > 0 && (!aligned16(k_new) || !aligned16(kr_new) || !aligned16(v_new))))
    return fail(MLA_ERR_INVALID_ARG, "q_nope, q_rope, k_new, kr_new, v_new, out_old and out must be 16-byte aligned");
  mla::HybridArgs a;
  a.q_nope = q_nope;
  a.q_rope = q_rope;
  a.k_new = k_new;
  a.kr_new = kr_new;
  a.v_new = v_new;
  a.out_old = out_old;
  a.lse_old = lse_old;
  a.out = out;
  a.lse = lse;
  a.batch = batch;
  a.s_q = s_q;
  a.heads = heads;
  a.n_new = n_new;
  a.causal = causal;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  hipError_t e = mla::launch_hybrid_merge(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(MLA_ERR_HIP, "hybrid merge kernel launch: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
