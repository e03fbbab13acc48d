/*
 * libmla -- latent-space Multi-head Latent Attention (MLA) decode for AMD Instinct
 * MI355X (gfx950). C ABI.
 *
 * What is computed. Page "Mla Analysis", section "Absorption Trick (FlashMLA)": the
 * score of a query against a decompressed key Z W_k equals the absorbed query
 * Qz = Q W_k^T against the latent row Z, and softmax(A)(Z W_v) = (softmax(A) Z) W_v,
 * so decode works on latent rows only and leaves the W_v decompression to a separate
 * kernel. For query row (sequence i, query token j, head e) with absorbed query
 * Qz[576] = [q_nope W_k^T (512) | q_rope (64)] and the sequence's cached latent rows
 * Z[u, 576] = [c_KV (512) | k_rope (64)] (section "Tensor Shapes": Z is [B, T, K],
 * KPE is [B, T, P]; here one 576-wide row), for the visible keys u:
 *
 *     a_u  = softmax_scale * sum_c Qz[c] * Z[u, c]
 *     lse  = log(sum_u exp(a_u))                       (natural log)
 *     out  = sum_u exp(a_u - lse) * Z[u, 0:512]        (normalised O_latent)
 *
 * Visible keys: all u < t_i; with causal != 0 and s_q > 1, query token j sees
 * u <= t_i - s_q + j (t_i counts the s_q new tokens, whose rows are already cached).
 * No visible key: out = 0, lse = -inf.
 *
 * Conventions shared by every call:
 *  - Every pointer argument named as device memory is caller-owned device memory.
 *    The library allocates nothing, keeps no pointer after a call returns, and
 *    enqueues all work on `stream` (a hipStream_t; NULL = the default stream). A call
 *    that returns MLA_OK has *enqueued* its work; device faults surface at the caller's
 *    next synchronisation. Buffers must stay valid until that work completes.
 *  - Every host-checkable error is returned before any work is enqueued, and then no
 *    output is written. mla_last_error_message() gives the reason (thread-local).
 *  - The cache is paged: 64 tokens per page. block_table[i, r] names the physical page
 *    holding tokens 64r .. 64r+63 of sequence i.
 *  - Device-resident preconditions the library cannot check on the host:
 *    0 <= seqlens[i] <= max_pages * 64 and block_table[i, r] in [0, num_pages) for
 *    r < ceil(seqlens[i] / 64), and a plan built for the call's arguments. The kernels never
 *    fault on a violation: a page id outside [0, num_pages) reads as zeros, a length above
 *    max_pages * 64 reads only max_pages pages, and a mismatched plan writes no output. Each
 *    violation sets a bit (MLA_DEVICE_*) in the call's optional device status word, and with
 *    the environment variable MLA_VALIDATE=1 the call synchronises its stream after the launch
 *    and returns MLA_ERR_INVALID_ARG naming the violations (not under stream capture).
 */
#ifndef LIBMLA_H
#define LIBMLA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MLA_ABI_VERSION 2

/* Status codes returned by every entry point that can fail. */
typedef enum {
  MLA_OK = 0,
  MLA_ERR_INVALID_ARG = 1,          /* null pointer, bad size, bad enum, misalignment */
  MLA_ERR_UNSUPPORTED = 2,          /* a shape outside the supported set (see each call) */
  MLA_ERR_WORKSPACE_TOO_SMALL = 3,  /* plan_bytes or workspace_bytes below the required size */
  MLA_ERR_HIP = 4,                  /* a HIP runtime call or kernel launch failed */
  MLA_ERR_INTERNAL = 5
} mla_status;

/* Bits of the device status word (int32, caller-owned device memory, OR-ed by the kernels and
 * never cleared by them: the caller zeroes it before the calls it wants to watch). */
#define MLA_DEVICE_PLAN_MISMATCH 1       /* plan built for other batch/s_q/heads/causal/num_workers */
#define MLA_DEVICE_PAGE_OUT_OF_RANGE 2   /* a needed block-table entry outside [0, num_pages) */
#define MLA_DEVICE_LENGTH_OVER_CAPACITY 4 /* a sequence length above max_pages * 64 */

/* Storage of the latent cache.
 * MLA_KV_BF16: kv_cache is bf16 [num_pages, 64, 576], a token row = 512 c_KV then 64 rope.
 * MLA_KV_FP8_E4M3: kv_cache is bytes [num_pages, 64, 640]; a token row = 512 OCP e4m3fn
 *   codes of c_KV then the 64 rope channels as bf16 (128 bytes); kv_scales is float32
 *   [num_pages, 64, 4] and c_KV[c] = e4m3fn(code[c]) * scale[token, c / 128]. (FlashMLA-2
 *   newsletter page, section "Architectural Analysis": an FP8 cache scaled up to bf16
 *   in registers before the matrix products.) */
typedef enum { MLA_KV_BF16 = 0, MLA_KV_FP8_E4M3 = 1 } mla_kv_dtype;

/* Returns MLA_ABI_VERSION of the built library. */
int32_t mla_abi_version(void);

/* Static string naming a status code ("MLA_OK", ...); "unknown status" otherwise. */
const char* mla_status_string(int32_t status);

/* Detail of the last error returned on the calling thread ("" if none). The pointer
 * stays valid until the next libmla call on this thread. */
const char* mla_last_error_message(void);

/* Number of compute units of HIP device `device` (256 on MI355X): the natural
 * num_workers for the calls below. Returns -1 (and sets the error message) if the
 * device cannot be queried. */
int32_t mla_default_num_workers(int32_t device);

/* Bytes of the plan buffer mla_get_split_plan writes for this shape, or 0 if the shape
 * is invalid or unsupported (see mla_get_split_plan). */
size_t mla_plan_bytes(int32_t batch, int32_t s_q, int32_t heads, int32_t num_workers);

/* Bytes of the workspace mla_decode_fwd needs for partial results of split sequences
 * (an upper bound over every length mix), or 0 if the shape is invalid. */
size_t mla_workspace_bytes(int32_t batch, int32_t s_q, int32_t heads, int32_t num_workers);

/* Split-KV plan for one decode step (FlashMLA-2 newsletter page, section "Architectural
 * Analysis": a radix-sorted scheduler that balances sequence partitions across compute
 * units so that short and very long sequences in one batch leave no stragglers).
 *
 * Work items are (sequence, 128-row tile of the s_q*heads query rows). Items are sorted
 * by page count, longest first (stable), laid end to end with a fixed per-item overhead
 * in page units spread evenly over the item's pages, and cut into at most num_workers
 * contiguous runs of equal cost (fewer for very small batches, so that no run inside a
 * split item is empty); an item cut across runs is "split" and its runs are merged by
 * log-sum-exp in mla_decode_fwd.
 * Runs entirely on the device (one work-group); no host synchronisation.
 *
 * seqlens   device int32 [batch]: cached tokens per sequence (incl. the s_q new ones).
 * batch     1 .. 16384; batch * ceil(s_q*heads/128) must be <= 16384.
 * s_q       query tokens per sequence, 1 .. 64.
 * heads     16, 32, 64 or 128.
 * causal    0 or 1 (see the header comment); affects the visible key counts.
 * num_workers  1 .. 4096; use mla_default_num_workers() for one run per compute unit.
 * plan      device buffer of at least mla_plan_bytes(batch, s_q, heads, num_workers)
 *           bytes, 16-byte aligned; written by the device. Opaque to the caller; valid
 *           for every mla_decode_fwd call with the same seqlens contents, batch, s_q,
 *           heads, causal and num_workers.
 * Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL (plan_bytes),
 * MLA_ERR_HIP. */
int32_t mla_get_split_plan(const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads,
                           int32_t causal, int32_t num_workers, void* plan, size_t plan_bytes,
                           void* stream);

/* Latent-space MLA decode (the formulas in the header comment).
 *
 * q           device bf16 [batch, s_q, heads, 576], contiguous: absorbed queries
 *             [q_nope W_k^T | q_rope] (rope rotation already applied).
 * kv_cache    device, layout per kv_dtype (see mla_kv_dtype), 16-byte aligned.
 * kv_scales   device float32 [num_pages, 64, 4] for MLA_KV_FP8_E4M3; must be NULL for bf16.
 * kv_dtype    MLA_KV_BF16 or MLA_KV_FP8_E4M3.
 * num_pages   pages in kv_cache (>= 1); page ids outside [0, num_pages) read as zeros.
 * block_table device int32 [batch, max_pages], row-major.
 * max_pages   1 .. 65535.
 * seqlens     device int32 [batch] (same contents as given to the plan).
 * batch, s_q, heads, causal   as for mla_get_split_plan (must match the plan).
 * softmax_scale  multiplies every score (e.g. 1/sqrt(192)); finite and > 0.
 * plan        device plan from mla_get_split_plan for the same arguments.
 * num_workers the num_workers given to mla_get_split_plan.
 * workspace   device buffer of at least mla_workspace_bytes(batch, s_q, heads,
 *             num_workers) bytes, 16-byte aligned, or NULL when that size is 0. Scratch:
 *             contents on entry are ignored, on return undefined.
 * out         device float32 [batch, s_q, heads, 512] (normalised O_latent), 16-byte aligned.
 * lse         device float32 [batch, s_q, heads] (natural-log log-sum-exp).
 * status      device int32 word or NULL: MLA_DEVICE_* bits of violated device-resident
 *             preconditions are OR-ed into it (see the header comment). 4-byte aligned.
 * Split sequences: the parts of a sequence cut across workers are merged by log-sum-exp in a
 * second kernel on the same stream.
 * Calls that overlap on the same workspace race. Results for a fixed plan are bitwise
 * reproducible.
 * Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP. */
int32_t mla_decode_fwd(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                       int64_t num_pages, const int32_t* block_table, int32_t max_pages,
                       const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads,
                       float softmax_scale, int32_t causal, const void* plan, int32_t num_workers,
                       void* workspace, size_t workspace_bytes, float* out, float* lse, int32_t* status,
                       void* stream);

/* mla_decode_fwd for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): the same computation, kernels and
 * arguments, with the split partials kept in a scratch array the library owns instead of a
 * caller workspace. The array, MLA_NOALLOC_SCRATCH_BYTES bytes, is a static device array: each
 * GPU the library runs on holds its own copy until the process ends, and its address is taken
 * once per device at the first call on it. The call allocates nothing (no hipMalloc, hipFree or
 * allocating library routine). Nothing in the scratch needs to start at zero: the decode
 * kernel writes every partial before the combine kernel reads it.
 * Every call on one GPU shares that GPU's scratch: calls that overlap on one GPU (other
 * streams, other threads) race. A shape whose workspace (mla_workspace_bytes) exceeds
 * MLA_NOALLOC_SCRATCH_BYTES -- more than 286 workers -- returns MLA_ERR_WORKSPACE_TOO_SMALL
 * before anything is enqueued. Arguments and errors otherwise as for mla_decode_fwd. */
#define MLA_NOALLOC_SCRATCH_BYTES (72u << 20)
int32_t mla_decode_fwd_noalloc(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                               int64_t num_pages, const int32_t* block_table, int32_t max_pages,
                               const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads,
                               float softmax_scale, int32_t causal, const void* plan, int32_t num_workers,
                               float* out, float* lse, int32_t* status, void* stream);

/* Query absorption (page "Mla Analysis", section "Absorption Trick (FlashMLA)": scoring the
 * absorbed query against a latent row equals scoring the query against the decompressed
 * key). Per token t and head h:
 *   qz[t, h, 0:512]   = q_nope[t, h, :] . W_k[h]^T   (fp32 accumulation, rounded to bf16)
 *   qz[t, h, 512:576] = q_rope[t, h, :]              (copied bit for bit)
 * The result is the `q` argument of mla_decode_fwd.
 *
 * q_nope  device bf16 [tokens, heads, 128] (tokens = batch * s_q, row-major).
 * q_rope  device bf16 [tokens, heads, 64] (rope rotation already applied).
 * w_k     device bf16 [heads, 512, 128]: for each head and latent channel its 128
 *         coefficients (the contraction index innermost).
 * qz      device bf16 [tokens, heads, 576].
 * All four 16-byte aligned and contiguous; tokens 1 .. 2,097,120, heads 1 .. 65535,
 * tokens * heads < 2^24.
 * Stream-ordered; allocates nothing. Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_HIP. */
int32_t mla_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int32_t tokens,
                         int32_t heads, void* qz, void* stream);

/* Output decompression (same page and section: softmax(A) (Z W_v) = (softmax(A) Z) W_v, so
 * the value projection is applied once to the latent output, by a separate kernel after
 * the attention). Per token t and head h:
 *   out[t, h, :] = out_latent[t, h, :] . W_v[h]^T
 * with out_latent rounded to bf16 on load and fp32 accumulation.
 *
 * out_latent  device float32 [tokens, heads, 512] (the `out` of mla_decode_fwd).
 * w_v         device bf16 [heads, 128, 512]: for each head and output channel its 512
 *             coefficients (the contraction index innermost; a linear layer's weight).
 * out         device float32 [tokens, heads, 128].
 * All three 16-byte aligned and contiguous; tokens 1 .. 2,097,120, heads 1 .. 65535,
 * tokens * heads < 2^21.
 * Stream-ordered; allocates nothing. Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_HIP. */
int32_t mla_decompress_output(const float* out_latent, const void* w_v, int32_t tokens, int32_t heads,
                              float* out, void* stream);

/* Token-level sparse decode (library card page "FlashMLA: Efficient Multi-head Latent Attention
 * Kernels": sparse attention over selected tokens in decoding, with an FP8 cache). Each query
 * token (sequence i, token j) attends to its own list indices[i, j, 0:topk] of logical token
 * positions of sequence i instead of all its cached tokens: an entry u with
 * 0 <= u < min(t_i, max_pages * 64) is a key (the latent row at block_table[i, u / 64], slot
 * u % 64; a listed position twice is two keys), any other entry is padding. The formulas of the
 * header comment apply with these keys as the visible set (no causal mask: the list is the
 * visible set); an empty list gives out = 0, lse = -inf. Two calls: mla_get_sparse_plan turns
 * the lists into cache-row lists and a split plan over the batch * s_q query tokens (each one a
 * sequence of one query row per head), mla_sparse_decode_fwd runs the decode. */

/* Bytes of the row-list buffer of mla_get_sparse_plan (batch * s_q lists of topk rounded up to
 * 32 entries, then batch * s_q counts), or 0 for an invalid shape. */
size_t mla_sparse_rows_bytes(int32_t batch, int32_t s_q, int32_t topk);

/* indices     device int32 [batch, s_q, topk].
 * topk        1 .. 2^20 entries per query token.
 * block_table, max_pages, seqlens, num_pages   as for mla_decode_fwd (the same preconditions).
 * batch, s_q  batch >= 1, s_q 1 .. 64, batch * s_q <= 16384.
 * heads       128 (one 128-row tile per query token).
 * num_pages   pages of the cache; num_pages * 64 * 640 must be below 2^31 (31-bit row offsets).
 * num_workers 1 .. 4096.
 * rows        device buffer of >= mla_sparse_rows_bytes(batch, s_q, topk) bytes, 16-byte aligned;
 *             written by the device; opaque; valid for mla_sparse_decode_fwd calls with the same
 *             indices, block table and lengths.
 * plan        device buffer of >= mla_plan_bytes(batch * s_q, 1, 128, num_workers) bytes, 16-byte
 *             aligned; written by the device.
 * status      device int32 word or NULL (MLA_DEVICE_PAGE_OUT_OF_RANGE for a listed key whose
 *             block-table entry is outside [0, num_pages); that key reads as zeros).
 * Runs entirely on the device. Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_WORKSPACE_TOO_SMALL (rows_bytes or plan_bytes), MLA_ERR_HIP. */
int32_t mla_get_sparse_plan(const int32_t* indices, int32_t topk, const int32_t* block_table, int32_t max_pages,
                            const int32_t* seqlens, int32_t batch, int32_t s_q, int32_t heads, int64_t num_pages,
                            int32_t num_workers, void* rows, size_t rows_bytes, void* plan, size_t plan_bytes,
                            int32_t* status, void* stream);

/* q, out, lse as for mla_decode_fwd ([batch, s_q, 128, ...]). kv_cache, kv_scales: the fp8 cache
 * (kv_dtype must be MLA_KV_FP8_E4M3; a bf16 cache is MLA_ERR_UNSUPPORTED here). rows, plan: from
 * mla_get_sparse_plan with the same batch, s_q, heads, topk, num_pages and num_workers.
 * workspace: >= mla_workspace_bytes(batch * s_q, 1, 128, num_workers) bytes (or NULL when that is
 * 0), 16-byte aligned. status: as for mla_decode_fwd. Results for a fixed plan are bitwise
 * reproducible.
 * Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED, MLA_ERR_WORKSPACE_TOO_SMALL, MLA_ERR_HIP. */
int32_t mla_sparse_decode_fwd(const void* q, const void* kv_cache, const float* kv_scales, int32_t kv_dtype,
                              int64_t num_pages, int32_t batch, int32_t s_q, int32_t heads, int32_t topk,
                              float softmax_scale, const void* rows, const void* plan, int32_t num_workers,
                              void* workspace, size_t workspace_bytes, float* out, float* lse, int32_t* status,
                              void* stream);

/* Split latent + decompressed attention (page "Mla Analysis", section "MLAvar6+ Design"): a
 * sequence's t cached tokens are split into o old tokens kept as latent rows and its n newest
 * kept decompressed (per head K and V of 128 channels, with the shared 64-channel rope key).
 * The old part is computed by mla_decode_fwd over the o latent tokens (seqlens = o, causal =
 * 0) followed by mla_decompress_output; this call attends over the n new tokens and merges the
 * two parts by their log-sum-exps, so that the result is the softmax attention over all t
 * tokens. Per query row (sequence i, token j, head e), with the new tokens visible to it
 * (all n; with causal, the first n - s_q + 1 + j, which keeps every old token visible):
 *
 *     a_u  = softmax_scale * ([q_nope | q_rope] . [k_new[i, u, e] | kr_new[i, u]])
 *     lse  = log(exp(lse_old) + sum_u exp(a_u))                  (natural log)
 *     out  = (exp(lse_old) out_old + sum_u exp(a_u) v_new[i, u, e]) / exp(lse)
 *
 * lse_old = -inf (an empty old part) and n_new = 0 are allowed; no key at all gives out = 0,
 * lse = -inf.
 *
 * q_nope   device bf16 [batch, s_q, heads, 128]; q_rope device bf16 [batch, s_q, heads, 64]
 *          (the unabsorbed query, rope rotation applied).
 * k_new    device bf16 [batch, n_new, heads, 128]; kr_new device bf16 [batch, n_new, 64];
 *          v_new device bf16 [batch, n_new, heads, 128]: the new tokens, oldest first (the
 *          last n_new of every sequence). May be NULL when n_new = 0.
 * out_old  device float32 [batch, s_q, heads, 128]: the old part's normalised output (the
 *          decompressed out of mla_decode_fwd); lse_old device float32 [batch, s_q, heads].
 * out      device float32 [batch, s_q, heads, 128]; lse device float32 [batch, s_q, heads].
 * batch, heads 1 .. 65535; s_q 1 .. 32; n_new 0 .. 2^24 with (n_new + 32) * heads * 256 < 2^31;
 * with causal, n_new >= s_q.
 * softmax_scale finite and > 0. All arrays but the lse ones 16-byte aligned and contiguous.
 * Stream-ordered; allocates nothing. Errors: MLA_ERR_INVALID_ARG, MLA_ERR_UNSUPPORTED,
 * MLA_ERR_HIP. */
int32_t mla_hybrid_merge(const void* q_nope, const void* q_rope, const void* k_new, const void* kr_new,
                         const void* v_new, int32_t n_new, const float* out_old, const float* lse_old,
                         int32_t batch, int32_t s_q, int32_t heads, float softmax_scale, int32_t causal,
                         float* out, float* lse, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBMLA_H */
