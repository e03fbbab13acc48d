// The two per-head projections around latent-space attention, as batched "NT" GEMMs on
// bf16 MFMA (page "Mla Analysis", section "Absorption Trick (FlashMLA)"):
//  * query absorption: Qz[t, h] = [q_nope[t, h] W_k[h]^T || q_rope[t, h]], W_k[h] of shape
//    [512, 128] (one row of 128 coefficients per latent channel), so that scoring against the
//    latent rows equals scoring the decompressed keys;
//  * output decompression: out[t, h] = O_latent[t, h] W_v[h]^T, W_v[h] of shape [128, 512]
//    (one row of 512 coefficients per output channel, the usual linear-layer layout); the
//    page leaves this to a separate kernel after the attention.
// In both, the contraction index is the innermost one of both operands, so an MFMA operand
// fragment (8 consecutive k of one row) is one 16-byte load and no staging is needed. One
// work-group per (128 output columns, 32 rows, head); wave w takes columns 32w .. 32w+31,
// the k loop runs in chunks of 8 MFMAs with all their operand loads in flight. The decode's
// fp32 O_latent is rounded to bf16 on load.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 pbf16x8;
typedef __attribute__((ext_vector_type(4))) float pf32x4;
typedef __attribute__((ext_vector_type(16))) float pf32x16;

constexpr int kProjThreads = 256;
constexpr int kProjChunk = 8;   // k-steps (16 each) per chunk

template <bool kAFloat>
__device__ __forceinline__ pbf16x8 load_a(const void* a, int64_t idx, bool ok) {
  pbf16x8 v;
  if (kAFloat) {
    const float* p = static_cast<const float*>(a) + idx;
    const pf32x4 lo = ok ? *reinterpret_cast<const pf32x4*>(p) : pf32x4{0.f, 0.f, 0.f, 0.f};
    const pf32x4 hi = ok ? *reinterpret_cast<const pf32x4*>(p + 4) : pf32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = (__bf16)lo[i];
      v[4 + i] = (__bf16)hi[i];
    }
  } else {
    const __bf16* p = static_cast<const __bf16*>(a) + idx;
    if (ok) {
      v = *reinterpret_cast<const pbf16x8*>(p);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) v[i] = (__bf16)0.f;
    }
  }
  return v;
}

// C[t, h, n] = sum_k A[t, h, k] B[h, n, k] for n < N (A rows of K elements, C rows of ldc
// elements); with a rope operand, C[t, h, N .. N+63] = rope[t, h, 0 .. 63] as well.
template <bool kAFloat, bool kCBf16>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(const void* __restrict__ A, const __bf16* __restrict__ B,
                                                            void* __restrict__ C, const __bf16* __restrict__ rope,
                                                            int T, int H, int K, int N, int ldc) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int h = blockIdx.z, m0 = 32 * blockIdx.y, n0 = 128 * blockIdx.x + 32 * wave;
  const int row = m0 + (lane & 31);
  const bool row_ok = row < T;
  const int kh = 8 * (lane >> 5);
  const int64_t a_row = ((int64_t)(row_ok ? row : 0) * H + h) * K + kh;
  const bool col_ok = n0 < N;   // (N is a multiple of 32)
  const int64_t b_row = ((int64_t)h * N + (col_ok ? n0 : 0) + (lane & 31)) * K + kh;
  pf32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  for (int kc = 0; kc < K; kc += 16 * kProjChunk) {
    pbf16x8 af[kProjChunk], bfr[kProjChunk];
#pragma unroll
    for (int j = 0; j < kProjChunk; ++j) {
      af[j] = load_a<kAFloat>(A, a_row + kc + 16 * j, row_ok);
      bfr[j] = *reinterpret_cast<const pbf16x8*>(B + b_row + kc + 16 * j);
    }
#pragma unroll
    for (int j = 0; j < kProjChunk; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[j], bfr[j], acc, 0, 0, 0);
  }
  if (col_ok) {
    // acc register r of lane l: row m0 + 8(r/4) + 4(l/32) + r%4, column n0 + l%32
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int m = m0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      if (m >= T) continue;
      const int64_t ci = ((int64_t)m * H + h) * ldc + n0 + (lane & 31);
      if (kCBf16) static_cast<__bf16*>(C)[ci] = (__bf16)acc[r];
      else static_cast<float*>(C)[ci] = acc[r];
    }
  }
  if (rope != nullptr && blockIdx.x == 0) {
    // 32 rows x 64 rope values (128 B per row): one 16-B chunk per thread
    const int rr = threadIdx.x >> 3, ch = threadIdx.x & 7;
    const int m = m0 + rr;
    if (m < T) {
      const int64_t src = ((int64_t)m * H + h) * 64 + 8 * ch;
      const int64_t dst = ((int64_t)m * H + h) * ldc + N + 8 * ch;
      *reinterpret_cast<pbf16x8*>(static_cast<__bf16*>(C) + dst) = *reinterpret_cast<const pbf16x8*>(rope + src);
    }
  }
}

}  // namespace

hipError_t launch_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int tokens, int heads,
                               void* qz, hipStream_t stream) {
  const dim3 grid(kLat / 128, (tokens + 31) / 32, heads);
  hipLaunchKernelGGL((proj_kernel<false, true>), grid, dim3(kProjThreads), 0, stream, q_nope,
                     static_cast<const __bf16*>(w_k), qz, static_cast<const __bf16*>(q_rope), tokens, heads,
                     kNope, kLat, kDqk);
  return hipGetLastError();
}

hipError_t launch_decompress_output(const float* out_latent, const void* w_v, int tokens, int heads, float* out,
                                    hipStream_t stream) {
  const dim3 grid(1, (tokens + 31) / 32, heads);
  hipLaunchKernelGGL((proj_kernel<true, false>), grid, dim3(kProjThreads), 0, stream,
                     static_cast<const void*>(out_latent), static_cast<const __bf16*>(w_v), static_cast<void*>(out),
                     static_cast<const __bf16*>(nullptr), tokens, heads, kLat, kDv, kDv);
  return hipGetLastError();
}

}  // namespace mla
