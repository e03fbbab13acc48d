// Split latent + decompressed attention (page "Mla Analysis", section "MLAvar6+ Design"): a
// sequence's o old tokens are latent rows, handled by the latent decode and the output
// decompression, and its n newest tokens are kept decompressed, per head K [n, h, 128] and
// V [n, h, 128] plus the shared rope key [n, 64]. This kernel attends over the new tokens and
// merges the result with the old part's (out, lse) by their log-sum-exps, which makes the
// softmax span all t = o + n tokens exactly.
//
// One work-group of four waves per (sequence, head); all s_q <= 32 query rows of the head form
// one 32-row MFMA tile (rows past s_q repeat row 0 and are not written). Wave w takes the new
// tokens' 32-token chunks w, w+4, ...: each chunk is loaded straight into the wave's LDS buffer
// by LDS-DMA (80 KiB per work-group, so that a second work-group on the CU streams while this
// one waits, starts or merges), as three regions whose 16-B chunks are
// XOR-swizzled by token so that the operand reads are free of bank conflicts: K (128 channels,
// 256-B rows, chunk ^ u%16), the rope keys (128-B rows, chunk ^ (u/2)%8) and V (256-B rows,
// chunk ^ 4(u%4)). Per chunk: S^T[32 tokens x 32 rows] = K Q^T (12
// v_mfma_f32_32x32x16_bf16, Q^T in registers), mask, online softmax in the log2 domain with a
// reference that moves only when a row's maximum passes it by more than 2^8, then
// O[32 rows x 128] += P V (8 MFMAs; P is the score accumulator rounded to bf16, read as the A
// operand with its token order, V^T tiles from transposing LDS reads). The four waves' partials
// and the old part are then merged through LDS. The new tokens' part moves w(2 h n d + n p)
// bytes for 4 h s n d flops per sequence, far below the MI355X ridge: it is bound by HBM.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kHyThreads = 256;
constexpr int kHyChunk = 32;                      // new tokens per chunk
constexpr int kHyR = kHyChunk * 256;              // buffer regions: K rows (256 B) at 0, rope rows (128 B),
constexpr int kHyV = kHyR + kHyChunk * 128;       // V rows (256 B)
constexpr int kHyBuf = kHyV + kHyChunk * 256;     // 20 KiB per chunk buffer
constexpr int kHyArea = kHyBuf;                   // per wave: one buffer
constexpr int kHyLds = 4 * kHyArea;               // 80 KiB: two work-groups per CU
constexpr int kHyDma = 20;                        // LDS-DMA instructions per chunk and wave
constexpr int kHyObufRow = 132;                   // floats per partial O row in the merge (528 B)
static_assert(kHyLds <= 160 * 1024, "LDS budget");
static_assert(4 * 32 * kHyObufRow * 4 + 4 * 32 * 8 <= kHyLds, "the merge area fits in the staging areas");

// physical byte offset of logical 16-B chunk ch of token row u in each region
__device__ __forceinline__ uint32_t hy_k(uint32_t u, uint32_t ch) { return u * 256u + 16u * (ch ^ (u & 15u)); }
__device__ __forceinline__ uint32_t hy_r(uint32_t u, uint32_t ch) { return u * 128u + 16u * (ch ^ ((u >> 1) & 7u)); }
__device__ __forceinline__ uint32_t hy_v(uint32_t u, uint32_t ch) { return u * 256u + 16u * (ch ^ (4u * (u & 3u))); }

__global__ __launch_bounds__(kHyThreads, 2) void hybrid_new_kernel(
    const __bf16* __restrict__ q_nope, const __bf16* __restrict__ q_rope, const __bf16* __restrict__ k_new,
    const __bf16* __restrict__ kr_new, const __bf16* __restrict__ v_new, const float* __restrict__ out_old,
    const float* __restrict__ lse_old, float* __restrict__ out, float* __restrict__ lse, int S, int N, int H,
    float scale_log2, int causal) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  const int h = blockIdx.x, b = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t area = (uint32_t)wave * kHyArea;
  const int row = lane & 31, hl = lane >> 5;

  // Q^T B operand: lane holds query row l%32, channels 16ks + 8(l/32) .. +7 (ks 0..7 nope, 8..11 rope)
  bf16x8 qb[12];
  {
    const int j = row < S ? row : 0;
    const __bf16* qn = q_nope + (((int64_t)b * S + j) * H + h) * 128 + 8 * hl;
    const __bf16* qr = q_rope + (((int64_t)b * S + j) * H + h) * 64 + 8 * hl;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qb[ks] = *reinterpret_cast<const bf16x8*>(qn + 16 * ks);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qb[8 + ks] = *reinterpret_cast<const bf16x8*>(qr + 16 * ks);
  }
  // The old part's (out, lse) of the rows this thread merges at the end (row tid / 8, channels
  // 32k + 4 (tid % 8) .. +3), requested now so that their latency passes during the new tokens
  // instead of after them.
  const int m_rr = threadIdx.x >> 3, m_q4 = 4 * (threadIdx.x & 7);
  f32x4 ov_pre[4];
  float lo_pre = -INFINITY;
  if (m_rr < S) {
    const int64_t orow = ((int64_t)b * S + m_rr) * H + h;
    lo_pre = lse_old[orow];
#pragma unroll
    for (int k = 0; k < 4; ++k) ov_pre[k] = *reinterpret_cast<const f32x4*>(out_old + orow * 128 + 32 * k + m_q4);
  }
  // new tokens visible to this lane's row (0 for padding rows)
  const int lim = row < S ? (causal ? N - S + 1 + row : N) : 0;

  // buffer descriptors over sequence b's new tokens: K and V rows of head h at (u H + h) 256 B,
  // rope rows at 128u B; tokens past N read as zeros (the host keeps N H 256 below 2^31)
  const i32x4 rk = make_rsrc(reinterpret_cast<uint64_t>(k_new) + (uint64_t)b * N * H * 256, N * H * 256);
  const i32x4 rv = make_rsrc(reinterpret_cast<uint64_t>(v_new) + (uint64_t)b * N * H * 256, N * H * 256);
  const i32x4 rr = make_rsrc(reinterpret_cast<uint64_t>(kr_new) + (uint64_t)b * N * 128, N * 128);
  // chunk c into buffer bf: instruction m of each region fills 1 KiB (K, V: 4 rows; rope: 8 rows);
  // lane l lands at 16 l, which holds the logical chunk the region's swizzle puts there. K and V
  // rows of a head are read by this work-group only, once: non-temporal (295 -> 282 us per merge
  // at b=32 s=16 n=640); the rope rows are shared by the sequence's heads and stay cached.
  auto dma_chunk = [&](int c, int bf) {
    const uint32_t dst = lds_u32 + area + (uint32_t)bf * kHyBuf;
    const uint32_t l = (uint32_t)lane;
#pragma unroll
    for (int m = 0; m < 8; ++m) {
      const uint32_t u = 4u * m + (l >> 4), un = (uint32_t)kHyChunk * c + u;
      const uint32_t rowoff = (un * (uint32_t)H + (uint32_t)h) * 256u;
      lds_dma_x4_stream(dst + 1024u * m, rowoff + 16u * ((l & 15u) ^ (u & 15u)), rk);
      lds_dma_x4_stream(dst + kHyV + 1024u * m, rowoff + 16u * ((l & 15u) ^ (4u * (u & 3u))), rv);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const uint32_t u = 8u * m + (l >> 3), un = (uint32_t)kHyChunk * c + u;
      lds_dma_x4(dst + kHyR + 1024u * m, un * 128u + 16u * ((l & 7u) ^ ((u >> 1) & 7u)), rr);
    }
  };
  // operand reads: K rows (lane: token l%32, logical chunk 2ks + l/32 of the 192 channels); V^T
  // tile (q, c): tokens 16q + 8e + 4(G/2) + j/4 and channels 32c + 16(G%2) + 4(j%4) .. +3 for
  // lane (G, j) = (l/16, l%16)
  auto k_read = [&](uint32_t base, int ks) -> bf16x8 {
    const uint32_t ch = (uint32_t)(2 * ks + hl);
    return lds_b128(lds + (ks < 8 ? base + hy_k((uint32_t)row, ch) : base + kHyR + hy_r((uint32_t)row, ch - 16u)));
  };
  auto v_read = [&](uint32_t base, int q, int c) -> bf16x8 {
    const uint32_t G = (uint32_t)lane >> 4, j = (uint32_t)lane & 15u;
    bf16x4 part[2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint32_t u = 16u * q + 8u * e + 4u * (G >> 1) + (j >> 2);
      const uint32_t ch = 4u * c + 2u * (G & 1u) + ((j >> 1) & 1u);
      part[e] = lds_tr16(lds + (base + kHyV + hy_v(u, ch) + 8u * (j & 1u)));
    }
    return __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
  };

  f32x16 o[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) o[c] = f32x16{};
  float m_ref = -INFINITY;   // the row's reference (log2 units): p = 2^(s - m_ref)
  float l_run = 0.f;
  const int nchunks = (N + kHyChunk - 1) / kHyChunk;
  bool first = true;
  // this wave's chunks c = wave + 4k, one in flight (the other work-group on the CU covers the
  // wait)
  if (wave < nchunks) dma_chunk(wave, 0);
#pragma unroll 1
  for (int c = wave, k = 0; c < nchunks; c += 4, ++k) {
    wait_vmcnt<0>();
    const uint32_t base = area;
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < 12; ++ks) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k_read(base, ks), qb[ks], s, 0, 0, 0);
    // mask (register r: token 32c + 8(r/4) + 4(l/32) + r%4) and the row maximum
    const int key0 = kHyChunk * c + 4 * hl;
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = (key0 + 8 * (r >> 2) + (r & 3)) < lim ? s[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, s[r]);
    }
    {
      const unsigned u = __float_as_uint(mx);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // move the reference when the row maximum passes it by more than 2^8
    const bool move = mx > m_ref + 8.f;
    const float new_ref = move ? mx : m_ref;
    const float alpha = move ? (m_ref == -INFINITY ? 0.f : exp2f(m_ref - new_ref)) : 1.f;
    if (__ballot(move) != 0) {   // (wave-uniform)
      l_run *= alpha;
      if (!first) {   // O rows live in other lanes: their factors go through LDS (the K rows, read by now)
        float __attribute__((address_space(3)))* alpha_s = (float __attribute__((address_space(3)))*)(lds + base);
        __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // (the K reads first)
        if (lane < 32) alpha_s[lane] = alpha;
        f32x4 a4[4];
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
          a4[jj] = *(const f32x4 __attribute__((address_space(3)))*)(alpha_s + 8 * jj + 4 * hl);
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[t][r] *= a4[r >> 2][r & 3];
      }
    }
    m_ref = new_ref;
    first = false;
    const float muse = m_ref == -INFINITY ? 0.f : m_ref;
    bf16x8 pk[2];
    float ps = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2f(s[r] - muse);
      ps += p;
      pk[r >> 3][r & 7] = (__bf16)p;
    }
    {
      const unsigned u = __float_as_uint(ps);
      const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
      l_run += __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
    }
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int t = 0; t < 4; ++t)
        o[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(pk[q], v_read(base, q, t), o[t], 0, 0, 0);
    // the buffer's next chunk, once this chunk's LDS reads are done
    if (c + 4 < nchunks) {
      __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
      dma_chunk(c + 4, 0);
    }
  }
  wait_vmcnt<0>();

  // ---- merge: the four waves' partials (relative to their references) and the old part
  __syncthreads();   // every wave is done with its staging area
  // partial O rows at a 640-B stride (128-B bank halves alternate), then the per-row (m, l)
  float __attribute__((address_space(3)))* obuf = (float __attribute__((address_space(3)))*)lds;
  float __attribute__((address_space(3)))* stat = obuf + 4 * 32 * kHyObufRow;
  if (lane < 32) {
    stat[2 * (32 * wave + row)] = m_ref;
    stat[2 * (32 * wave + row) + 1] = l_run;
  }
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int rr = 8 * (r >> 2) + 4 * hl + (r & 3);
      obuf[(32 * wave + rr) * kHyObufRow + 32 * t + row] = o[t][r];
    }
  __syncthreads();
  {
    // thread: row tid / 8, channels 32k + 4(tid % 8) .. +3 for k = 0..3
    const int tid = threadIdx.x, rr = m_rr, q4 = m_q4;
    if (rr < S) {
      const int64_t orow = ((int64_t)b * S + rr) * H + h;
      const float lo = lo_pre;
      const float m_old = lo == -INFINITY ? -INFINITY : lo * 1.4426950408889634f;
      float M = m_old;
#pragma unroll
      for (int w = 0; w < 4; ++w) M = fmaxf(M, stat[2 * (32 * w + rr)]);
      float a[4], den = 0.f;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float mw = stat[2 * (32 * w + rr)];
        a[w] = (mw == -INFINITY) ? 0.f : exp2f(mw - M);
        den += a[w] * stat[2 * (32 * w + rr) + 1];
      }
      const float a_old = (m_old == -INFINITY) ? 0.f : exp2f(m_old - M);
      den += a_old;
      const float inv = den > 0.f ? 1.f / den : 0.f;
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const int c0 = 32 * k + q4;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (a_old != 0.f) {
          const f32x4 ov = ov_pre[k];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = a_old * ov[e];
        }
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const f32x4 pv = *(const f32x4 __attribute__((address_space(3)))*)(obuf + (32 * w + rr) * kHyObufRow + c0);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] += a[w] * pv[e];
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= inv;
        *reinterpret_cast<f32x4*>(out + orow * 128 + c0) = acc;
      }
      if ((tid & 7) == 0) lse[orow] = den > 0.f ? (M + __log2f(den)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

}  // namespace

hipError_t launch_hybrid_merge(const HybridArgs& a, hipStream_t stream) {
  static thread_local int configured = -1;   // the LDS opt-in is per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)hybrid_new_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kHyLds);
    if (e != hipSuccess) return e;
    configured = dev;
  }
  hipLaunchKernelGGL(hybrid_new_kernel, dim3(a.heads, a.batch), dim3(kHyThreads), kHyLds, stream,
                     static_cast<const __bf16*>(a.q_nope), static_cast<const __bf16*>(a.q_rope),
                     static_cast<const __bf16*>(a.k_new), static_cast<const __bf16*>(a.kr_new),
                     static_cast<const __bf16*>(a.v_new), a.out_old, a.lse_old, a.out, a.lse, a.s_q, a.n_new,
                     a.heads, a.scale_log2, a.causal);
  return hipGetLastError();
}

}  // namespace mla
