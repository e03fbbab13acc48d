// The two per-head projections around latent-space attention, as batched "NT" GEMMs on
// bf16 MFMA (page "Mla Analysis", section "Absorption Trick (FlashMLA)"):
//  * query absorption: Qz[t, h] = [q_nope[t, h] W_k[h]^T || q_rope[t, h]], W_k[h] of shape
//    [512, 128] (one row of 128 coefficients per latent channel), so that scoring against the
//    latent rows equals scoring the decompressed keys;
//  * output decompression: out[t, h] = O_latent[t, h] W_v[h]^T, W_v[h] of shape [128, 512]
//    (one row of 512 coefficients per output channel, the usual linear-layer layout); the
//    page leaves this to a separate kernel after the attention.
// In both, the contraction index is the innermost one of both operands. One work-group per
// (128 output columns, 32 rows, head); wave w takes columns 32w .. 32w+31. The 1-D grid puts
// the token tiles of one (head, column tile), which read the same weight block, on one XCD
// (work-groups are dealt to the 8 XCDs by block index), so that the block comes from HBM once
// and from that XCD's L2 after: 10.1 -> 8.3 us (absorption) and 9.2 -> 7.9 us
// (decompression) at 64 tokens x 128 heads. The k loop runs in
// chunks of 128: the chunk's operand blocks are copied into LDS by LDS-DMA (1 KiB contiguous
// per instruction; loaded straight into MFMA fragments, every load instruction would touch
// 32 rows), 16-byte chunks XOR-swizzled by row so that the fragment reads (32 rows x one
// chunk) are free of bank conflicts, then 8 MFMAs per wave. With more than one chunk (the
// decompression, k = 512) the blocks are double-buffered: chunk c+1 loads while chunk c is
// multiplied. Rows past the last token read as
// zeros (buffer range check). The decode's fp32 O_latent is rounded to bf16 when read.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kProjThreads = 256;
constexpr int kProjKc = 128;                  // k per chunk
constexpr int kProjBBytes = 128 * kProjKc * 2;   // B block: 128 rows x 128 k, bf16 (32 KiB)

// LDS-DMA of a block of `rows` rows x kProjKc elements of `esz` bytes from a row-major source
// (row stride `src_stride` bytes, block start at byte `src0` of the buffer): LDS holds row r at
// r * row_bytes with chunk c' holding source chunk c' ^ (r % 16). The work-group's 256
// threads issue the 1-KiB instructions in turn.
__device__ __forceinline__ void stage_block(const i32x4& rsrc, uint32_t lds_dst, uint32_t src0, uint32_t src_stride,
                                            int rows, int esz, int tid) {
  const int row_chunks = kProjKc * esz / 16;           // 16 (bf16) or 32 (fp32)
  const int instrs = rows * row_chunks / 64;
  const int lane = tid & 63, wave = tid >> 6;
  for (int i = wave; i < instrs; i += 4) {
    const int p = 64 * i + lane;
    const int r = p / row_chunks, cp = p % row_chunks;
    const int c = cp ^ (r & 15);
    lds_dma_x4(lds_dst + 1024u * (uint32_t)i, src0 + (uint32_t)r * src_stride + 16u * (uint32_t)c, rsrc);
  }
}

// DMA instructions one wave issues for one chunk (B block, then A block)
template <bool kAFloat>
constexpr int chunk_dma_per_wave() {
  return (128 * kProjKc * 2 / 16 / 64 + 32 * kProjKc * (kAFloat ? 4 : 2) / 16 / 64) / 4;
}

// C[t, h, n] = sum_k A[t, h, k] B[h, n, k] for n < N (A rows of K elements, C rows of ldc
// elements); with a rope operand, C[t, h, N .. N+63] = rope[t, h, 0 .. 63] as well. kDb: two
// LDS buffers (K > kProjKc).
template <bool kAFloat, bool kCBf16, bool kDb>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(const void* __restrict__ A, const __bf16* __restrict__ B,
                                                            void* __restrict__ C, const __bf16* __restrict__ rope,
                                                            int T, int H, int K, int N, int ldc) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  constexpr int esz = kAFloat ? 4 : 2;
  constexpr int a_row_bytes = kProjKc * esz;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block -> (column tile, token tile, head): the token tiles of one (head, column tile), which read
  // the same weight block, share a block-index residue mod 8 and so an XCD and its L2
  const int ncol = N / 128, ntile = (T + 31) / 32;
  const int lin = blockIdx.x, x8 = lin & 7, r = lin >> 3;
  const int ytile = r % ntile, pair = (r / ntile) * 8 + x8;
  if (pair >= ncol * H) return;
  const int h = pair / ncol, m0 = 32 * ytile, nb = 128 * (pair - h * ncol);
  // A: all T rows of head h; row m at byte (m H + h) K esz; the range check zero-fills m >= T
  const i32x4 ra = make_rsrc(reinterpret_cast<uint64_t>(A), (int)((int64_t)T * H * K * esz));
  // B: rows nb .. nb+127 of head h, K elements each
  const i32x4 rb = make_rsrc(reinterpret_cast<uint64_t>(B) + ((uint64_t)h * N + nb) * K * 2, 128 * K * 2);
  constexpr uint32_t kBufBytesP = kProjBBytes + 32 * a_row_bytes;   // one buffer: B block, then A block
  f32x16 acc;
#pragma unroll
  for (int r = 0; r < 16; ++r) acc[r] = 0.f;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nrow = 32 * wave + l32;   // this lane's row of the B block
  auto stage = [&](int kc, uint32_t buf) {
    stage_block(rb, lds_u32 + buf, (uint32_t)kc * 2, (uint32_t)K * 2, 128, 2, tid);
    stage_block(ra, lds_u32 + buf + kProjBBytes, (uint32_t)(((int64_t)m0 * H + h) * K + kc) * esz,
                (uint32_t)H * K * esz, 32, esz, tid);
  };
  if (kDb) stage(0, 0u);
  for (int kc = 0; kc < K; kc += kProjKc) {
    const uint32_t buf = kDb ? ((kc / kProjKc) & 1) * kBufBytesP : 0u;
    if (kDb) {
      if (kc + kProjKc < K) {
        stage(kc + kProjKc, kBufBytesP - buf);   // the next chunk into the other buffer
        wait_vmcnt<chunk_dma_per_wave<kAFloat>()>();
      } else {
        wait_vmcnt<0>();
      }
    } else {
      stage(kc, 0u);
      wait_vmcnt<0>();
    }
    barrier_lds();
#pragma unroll
    for (int j = 0; j < kProjKc / 16; ++j) {
      const int c = 2 * j + hh;   // logical 16-B chunk of k 16j + 8hh .. +7 (bf16)
      const bf16x8 bf = lds_b128(lds + (buf + nrow * 256 + 16 * (c ^ (nrow & 15))));
      bf16x8 af;
      if (kAFloat) {
        // fp32: the 8 values are logical chunks 2c, 2c+1 of a 512-B row
        const f32x4 lo = *(const f32x4 __attribute__((address_space(3)))*)(
            lds + (buf + kProjBBytes + l32 * a_row_bytes + 16 * ((2 * c) ^ (l32 & 15))));
        const f32x4 hi = *(const f32x4 __attribute__((address_space(3)))*)(
            lds + (buf + kProjBBytes + l32 * a_row_bytes + 16 * ((2 * c + 1) ^ (l32 & 15))));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          af[i] = (__bf16)lo[i];
          af[4 + i] = (__bf16)hi[i];
        }
      } else {
        af = lds_b128(lds + (buf + kProjBBytes + l32 * a_row_bytes + 16 * (c ^ (l32 & 15))));
      }
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc, 0, 0, 0);
    }
    barrier_lds();   // the blocks are read before a later chunk overwrites them
  }
  const int n0 = nb + 32 * wave;
  // acc register r of lane l: row m0 + 8(r/4) + 4(l/32) + r%4, column n0 + l%32
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int m = m0 + 8 * (r >> 2) + 4 * hh + (r & 3);
    if (m >= T) continue;
    const int64_t ci = ((int64_t)m * H + h) * ldc + n0 + l32;
    if (kCBf16) static_cast<__bf16*>(C)[ci] = (__bf16)acc[r];
    else static_cast<float*>(C)[ci] = acc[r];
  }
  if (rope != nullptr && nb == 0) {
    // 32 rows x 64 rope values (128 B per row): one 16-B chunk per thread
    const int rr = tid >> 3, ch = tid & 7;
    const int m = m0 + rr;
    if (m < T) {
      const int64_t src = ((int64_t)m * H + h) * 64 + 8 * ch;
      const int64_t dst = ((int64_t)m * H + h) * ldc + N + 8 * ch;
      *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(C) + dst) = *reinterpret_cast<const bf16x8*>(rope + src);
    }
  }
}

constexpr int proj_lds_bytes(bool a_float, bool db) {
  return (db ? 2 : 1) * (kProjBBytes + 32 * kProjKc * (a_float ? 4 : 2));
}

}  // namespace

hipError_t launch_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int tokens, int heads,
                               void* qz, hipStream_t stream) {
  const int pairs = (kLat / 128) * heads;
  const dim3 grid(((pairs + 7) / 8) * 8 * ((tokens + 31) / 32));
  hipLaunchKernelGGL((proj_kernel<false, true, false>), grid, dim3(kProjThreads), proj_lds_bytes(false, false), stream,
                     q_nope,
                     static_cast<const __bf16*>(w_k), qz, static_cast<const __bf16*>(q_rope), tokens, heads,
                     kNope, kLat, kDqk);
  return hipGetLastError();
}

hipError_t launch_decompress_output(const float* out_latent, const void* w_v, int tokens, int heads, float* out,
                                    hipStream_t stream) {
  static thread_local int configured = -1;   // the LDS opt-in (96 KiB, two buffers) is per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)proj_kernel<true, false, true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            proj_lds_bytes(true, true));
    if (e != hipSuccess) return e;
    configured = dev;
  }
  const int pairs = heads;
  const dim3 grid(((pairs + 7) / 8) * 8 * ((tokens + 31) / 32));
  hipLaunchKernelGGL((proj_kernel<true, false, true>), grid, dim3(kProjThreads), proj_lds_bytes(true, true), stream,
                     static_cast<const void*>(out_latent), static_cast<const __bf16*>(w_v), static_cast<void*>(out),
                     static_cast<const __bf16*>(nullptr), tokens, heads, kLat, kDv, kDv);
  return hipGetLastError();
}

}  // namespace mla
