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
constexpr int kProjSmallTokens = 64;             // up to this many tokens: 32-token tiles
constexpr int kAbsorbTile = 32;                  // absorption token tile above that (32: 1-4% faster than 64)

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

// DMA instructions one wave issues for one chunk (B block, then A block of kMT rows)
template <bool kAFloat, int kMT>
constexpr int chunk_dma_per_wave() {
  return (128 * kProjKc * 2 / 16 / 64 + kMT * kProjKc * (kAFloat ? 4 : 2) / 16 / 64) / 4;
}

// C[t, h, n] = sum_k A[t, h, k] B[h, n, k] for n < N (A rows of K elements, C rows of ldc
// elements); with a rope operand, C[t, h, N .. N+63] = rope[t, h, 0 .. 63] as well. kDb: two
// LDS buffers (K > kProjKc). kMT: tokens per work-group (32, 64 or 128); each wave multiplies
// its 32 columns of the weight block with every 32-row block of the token tile, so a weight
// fragment read from LDS serves kMT / 32 MFMAs and the weight block is staged once per kMT
// tokens.
// bf16 output (the absorption): the MFMA takes the weight rows as its first operand, so a
// lane's accumulator holds one token and runs of four consecutive columns; the tile goes to
// LDS as 8-B runs (16-B chunks XOR-swizzled by row) and leaves as whole 256-B row segments,
// 16 B per thread. fp32 output (the decompression): a lane holds one column and 16 rows, so
// each store instruction already writes two whole 128-B row segments.
template <bool kAFloat, bool kCBf16, bool kDb, int kMT>
__global__ __launch_bounds__(kProjThreads) void proj_kernel(const void* __restrict__ A, const __bf16* __restrict__ B,
                                                            void* __restrict__ C, const __bf16* __restrict__ rope,
                                                            int T, int H, int K, int N, int ldc) {
  static_assert(kMT == 32 || kMT == 64 || kMT == 128, "token tile");
  // (with a rope operand N = 512: four column tiles, kMT / 4 rope rows each, at most 256 threads' worth)
  constexpr int kRB = kMT / 32;   // 32-row blocks per tile
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  constexpr int esz = kAFloat ? 4 : 2;
  constexpr int a_row_bytes = kProjKc * esz;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // block -> (column tile, token tile, head): the token tiles of one (head, column tile), which read
  // the same weight block, share a block-index residue mod 8 and so an XCD and its L2
  const int ncol = N / 128, ntile = (T + kMT - 1) / kMT;
  const int lin = blockIdx.x, x8 = lin & 7, r = lin >> 3;
  const int ytile = r % ntile, pair = (r / ntile) * 8 + x8;
  if (pair >= ncol * H) return;
  const int h = pair / ncol, m0 = kMT * ytile, nb = 128 * (pair - h * ncol);
  // A: all T rows of head h; row m at byte (m H + h) K esz; the range check zero-fills m >= T
  const i32x4 ra = make_rsrc(reinterpret_cast<uint64_t>(A), (int)((int64_t)T * H * K * esz));
  // B: rows nb .. nb+127 of head h, K elements each
  const i32x4 rb = make_rsrc(reinterpret_cast<uint64_t>(B) + ((uint64_t)h * N + nb) * K * 2, 128 * K * 2);
  constexpr uint32_t kBufBytesP = kProjBBytes + kMT * a_row_bytes;   // one buffer: B block, then A block
  // rope rows of the tile (16 B per thread, kMT x 128 B per tile): shared by the ncol column tiles
  // of the head, each taking kMT / ncol rows, loaded now so that their latency passes under the
  // operand loads, stored at the end
  bf16x8 rope_v;
  int64_t rope_dst = -1;
  if (rope != nullptr) {
    const int rows = kMT / ncol, ct = nb / 128;
    if (tid < 8 * rows) {
      const int m = m0 + ct * rows + (tid >> 3), ch = tid & 7;
      if (m < T) {
        rope_v = *reinterpret_cast<const bf16x8*>(rope + ((int64_t)m * H + h) * 64 + 8 * ch);
        rope_dst = ((int64_t)m * H + h) * ldc + N + 8 * ch;
      }
    }
  }
  f32x16 acc[kRB];
#pragma unroll
  for (int i = 0; i < kRB; ++i)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[i][r] = 0.f;
  const int l32 = lane & 31, hh = lane >> 5;
  const int nrow = 32 * wave + l32;   // this lane's row of the B block
  auto stage = [&](int kc, uint32_t buf) {
    stage_block(rb, lds_u32 + buf, (uint32_t)kc * 2, (uint32_t)K * 2, 128, 2, tid);
    stage_block(ra, lds_u32 + buf + kProjBBytes, (uint32_t)(((int64_t)m0 * H + h) * K + kc) * esz,
                (uint32_t)H * K * esz, kMT, esz, tid);
  };
  if (kDb) stage(0, 0u);
  for (int kc = 0; kc < K; kc += kProjKc) {
    const uint32_t buf = kDb ? ((kc / kProjKc) & 1) * kBufBytesP : 0u;
    if (kDb) {
      if (kc + kProjKc < K) {
        stage(kc + kProjKc, kBufBytesP - buf);   // the next chunk into the other buffer
        wait_vmcnt<chunk_dma_per_wave<kAFloat, kMT>()>();
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
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        // A row 32 i + l32 of the tile (the swizzle depends on the row's low 4 bits only)
        const uint32_t arow = buf + kProjBBytes + (uint32_t)(32 * i + l32) * a_row_bytes;
        bf16x8 af;
        if (kAFloat) {
          // fp32: the 8 values are logical chunks 2c, 2c+1 of a 512-B row
          const f32x4 lo = *(const f32x4 __attribute__((address_space(3)))*)(lds + (arow + 16 * ((2 * c) ^ (l32 & 15))));
          const f32x4 hi =
              *(const f32x4 __attribute__((address_space(3)))*)(lds + (arow + 16 * ((2 * c + 1) ^ (l32 & 15))));
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            af[q] = (__bf16)lo[q];
            af[4 + q] = (__bf16)hi[q];
          }
        } else {
          af = lds_b128(lds + (arow + 16 * (c ^ (l32 & 15))));
        }
        if (kCBf16) acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bf, af, acc[i], 0, 0, 0);
        else acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bf, acc[i], 0, 0, 0);
      }
    }
    barrier_lds();   // the blocks are read before a later chunk (or the output tile) overwrites them
  }
  if constexpr (kCBf16) {
    // acc[i] register 4q + v of lane l: token 32 i + l%32 of the tile, column 32 wave + 8q + 4(l/32) + v
    // -> LDS row t (256 B), 16-B chunk (4 wave + q) ^ (t % 16), bytes 8(l/32) .. +7
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const uint32_t t = (uint32_t)(32 * i + l32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[i][4 * q + e];
        const uint32_t off = t * 256u + 16u * (((uint32_t)(4 * wave + q)) ^ (t & 15u)) + 8u * (uint32_t)hh;
        *(bf16x4 __attribute__((address_space(3)))*)(lds + off) = v;
      }
    }
    barrier_lds();
    // row t, logical chunk q (columns nb + 8q .. +7): 16 threads per row
#pragma unroll
    for (int s2 = 0; s2 < kMT * 16 / kProjThreads; ++s2) {
      const int k = tid + kProjThreads * s2;
      const int t = k >> 4, q = k & 15;
      const int m = m0 + t;
      const u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)(lds + (t * 256 + 16 * (q ^ (t & 15))));
      if (m < T) {
        const int64_t ci = ((int64_t)m * H + h) * ldc + nb + 8 * q;
        *reinterpret_cast<u32x4*>(static_cast<__bf16*>(C) + ci) = v;
      }
    }
  } else {
    const int n0 = nb + 32 * wave;
    // acc[i] register r of lane l: row m0 + 32 i + 8(r/4) + 4(l/32) + r%4, column n0 + l%32
#pragma unroll
    for (int i = 0; i < kRB; ++i)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int m = m0 + 32 * i + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (m >= T) continue;
        static_cast<float*>(C)[((int64_t)m * H + h) * ldc + n0 + l32] = acc[i][r];
      }
  }
  if (rope_dst >= 0) *reinterpret_cast<bf16x8*>(static_cast<__bf16*>(C) + rope_dst) = rope_v;
}

// Query absorption for many tokens: one work-group per (head, 128-column tile, token share).
// Each wave keeps its 32 weight columns (all 128 k) in 32 VGPRs for the whole work-group, so
// the weight block is read once per work-group; the work-group then walks its token tiles of
// kMT rows (tiles split, split + S, ...), staging each q_nope tile in LDS by LDS-DMA and
// writing the bf16 output through LDS as 16-B row stores (as in proj_kernel). LDS is only the
// operand tile and the output tile (2 x kMT x 256 B), so several work-groups share a CU and
// cover each other's load and store latencies. The S token shares of one (head, column tile)
// and the four column tiles of a head (which read the same q_nope rows) share a block-index
// residue mod 8, hence an XCD and its L2. The head's rope rows are copied by its four column
// tiles, a quarter of each token tile each.
template <int kMT>
__global__ __launch_bounds__(kProjThreads) void absorb_tiles_kernel(const __bf16* __restrict__ A,
                                                                    const __bf16* __restrict__ B,
                                                                    __bf16* __restrict__ C,
                                                                    const __bf16* __restrict__ rope, int T, int H,
                                                                    int S) {
  static_assert(kMT == 32 || kMT == 64 || kMT == 128, "token tile");
  constexpr int kRB = kMT / 32;
  constexpr int K = kNope, N = kLat, ldc = kDqk;
  constexpr uint32_t kOut = kMT * 256;   // output tile after the operand tile
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int lin = blockIdx.x, x8 = lin & 7, r = lin >> 3;
  const int ct = r & 3, split = (r >> 2) % S, h = (r / (4 * S)) * 8 + x8;
  if (h >= H) return;
  const int nb = 128 * ct, ntile = (T + kMT - 1) / kMT;
  // this lane's weight fragments: row nb + 32 wave + l32 of W_k[h], k 16j + 8hh .. +7
  bf16x8 bfr[8];
  {
    const __bf16* wrow = B + ((int64_t)h * N + nb + 32 * wave + l32) * K + 8 * hh;
#pragma unroll
    for (int j = 0; j < 8; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(wrow + 16 * j);
  }
  const i32x4 ra = make_rsrc(reinterpret_cast<uint64_t>(A), (int)((int64_t)T * H * K * 2));
#pragma unroll 1
  for (int it = split; it < ntile; it += S) {
    const int m0 = kMT * it;
    stage_block(ra, lds_u32, (uint32_t)(((int64_t)m0 * H + h) * K) * 2, (uint32_t)H * K * 2, kMT, 2, tid);
    // this column tile's quarter of the tile's rope rows: 16 B per thread
    bf16x8 rope_v;
    int64_t rope_dst = -1;
    if (tid < 2 * kMT) {
      const int m = m0 + ct * (kMT / 4) + (tid >> 3), ch = tid & 7;
      if (m < T) {
        rope_v = *reinterpret_cast<const bf16x8*>(rope + ((int64_t)m * H + h) * 64 + 8 * ch);
        rope_dst = ((int64_t)m * H + h) * ldc + N + 8 * ch;
      }
    }
    wait_vmcnt<0>();
    barrier_lds();
    f32x16 acc[kRB];
#pragma unroll
    for (int i = 0; i < kRB; ++i)
#pragma unroll
      for (int q = 0; q < 16; ++q) acc[i][q] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int c = 2 * j + hh;
#pragma unroll
      for (int i = 0; i < kRB; ++i) {
        const bf16x8 af = lds_b128(lds + ((uint32_t)(32 * i + l32) * 256u + 16u * (uint32_t)(c ^ (l32 & 15))));
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[j], af, acc[i], 0, 0, 0);
      }
    }
    // acc[i] register 4q + v of lane l: token 32 i + l%32, column 32 wave + 8q + 4(l/32) + v
#pragma unroll
    for (int i = 0; i < kRB; ++i) {
      const uint32_t t = (uint32_t)(32 * i + l32);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bf16x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = (__bf16)acc[i][4 * q + e];
        *(bf16x4 __attribute__((address_space(3)))*)(lds + (kOut + t * 256u +
                                                            16u * (((uint32_t)(4 * wave + q)) ^ (t & 15u)) +
                                                            8u * (uint32_t)hh)) = v;
      }
    }
    barrier_lds();   // (also: every wave has read the operand tile before the next one is loaded)
#pragma unroll
    for (int s2 = 0; s2 < kMT * 16 / kProjThreads; ++s2) {
      const int k = tid + kProjThreads * s2;
      const int t = k >> 4, q = k & 15;
      const int m = m0 + t;
      const u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)(lds + (kOut + t * 256 + 16 * (q ^ (t & 15))));
      if (m < T) *reinterpret_cast<u32x4*>(C + ((int64_t)m * H + h) * ldc + nb + 8 * q) = v;
    }
    if (rope_dst >= 0) *reinterpret_cast<bf16x8*>(C + rope_dst) = rope_v;
  }
}

// Output decompression for many tokens: one work-group per (head, token share). Each wave keeps
// its 32 output columns of W_v[h] over all 512 k in 128 VGPRs for the whole work-group, so the
// weights are read once per work-group; the fp32 O_latent rows of each 32-token tile stream
// through LDS in four 128-k chunks of 16 KiB by LDS-DMA, kDecAhead chunks ahead of the one
// multiplied (kDecAhead + 1 buffers). The waits count exactly what is younger than the chunk
// awaited: the later chunks' DMA instructions (issued for every chunk position, with zero
// records past the work-group's last chunk) and, for the first kDecAhead chunks of a tile, the
// previous tile's output stores, which are range-checked buffer stores (rows past the last
// token are dropped by the buffer's record count) so that every wave issues exactly 16 of them
// per tile. The S token shares of a head share a block-index residue mod 8, hence an XCD and
// the L2 that serves their weight reads.
constexpr int kDecAhead = 3;
__global__ __launch_bounds__(kProjThreads) void decompress_tiles_kernel(const float* __restrict__ A,
                                                                        const __bf16* __restrict__ B,
                                                                        float* __restrict__ C, int T, int H, int S) {
  constexpr int K = kLat, N = kDv, kMT = 32;
  constexpr uint32_t kChunk = kMT * kProjKc * 4;          // 16 KiB of fp32 rows
  constexpr int kBufs = kDecAhead + 1;
  constexpr int kDmaW = kChunk / 1024 / 4;                // LDS-DMA instructions per wave and chunk
  constexpr int kStores = 16;                             // output stores per wave and tile
  static_assert(kDmaW * 4 * 1024 == (int)kChunk && (kDecAhead * kDmaW + kStores) < 64, "wait counts");
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int l32 = lane & 31, hh = lane >> 5;
  const int lin = blockIdx.x, x8 = lin & 7, r = lin >> 3;
  const int split = r % S, h = (r / S) * 8 + x8;
  const int ntile = (T + kMT - 1) / kMT;
  if (h >= H || split >= ntile) return;
  const int nchunks = 4 * ((ntile - split + S - 1) / S);
  // this lane's weight fragments: row 32 wave + l32 of W_v[h] (512 k), k 16j + 8hh .. +7
  bf16x8 bfr[32];
  {
    const __bf16* wrow = B + ((int64_t)h * N + 32 * wave + l32) * K + 8 * hh;
#pragma unroll
    for (int j = 0; j < 32; ++j) bfr[j] = *reinterpret_cast<const bf16x8*>(wrow + 16 * j);
  }
  const i32x4 ra = make_rsrc(reinterpret_cast<uint64_t>(A), (int)((int64_t)T * H * K * 4));
  const i32x4 rnone = make_rsrc(reinterpret_cast<uint64_t>(A), 0);
  const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(C, (short)0, (int)((int64_t)T * H * N * 4),
                                                                      (int)kRsrcWord3);
  auto issue = [&](int g) {
    const uint32_t dst = lds_u32 + (uint32_t)(g % kBufs) * kChunk;
    const int tile = split + S * (g >> 2);
    const uint32_t src = (uint32_t)(((int64_t)kMT * tile * H + h) * K + 128 * (g & 3)) * 4u;
    stage_block(g < nchunks ? ra : rnone, dst, g < nchunks ? src : 0u, (uint32_t)H * K * 4, kMT, 4, tid);
  };
#pragma unroll
  for (int g = 0; g < kDecAhead; ++g) issue(g);
#pragma unroll 1
  for (int tl = 0; tl < nchunks / 4; ++tl) {
    f32x16 acc;
#pragma unroll
    for (int q = 0; q < 16; ++q) acc[q] = 0.f;
#pragma unroll
    for (int c = 0; c < 4; ++c) {   // (unrolled: the weight fragments are indexed by c at compile time)
      const int g = 4 * tl + c;
      issue(g + kDecAhead);
      if (c < kDecAhead && tl > 0) wait_vmcnt<kDecAhead * kDmaW + kStores>();
      else wait_vmcnt<kDecAhead * kDmaW>();
      barrier_lds();
      const uint32_t buf = (uint32_t)(g % kBufs) * kChunk;
#pragma unroll
      for (int j = 0; j < kProjKc / 16; ++j) {
        const int cc = 2 * j + hh;   // bf16 chunk of k 16j + 8hh: fp32 chunks 2cc, 2cc + 1 of the 512-B row
        const f32x4 lo = *(const f32x4 __attribute__((address_space(3)))*)(
            lds + (buf + l32 * 512 + 16 * ((2 * cc) ^ (l32 & 15))));
        const f32x4 hi = *(const f32x4 __attribute__((address_space(3)))*)(
            lds + (buf + l32 * 512 + 16 * ((2 * cc + 1) ^ (l32 & 15))));
        bf16x8 af;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          af[q] = (__bf16)lo[q];
          af[4 + q] = (__bf16)hi[q];
        }
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr[8 * c + j], acc, 0, 0, 0);
      }
      barrier_lds();   // this chunk's buffer is read before it is loaded again
    }
    // acc register q of lane l: row m0 + 8(q/4) + 4(l/32) + q%4, column 32 wave + l%32
    const int m0 = kMT * (split + S * tl);
#pragma unroll
    for (int q = 0; q < 16; ++q) {
      const int m = m0 + 8 * (q >> 2) + 4 * hh + (q & 3);
      const uint32_t off = (uint32_t)(((int64_t)m * H + h) * N + 32 * wave + l32) * 4u;
      // (the value is moved to a plain VGPR first: taken straight from the accumulator vector, the
      // store builtin was compiled to store its first element for every q)
      float v = acc[q];
      asm volatile("" : "+v"(v));
      __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, (int)off, 0, 0);
    }
  }
  // the trailing zero-record DMAs land in LDS before the work-group ends (the last stores may
  // stay in flight)
  wait_vmcnt<kStores>();
}

constexpr int proj_lds_bytes(bool a_float, bool db, int mt) {
  return (db ? 2 : 1) * (kProjBBytes + mt * kProjKc * (a_float ? 4 : 2));
}

// token tiles: 32 for a few tokens (more work-groups), larger ones when the weight block would
// otherwise be staged again for every 32 tokens
template <int kMT>
void absorb_launch(const void* q_nope, const void* q_rope, const void* w_k, int tokens, int heads, void* qz,
                   hipStream_t stream) {
  const int pairs = (kLat / 128) * heads;
  const dim3 grid(((pairs + 7) / 8) * 8 * ((tokens + kMT - 1) / kMT));
  hipLaunchKernelGGL((proj_kernel<false, true, false, kMT>), grid, dim3(kProjThreads), proj_lds_bytes(false, false, kMT),
                     stream, q_nope, static_cast<const __bf16*>(w_k), qz, static_cast<const __bf16*>(q_rope), tokens,
                     heads, kNope, kLat, kDqk);
}

template <int kMT>
hipError_t decompress_launch(const float* out_latent, const void* w_v, int tokens, int heads, float* out,
                             hipStream_t stream) {
  static thread_local int configured = -1;   // the LDS opt-in (two buffers) is per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)proj_kernel<true, false, true, kMT>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            proj_lds_bytes(true, true, kMT));
    if (e != hipSuccess) return e;
    configured = dev;
  }
  const int pairs = heads;
  const dim3 grid(((pairs + 7) / 8) * 8 * ((tokens + kMT - 1) / kMT));
  hipLaunchKernelGGL((proj_kernel<true, false, true, kMT>), grid, dim3(kProjThreads), proj_lds_bytes(true, true, kMT),
                     stream, static_cast<const void*>(out_latent), static_cast<const __bf16*>(w_v),
                     static_cast<void*>(out), static_cast<const __bf16*>(nullptr), tokens, heads, kLat, kDv, kDv);
  return hipSuccess;
}

}  // namespace

hipError_t launch_absorb_query(const void* q_nope, const void* q_rope, const void* w_k, int tokens, int heads,
                               void* qz, hipStream_t stream) {
  if (tokens <= kProjSmallTokens) {
    absorb_launch<32>(q_nope, q_rope, w_k, tokens, heads, qz, stream);
  } else {
    // token shares per (head, column tile): enough work-groups for about four per CU
    constexpr int kMT = kAbsorbTile;
    const int ntile = (tokens + kMT - 1) / kMT;
    const int pairs = 4 * heads;
    int S = (1024 + pairs - 1) / pairs;
    S = S < 1 ? 1 : (S > ntile ? ntile : S);
    const dim3 grid(8 * 4 * S * ((heads + 7) / 8));
    hipLaunchKernelGGL(absorb_tiles_kernel<kMT>, grid, dim3(kProjThreads), 2 * kMT * 256, stream,
                       static_cast<const __bf16*>(q_nope), static_cast<const __bf16*>(w_k), static_cast<__bf16*>(qz),
                       static_cast<const __bf16*>(q_rope), tokens, heads, S);
  }
  return hipGetLastError();
}

hipError_t launch_decompress_output(const float* out_latent, const void* w_v, int tokens, int heads, float* out,
                                    hipStream_t stream) {
  // token shares per head for decompress_tiles_kernel: enough work-groups for about two per CU;
  // that kernel only pays when every work-group walks at least two tiles (each loads its head's
  // 128 KiB of weights once)
  const int ntile = (tokens + 31) / 32;
  const int S = (512 + heads - 1) / heads;
  if (tokens <= kProjSmallTokens) {
    const hipError_t e = decompress_launch<32>(out_latent, w_v, tokens, heads, out, stream);
    if (e != hipSuccess) return e;
  } else if (ntile < 2 * S) {
    const hipError_t e = decompress_launch<64>(out_latent, w_v, tokens, heads, out, stream);
    if (e != hipSuccess) return e;
  } else {
    const dim3 grid(8 * S * ((heads + 7) / 8));
    hipLaunchKernelGGL(decompress_tiles_kernel, grid, dim3(kProjThreads), (kDecAhead + 1) * 32 * kProjKc * 4, stream,
                       out_latent, static_cast<const __bf16*>(w_v), out, tokens, heads, S);
  }
  return hipGetLastError();
}

}  // namespace mla
