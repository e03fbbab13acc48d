// Latent-space MLA decode over a bf16 cache: one persistent work-group of four waves (one per
// SIMD) per compute unit; each wave owns the softmax of 32 query rows of the 128-row tile and
// the values of a quarter of the 512 latent channels.
//
// Page "Mla Analysis", section "Absorption Trick (FlashMLA)": scores are Qz . Z^T with the
// absorbed 576-wide queries and the value is the latent row itself, so one pass over the
// paged latent cache gives O_latent = softmax(scale Qz Z^T) Z[:, :512] and a log-sum-exp per
// (token, head). Section "Cost Models": at s=1 this is about 228 FLOP per byte, under the
// MI355X bf16 ridge, so the kernel streams every cached row from HBM once per 128-row tile
// and keeps the matrix cores busy underneath.
//
// Per 32-token step, per wave w:
//  * Scores S^T[32 tokens x 32 rows] = Z Q^T for the wave's rows 32w .. 32w+31: 36
//    v_mfma_f32_32x32x16_bf16 over the 576 channels; A = Z rows from LDS (ds_read_b128),
//    B = Q^T held in 144 VGPRs.
//  * The 32x32 accumulator layout (lane: row l%32, tokens 8j + 4(l/32) + v) is, after the
//    bf16 rounding, exactly an MFMA operand of P[32 rows x 16 tokens] when the 16 k slots
//    of k-step q are taken as tokens 16q + 8(i/4) + 4(l/32) + i%4, and the softmax state of
//    a row (reference max, sum) is lane-local (lanes l and l^32 share a row and combine with
//    a permlane32 swap).
//  * Values: the wave accumulates O[all 128 rows x its 128 channels 128w ..] += P Z, 32
//    v_mfma_f32_32x32x16_bf16 into the 256 AGPRs. A = P of each row block: the wave's own
//    from registers, the other three waves' from a double-buffered P area in LDS (each wave
//    writes its P there in the A-operand layout, 2 KiB per step); B = Z^T tiles of the
//    wave's channels, two ds_read_b64_tr_b16 each. Splitting the channels rather than the
//    rows reads each Z^T tile once per work-group instead of once per wave.
//  * The reference max of a row is set at its first finite score and never moves, so O is
//    never rescaled inside the loop (a rare redo of the segment covers rows whose scores
//    later run far above it).
//  * LDS ring of 4 steps (36 KiB each) filled by LDS-DMA (buffer_load_dwordx4 ... lds, 9 per
//    wave and step, source offsets from three packed per-lane words), rows XOR-swizzled in
//    16-B chunks so that both operand reads are free of bank conflicts. The ring and the two
//    P buffers fill the 160 KiB. One barrier per step: it publishes the next step's rows and
//    every wave's P, and frees the slot and the P buffer the previous step read.
//  * Order inside a step: the first value MFMAs of step i (own rows, operands in registers),
//    the score MFMAs of step i+1 (the step's DMA instructions between them), the remaining
//    value MFMAs of step i with the softmax of step i+1 (VALU) between them, P of step i+1 to
//    LDS.
//  * The MFMAs are written as inline asm so that O can be pinned to AGPRs while the score
//    accumulator stays in VGPRs; explicit waits (12+ states) precede every VALU read of an
//    MFMA result.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kR32Threads = 256;                 // 4 waves, one per SIMD
constexpr int kR32Slots = 4;                     // LDS ring depth (steps)
constexpr int kR32Dma = kDmaInstr / 4;           // 9 LDS-DMA instructions per wave and step
constexpr int kR32LdsBytes = kR32Slots * kBufBytes;   // the ring; then two P buffers
constexpr int kR32PBytes = kRowsPerTile * kStep * 2;  // P of one step: 128 rows x 32 tokens, bf16
constexpr int kR32PBase = kR32LdsBytes;
constexpr int kR32PvLead = 4;                    // value MFMAs of step i before the scores of step i+1
constexpr int kR32QkRing = 4;                    // score operand reads in flight
constexpr int kF8QkRing = 3;                     // (fp8 cache)
constexpr int kR32LdsTotal = kR32PBase + 2 * kR32PBytes;
static_assert(kR32LdsTotal <= 160 * 1024, "LDS budget");
// fp8 cache: two slots of dequantised steps (bf16, the ring layout above), three staging
// slots of raw steps as loaded, then the two P buffers.
constexpr int kR8Bf16Slots = 2;
constexpr int kR8Stage = 3;
constexpr int kR8StRope = kStep * kLat;                      // codes: 32 rows of 512 B
constexpr int kR8StScales = kR8StRope + kStep * 2 * kRope;   // rope: 32 rows of 128 B
constexpr int kR8StBytes = kR8StScales + 1024;               // scales: 32 x 16 B (+ 512 B of zeros)
constexpr int kR8StBase = kR8Bf16Slots * kBufBytes;
constexpr int kR8PBase = kR8StBase + kR8Stage * kR8StBytes;
constexpr int kR8QBase = kR8PBase + 2 * kR32PBytes;         // Q^T k-steps 34, 35 (2 KiB per wave)
constexpr int kR8LdsTotal = kR8QBase + 4 * 2048;
static_assert(kR8LdsTotal <= 160 * 1024, "LDS budget (fp8)");
static_assert(kR8LdsTotal >= kR32Slots * kBufBytes, "the query rows are staged through LDS at start-up");
// token-sparse fp8: a ring of 4 x 32 cache-row numbers (one per step; 256 B per slot) in the
// last KiB
constexpr int kR8RowRing = kR8LdsTotal;
constexpr int kR8SparseLdsTotal = kR8RowRing + 4 * 256;
static_assert(kR8SparseLdsTotal <= 160 * 1024, "LDS budget (token-sparse fp8)");
static_assert(kR8StBase % 128 == 0 && kR8StBytes % 128 == 0 && kBufBytes % 128 == 0,
              "slot offsets leave the low 7 address bits to the lane's swizzle");
constexpr float kWindow = 64.f;                  // rows may exceed their reference max by 2^64
static_assert(kDmaInstr % 4 == 0, "DMA split");
static_assert(32 - kR32PvLead >= 23, "softmax pieces fit between the value MFMAs");

// 16-B chunk swizzle within 8-chunk groups: physical = logical ^ sw(token). Over 16
// consecutive tokens of one parity sw is a permutation of 0..7 (conflict-free score reads of
// 16 tokens x one chunk), and sw(t) ^ sw(t+2) = 4 for t = 0, 1 mod 4 (conflict-free
// transposing reads of 4 consecutive tokens x 4 chunks).
__device__ __forceinline__ uint32_t sw32(uint32_t u) { return (((u >> 1) & 1u) << 2) | ((u >> 2) & 3u); }

// Source offset (bytes from the step's first row) of LDS-DMA instruction i = wave + 4n,
// lane l: it fills LDS chunk position p = 64i + l = 72u + pc (token u = floor(p / 72)),
// which holds logical chunk pc ^ sw(u) of token u, i.e. source byte 1152u + 16 (pc ^ sw(u))
// = 16 (p ^ sw(u)) (72u has no low bits). With p = 256n + b, b = 64 wave + l < 256, that is
// 4096n + (16b ^ 16 sw(u)). Per lane the nine 16 sw(u) (7 bits each) are packed into three
// words once; an instruction's offset is then one field extract and one xor-add. (All of it
// stays in the vector offset: the buffer's range check, which zero-fills rows past the
// visible ones, does not cover the scalar offset.)
struct DmaOffsets { uint32_t b16, packed[3]; };
__device__ __forceinline__ DmaOffsets dma_offsets(int wave, int lane) {
  DmaOffsets d;
  const uint32_t b = 64u * (uint32_t)wave + (uint32_t)lane;
  d.b16 = 16u * b;
  d.packed[0] = d.packed[1] = d.packed[2] = 0u;
#pragma unroll
  for (int n = 0; n < kDmaInstr / 4; ++n) {
    const uint32_t u = (256u * (uint32_t)n + b) / 72u;
    d.packed[n >> 2] |= (sw32(u) << 4) << (7 * (n & 3));
  }
  return d;
}
__device__ __forceinline__ uint32_t dma_voff(const DmaOffsets& d, int n) {
  return (__builtin_amdgcn_ubfe(d.packed[n >> 2], 7 * (n & 3), 7) ^ d.b16) + 4096u * (uint32_t)n;
}
__device__ __forceinline__ void issue32(const i32x4& rsrc, uint32_t lds_slot, int n, uint32_t voff, int wave) {
  lds_dma_x4(lds_slot + 1024u * (uint32_t)(wave + 4 * n), voff, rsrc);
}
// the same for cache rows (read once: non-temporal)
__device__ __forceinline__ void issue32_rows(const i32x4& rsrc, uint32_t lds_slot, int n, uint32_t voff, int wave) {
  lds_dma_x4_stream(lds_slot + 1024u * (uint32_t)(wave + 4 * n), voff, rsrc);
}

// fp8 staging slot of one step, filled by 21 LDS-DMA instructions:
//  * codes: token u's 512 codes at 512u, its 32-B pieces (32 channels) permuted within each
//    256-B half by piece ^ (u % 8), so that the dequantisation's reads of 8 tokens x one
//    32-channel piece cover all 64 banks. Instruction n (1 KiB: tokens 2n, 2n+1) is issued
//    by wave n % 4, so a lane's permutation is the same for all its instructions and
//    instruction n = wave + 4m reads at base + 8 * 640 m.
//  * rope: token u's 128 B at 16384 + 128u, one instruction per wave (8 tokens);
//  * scales: 32 x 4 floats at 20480, one instruction by wave 0 (lanes 32.. read past the
//    range and write zeros after them).
// The (token, byte) -> (LDS position) map is a permutation of 16-B units, so every source
// byte lands once.
struct F8Dma { uint32_t codes, rope, scales; };
__device__ __forceinline__ F8Dma f8_dma_offsets(int wave, int lane) {
  const uint32_t l = (uint32_t)lane, u0 = 2u * (uint32_t)wave + (l >> 5);
  F8Dma d;
  d.codes = u0 * kF8Row + 16u * ((l & 31u) ^ (2u * (u0 & 7u)));
  d.rope = (8u * (uint32_t)wave + (l >> 3)) * kF8Row + kLat + 16u * (l & 7u);
  d.scales = l < 32u ? 16u * l : 0x40000000u;
  return d;
}
// Four e4m3fn codes (one word, channel order) times their tile's scale: the fp32 product
// rounded to bf16.
__device__ __forceinline__ bf16x4 dequant4(uint32_t w, float sc) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
  bf16x4 r;
  r[0] = (__bf16)(lo[0] * sc);
  r[1] = (__bf16)(lo[1] * sc);
  r[2] = (__bf16)(hi[0] * sc);
  r[3] = (__bf16)(hi[1] * sc);
  return r;
}
// s_waitcnt for the fp8 DMA steps: wave 0 issues 6 instructions per step (the scales), wave 1
// 6 on a token-sparse cache (the next row numbers), the others 5
template <int kSteps, bool kSparse>
__device__ __forceinline__ void wait_f8_steps(int wave) {
  if (wave == 0 || (kSparse && wave == 1)) wait_vmcnt<6 * kSteps>();
  else wait_vmcnt<5 * kSteps>();
}

// v_mfma_f32_32x32x16_bf16 with the accumulator in VGPRs (scores) or AGPRs (values). A VALU
// write of an operand needs two wait states before an MFMA reads it: the operands here come
// from LDS/global loads, or (P, the zeroed accumulators) are written by VALU many
// instructions before their first MFMA.
__device__ __forceinline__ void mfma_v0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_v(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a0(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&a"(d) : "v"(a), "v"(b));
}
__device__ __forceinline__ void mfma_a(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// An MFMA result may be read by VALU (or v_accvgpr_read) only 12 wait states after the
// MFMA; 18 here.
__device__ __forceinline__ void mfma_result_wait(f32x16& s) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" : "+v"(s));
}
// Before the accumulator tiles are read (finalize): 18 wait states after the last MFMA. A
// plain asm statement plus a scheduling barrier, so that the compiler's AGPR reads stay
// behind it and are made per use (an asm with the tiles as operands would make it copy all
// 256 AGPRs to VGPRs at once).
__device__ __forceinline__ void mfma_results_settle() {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 1" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float max_across_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_halves(float x) {
  const unsigned u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane LDS byte addresses of the operand reads of one ring slot: the lane's part is
// computed once (8 VGPRs held across the loop) and the slot offset added per use; the
// tile's part goes into the instructions' offset field.
// scores: lane reads token l%32, logical chunk 2ks + l/32 -> b[ks % 4] + 128 (ks / 4)
struct QkAddr { uint32_t b[4]; };
__device__ __forceinline__ QkAddr qk_addr(uint32_t zoff, int lane) {
  const int l = lane;
  const uint32_t T = l & 31, h = l >> 5;
  QkAddr r;
#pragma unroll
  for (int x = 0; x < 4; ++x) r.b[x] = zoff + T * kRowBytes + 16 * ((2 * x + h) ^ sw32(T));
  return r;
}
__device__ __forceinline__ QkAddr qk_at(const QkAddr& base, uint32_t zoff) {
  QkAddr r;
#pragma unroll
  for (int x = 0; x < 4; ++x) r.b[x] = base.b[x] + zoff;
  return r;
}
// values: lane (G = l/16, j = l%16) reads token 16q + 8e + 4(G/2) + j/4, channels
// 32c + 16(G%2) + 4(j%4) .. +3 -> b[e][c % 2] + 16q rows + 128 (c / 2)
struct PvAddr { uint32_t b[2][2]; };
__device__ __forceinline__ PvAddr pv_addr(uint32_t zoff, int lane) {
  const int l = lane;
  const uint32_t G = l >> 4, j = l & 15;
  PvAddr r;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1)
      r.b[e][c1] = zoff + (8 * e + 4 * (G >> 1) + (j >> 2)) * kRowBytes +
                   16 * ((4 * c1 + 2 * (G & 1) + ((j >> 1) & 1)) ^ (4 * (j >> 3) + 2 * e + (G >> 1))) + 8 * (j & 1);
  return r;
}
__device__ __forceinline__ PvAddr pv_at(const PvAddr& base, uint32_t zoff) {
  PvAddr r;
#pragma unroll
  for (int e = 0; e < 2; ++e)
#pragma unroll
    for (int c1 = 0; c1 < 2; ++c1) r.b[e][c1] = base.b[e][c1] + zoff;
  return r;
}

template <bool kFp8, bool kSparse>
__global__ __launch_bounds__(kR32Threads, 1) void decode_rows32_kernel(
    const __bf16* __restrict__ q_ptr, const char* __restrict__ kv_ptr, const float* __restrict__ kv_scales,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ plan, float* __restrict__ ws,
    float* __restrict__ out_ptr, float* __restrict__ lse_ptr, const int32_t* __restrict__ srows, int srow_stride,
    int32_t* __restrict__ status, Scalars a) {
  static_assert(kFp8 || !kSparse, "the token-sparse path reads an fp8 cache");
  constexpr int kPBase = kFp8 ? kR8PBase : kR32PBase;   // P buffers; votes and 1/l after the loop
  constexpr int kLoadSlots = kFp8 ? kR8Stage : kR32Slots;
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = xcd_worker();
  // device-side precondition violations of this work-group, reported once at the end
  int dev_err = 0;
  auto report = [&]() {
    if (status != nullptr && dev_err != 0 && threadIdx.x == 0)
      __hip_atomic_fetch_or(status, dev_err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };
  const int n_items = a.batch * tiles_per_seq(a.s_q, a.heads);
  if (!plan_header_matches(load_plan_header(plan), a.batch, a.s_q, a.heads, a.causal, (int)gridDim.x, n_items)) {
    dev_err = kDevPlanMismatch;
    report();
    return;
  }
  const int32_t* wr = plan + plan_workers_off(n_items) + kWorkerWords * worker;
  const int kb = wr[0], pb = wr[1], ke = wr[2], pe = wr[3];
  int k_last = pe > 0 ? ke : ke - 1;
  k_last = k_last < n_items - 1 ? k_last : n_items - 1;
  if (kb >= n_items || k_last < kb) return;
  const int rows_total = a.s_q * a.heads;
  const QkAddr qk0 = qk_addr(0, lane);                        // operand addresses in slot 0
  const PvAddr pv0 = pv_addr(256u * (uint32_t)wave, lane);    // (this wave's 128 channels)
  const uint32_t plane = (uint32_t)kPBase + 16u * (uint32_t)lane;   // P tiles: 16 B per lane
  // fp8: Q^T k-step ks (34, 35) of this lane in LDS
  auto q_lds_addr = [&](int ks) -> uint32_t {
    return (uint32_t)kR8QBase + 2048u * (uint32_t)wave + 1024u * (uint32_t)(ks - 34) + 16u * (uint32_t)lane;
  };
  auto q_lds = [&](int ks) -> bf16x8 { return lds_b128(lds + q_lds_addr(ks)); };

  // Q^T B operand of item k: lane holds query row 32*wave + l%32 of the item's tile, channels
  // 16ks + 8(l/32) .. +7. Rows past the last query row (a partial tile) load the sequence's
  // first row: every output column depends on its own row only, and no such row is written.
  bf16x8 qreg[36];
  auto load_q = [&](int k) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int32_t* it = plan + plan_items_off() + kItemWords * k;
    const int g_row = kRowsPerTile * it[kITile] + 32 * wave + (l & 31);
    const bool ok = g_row < rows_total;
    const int jt = ok ? g_row / a.heads : 0;
    const int hd = ok ? g_row - jt * a.heads : 0;
    const __bf16* qrow = q_ptr + ((int64_t)(it[kISeq] * a.s_q + jt) * a.heads + hd) * kDqk + 8 * (l >> 5);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + 16 * ks);
  };
  // ---- load cursor: the first kR32Slots-1 steps are issued up front, then one step per
  // compute region (its DMA instructions spread between the score MFMAs)
  LoadCursor lc;
  auto settle_c = [&](LoadCursor& c) {
    while (c.k <= k_last && c.hh >= c.hh1) {
      if (c.k == k_last) {
        c.k = k_last + 1;
        break;
      }
      cursor_enter(c, plan, c.k + 1, kb, pb, ke, pe);
    }
  };
  auto restart = [&](LoadCursor& c, int k) {
    cursor_enter(c, plan, k, kb, pb, ke, pe);
    settle_c(c);
    if (!kSparse && c.k <= k_last) cursor_fetch(c, a, block_table);
  };
  restart(lc, kb);
  int load_slot = 0;   // ring slot (bf16) or staging slot (fp8) of the cursor's step
  // token-sparse: a second cursor two steps ahead loads each step's 32 cache-row numbers
  // (stored + 1; 0 = none) into the row ring; row_slot is the ring slot of lc's step
  LoadCursor pc;
  int row_slot = 0;
  if constexpr (kSparse) restart(pc, kb);
  auto advance = [&]() {
    load_slot = load_slot + 1 == kLoadSlots ? 0 : load_slot + 1;
    ++lc.hh;
    settle_c(lc);
    if (!kSparse && lc.k <= k_last) cursor_fetch(lc, a, block_table);
    if constexpr (kSparse) row_slot = (row_slot + 1) & 3;
  };
  auto advance_pc = [&]() {
    ++pc.hh;
    settle_c(pc);
  };
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
  const DmaOffsets dmo = dma_offsets(wave, lane);   // this wave's DMA source offsets
  // descriptors of the cursor's step (zero-record loads past the worker's range)
  auto step_rsrc = [&]() -> StepRsrc {
    StepRsrc z;
    if (lc.k <= k_last) {
      if constexpr (kSparse) {   // the whole cache (its size is checked below 2^31 on the host)
        z.kv = make_rsrc(reinterpret_cast<uint64_t>(kv_ptr), (int)(a.num_pages * (kPage * kF8Row)));
        z.sc = make_rsrc(reinterpret_cast<uint64_t>(kv_scales), (int)(a.num_pages * (kPage * 16)));
        return z;
      } else {
        return cursor_rsrc<kFp8>(lc, a, kv_ptr, kv_scales, dev_err);
      }
    }
    z.kv = z.sc = make_rsrc(reinterpret_cast<uint64_t>(kv_ptr), 0);
    return z;
  };
  // token-sparse: the row numbers of pc's step into row ring slot rs_slot (wave 1; lanes 32..63
  // read on into the slot's second half or past the list, harmlessly)
  auto dma_rows = [&](int rs_slot) {
    if constexpr (kSparse) {
      if (wave == 1) {
        const i32x4 r = pc.k <= k_last ? make_rsrc(reinterpret_cast<uint64_t>(srows) +
                                                        (uint64_t)pc.seq * (uint64_t)srow_stride * 4u,
                                                    srow_stride * 4)
                                       : make_rsrc(reinterpret_cast<uint64_t>(srows), 0);
        lds_dma_x1(lds_u32 + kR8RowRing + 256u * (uint32_t)rs_slot, 4u * (32u * (uint32_t)pc.hh + (uint32_t)lane), r);
      }
      advance_pc();
    }
  };
  // fp8: this lane's DMA source offsets and its addresses for dequantising (token
  // 16 half + l/4, channels 128 wave + 32c + 8(l%4) .. +7 of piece c: the staging read, where
  // XOR 32c selects the piece; the bf16 slot write, where XOR 64 (c%2) plus 128 (c/2) does;
  // the scale) and for copying the rope (token 8 wave + l/8, 16 B), packed two 16-bit
  // offsets per register
  uint32_t f8_dma = 0, f8_dq = 0, f8_aux = 0;
  if constexpr (kFp8) {
    const uint32_t l = (uint32_t)lane, u = l >> 2, sub = l & 3u, ur = 8u * (uint32_t)wave + (l >> 3);
    const F8Dma d = f8_dma_offsets(wave, lane);
    // (token-sparse: the offsets within the lane's row; the row comes from the row ring)
    const uint32_t u0 = 2u * (uint32_t)wave + (l >> 5);
    f8_dma = kSparse ? (d.codes - u0 * kF8Row) | ((d.rope - ur * kF8Row) << 16) : d.codes | (d.rope << 16);
    f8_dq = (u * kLat + ((128u * (uint32_t)wave + 8u * sub) ^ (32u * (u & 7u)))) |
            ((u * kRowBytes + 256u * (uint32_t)wave + 16u * (sub ^ sw32(u))) << 16);
    f8_aux = (kR8StScales + 16u * u + 4u * (uint32_t)wave) | ((ur * kRowBytes + 16u * (64u + ((l & 7u) ^ sw32(ur)))) << 16);
    static_assert(kR8StBytes < 65536 && 16 * kRowBytes < 65536 && kBufBytes < 65536, "16-bit offsets");
  }
  // token-sparse: the stored row number (+1; 0 = none) of the token this lane loads with fp8
  // instruction j of lc's step (codes: token 8j + 2 wave + l/32; rope: 8 wave + l/8; scales: l)
  auto f8_row = [&](int j) -> uint32_t {
    const uint32_t tok = j < 4 ? 8u * (uint32_t)j + 2u * (uint32_t)wave + ((uint32_t)lane >> 5)
                               : (j == 4 ? 8u * (uint32_t)wave + ((uint32_t)lane >> 3) : ((uint32_t)lane & 31u));
    return *(const uint32_t __attribute__((address_space(3)))*)(lds + (kR8RowRing + 256u * (uint32_t)row_slot + 4u * tok));
  };
  // one step's DMA instructions into staging slot st (LDS address); fp8 instruction j of
  // this wave (0..3 codes, 4 rope, 5 scales on wave 0); sv: f8_row(j) on a token-sparse
  // cache (a row of none reads past the range: zeros)
  auto dma_f8 = [&](const StepRsrc& rs, uint32_t st, int j, uint32_t sv) {
    if constexpr (kSparse) {
      const uint32_t none = 0xFFFFFFF0u;
      if (j < 4) {
        lds_dma_x4_stream(st + 1024u * (uint32_t)(wave + 4 * j), sv ? (sv - 1u) * kF8Row + (f8_dma & 0xFFFFu) : none, rs.kv);
      } else if (j == 4) {
        lds_dma_x4_stream(st + kR8StRope + 1024u * (uint32_t)wave, sv ? (sv - 1u) * kF8Row + (f8_dma >> 16) : none, rs.kv);
      } else if (wave == 0) {
        lds_dma_x4(st + kR8StScales, (sv && lane < 32) ? (sv - 1u) * 16u : none, rs.sc);
      }
    } else {
      if (j < 4) {
        lds_dma_x4_stream(st + 1024u * (uint32_t)(wave + 4 * j), (f8_dma & 0xFFFFu) + 8u * kF8Row * (uint32_t)j, rs.kv);
      } else if (j == 4) {
        lds_dma_x4_stream(st + kR8StRope + 1024u * (uint32_t)wave, f8_dma >> 16, rs.kv);
      } else if (wave == 0) {
        lds_dma_x4(st + kR8StScales, lane < 32 ? 16u * (uint32_t)lane : 0x40000000u, rs.sc);
      }
    }
  };
  auto issue_step = [&]() {
    const StepRsrc rs = step_rsrc();
    if constexpr (kFp8) {
      const uint32_t st = lds_u32 + kR8StBase + (uint32_t)load_slot * kR8StBytes;
#pragma unroll
      for (int j = 0; j < 6; ++j) dma_f8(rs, st, j, kSparse ? f8_row(j) : 0u);
    } else {
#pragma unroll
      for (int n = 0; n < kR32Dma; ++n) issue32_rows(rs.kv, lds_u32 + load_slot * kBufBytes, n, dma_voff(dmo, n), wave);
    }
    advance();
  };
  // fp8 dequantisation of half h (tokens 16h .. 16h+15) of staging slot st into bf16 slot bs
  // (LDS byte offsets): the lane's read and write bases, then per piece c
  struct F8Half { uint32_t rd, wr; };
  auto f8_half = [&](uint32_t st, uint32_t bs, int h) -> F8Half {
    F8Half b;
    b.rd = st + (f8_dq & 0xFFFFu) + (uint32_t)h * 16u * kLat;
    b.wr = bs + (f8_dq >> 16) + (uint32_t)h * 16u * kRowBytes;
    return b;
  };
  auto f8_scale = [&](uint32_t st, int h) -> float {
    return *(const float __attribute__((address_space(3)))*)(lds + (st + (f8_aux & 0xFFFFu) + 256u * (uint32_t)h));
  };
  auto f8_codes = [&](const F8Half& b, int c) -> u32x2 {
    return *(const u32x2 __attribute__((address_space(3)))*)(lds + (b.rd ^ (32u * (uint32_t)c)));
  };
  auto f8_store = [&](const F8Half& b, int c, bf16x4 lo, bf16x4 hi) {
    *(bf16x8 __attribute__((address_space(3)))*)(lds + ((b.wr ^ (64u * (uint32_t)(c & 1))) + 128u * (uint32_t)(c >> 1))) =
        __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
  };
  auto f8_rope = [&](uint32_t st) -> u32x4 {
    return *(const u32x4 __attribute__((address_space(3)))*)(lds + (st + kR8StRope + 1024u * (uint32_t)wave +
                                                                     16u * (uint32_t)lane));
  };
  auto f8_rope_store = [&](uint32_t bs, u32x4 v) {
    *(u32x4 __attribute__((address_space(3)))*)(lds + (bs + (f8_aux >> 16))) = v;
  };
  // a whole step (start-up and redo passes only)
  auto f8_dequant_step = [&](uint32_t st, uint32_t bs) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const float sc = f8_scale(st, h);
      const F8Half b = f8_half(st, bs, h);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const u32x2 w = f8_codes(b, c);
        f8_store(b, c, dequant4(w[0], sc), dequant4(w[1], sc));
      }
    }
    f8_rope_store(bs, f8_rope(st));
  };
  // fp8: fill the pipeline from the cursor's step g0 in an empty ring: staging 0, 1, 2 <-
  // steps g0 .. g0+2, bf16 slots 0, 1 <- steps g0, g0+1 dequantised, staging 0 <- step g0+3
  // (in flight); on return every slot is visible and the next step loads into staging 1.
  // That is the state every step region starts from: region i computes the values of step i
  // and the scores of step i+1, dequantises step i+2 (staging slot) into the bf16 slot of
  // step i, and loads step i+4.
  // Token-sparse: first the row numbers of steps g0 .. g0+3 (row ring slots 0..3), and of
  // g0+4, g0+5 into slots 0, 1 once the loads of g0, g0+1 have read them; afterwards row_slot
  // is 0 (step g0+4) and region i loads the rows of step i+6 into the slot two ahead.
  auto f8_fill = [&](bool rows_loaded) {
    if constexpr (kSparse) {
      if (!rows_loaded) {
#pragma unroll 1
        for (int r = 0; r < 4; ++r) dma_rows(r);
      }
      wait_vmcnt<0>();
      barrier_lds();
      issue_step();
      issue_step();
      barrier_lds();   // every wave has read ring slots 0, 1
      dma_rows(0);
      dma_rows(1);
      issue_step();
      wait_vmcnt<0>();
      barrier_lds();
      f8_dequant_step(kR8StBase, 0);
      barrier_lds();   // staging slot 0 read by every wave
      issue_step();
      f8_dequant_step(kR8StBase + kR8StBytes, kBufBytes);
      wait_f8_steps<1, true>(wave);
      barrier_lds();
    } else {
      issue_step();
      issue_step();
      issue_step();
      wait_f8_steps<2, false>(wave);
      barrier_lds();
      f8_dequant_step(kR8StBase, 0);
      wait_f8_steps<1, false>(wave);
      barrier_lds();
      issue_step();
      f8_dequant_step(kR8StBase + kR8StBytes, kBufBytes);
      wait_f8_steps<1, false>(wave);
      barrier_lds();
    }
  };
  // token-sparse: the row numbers of the first four steps go first (the row ring lies outside
  // the area the queries are staged through), so that their latency hides under the staging
  if constexpr (kSparse) {
#pragma unroll 1
    for (int r = 0; r < 4; ++r) dma_rows(r);
  }
  int comp_slot = 0;   // ring slot of the segment's current step
  // Start-up, for the first item. Its query rows are staged through LDS by LDS-DMA, 32 rows
  // per ring slot in the cache-step layout, and each wave reads its 32 rows back with the
  // score-operand read pattern; rows past the last query row read as zeros. (Loaded straight
  // into registers, each load instruction touches 32 rows; with every worker starting at
  // once, that burst is bound by the number of cache lines.)
  //  * bf16 cache: the rows of waves 0..2 go through slots 0..2 while the first ring step is
  //    already loading into slot 3 (the ring starts there), and wave 3 loads its 32 rows into
  //    registers; then the next two ring steps go into slots 0 and 1.
  //  * fp8 cache: all four waves' rows through the four slots, then the fp8 pipeline fill.
  auto start_up = [&]() {
    const int32_t* it = plan + plan_items_off() + kItemWords * kb;
    const int tile0 = kRowsPerTile * it[kITile];
    const int valid_rows = rows_total - tile0 < kRowsPerTile ? rows_total - tile0 : kRowsPerTile;
    const uint64_t qbase = reinterpret_cast<uint64_t>(q_ptr) +
                           ((uint64_t)it[kISeq] * (uint64_t)rows_total + (uint64_t)tile0) * kRowBytes;
    constexpr int kStaged = kFp8 ? kR32Slots : kR32Slots - 1;   // slots (waves) staged by DMA
#pragma unroll 1
    for (int sl = 0; sl < kStaged; ++sl) {
      int bytes = valid_rows * kRowBytes - sl * kBufBytes;
      bytes = bytes < 0 ? 0 : (bytes > kBufBytes ? kBufBytes : bytes);
      const i32x4 rs = make_rsrc(qbase + (uint64_t)sl * kBufBytes, bytes);
#pragma unroll
      for (int n = 0; n < kR32Dma; ++n) issue32(rs, lds_u32 + sl * kBufBytes, n, dma_voff(dmo, n), wave);
    }
    if constexpr (!kFp8) {
      load_slot = kR32Slots - 1;   // the first ring step into the free slot
      comp_slot = kR32Slots - 1;
      issue_step();
      wait_vmcnt<kR32Dma>();       // this wave's staging DMA done (the ring step may stay in flight)
    } else {
      wait_vmcnt<0>();
    }
    barrier_lds();
    if (kFp8 || wave < kStaged) {
      const QkAddr qa = qk_at(qk0, (uint32_t)wave * kBufBytes);
#pragma unroll
      for (int ks = 0; ks < 36; ++ks) qreg[ks] = lds_b128(lds + (qa.b[ks & 3] + 128 * (ks >> 2)));
    } else {
      // (bf16) the last wave's rows straight into registers: the compiler waits for these
      // loads at their first use
      load_q(kb);
    }
    barrier_lds();   // every wave holds its rows before the ring is refilled
    if constexpr (kFp8) {
      f8_fill(true);
    } else {
#pragma unroll 1
      for (int i = 0; i < kR32Slots - 2; ++i) issue_step();
    }
  };

#pragma unroll 1
  for (int k = kb; k <= k_last; ++k) {
    const Seg sg = seg_of(plan, k, kb, pb, ke, pe);
    const int32_t* it = plan + plan_items_off() + kItemWords * k;

    // ---- keys visible to this lane's query row 32*wave + l%32, from the item's visible count
    // (that of its last row; the plan holds it, so no length load sits on the item's start):
    // row j of a causal tile sees j_last - j keys fewer; lengths above the block table's
    // capacity read as that capacity
    int lim = 0;
    int lim_min;   // smallest count over the wave's valid rows: steps below it need no mask
    {
      const int tile_row0 = kRowsPerTile * it[kITile];
      const int g_row = tile_row0 + 32 * wave + (lane & 31);
      if (it[kIVis] > a.max_pages * kPage) dev_err |= kDevLengthOverCap;
      if (g_row < rows_total) {
        const int vis = it[kIVis];
        const int cap = a.max_pages * kPage;
        if (a.causal) {
          const int last_row = (tile_row0 + kRowsPerTile < rows_total ? tile_row0 + kRowsPerTile : rows_total) - 1;
          const int jt = g_row / a.heads, jt_last = last_row / a.heads;
          int lv = vis > 0 ? vis - (jt_last - jt) : 0;
          lv = lv < 0 ? 0 : lv;
          int lc = cap - a.s_q + 1 + jt;
          lc = lc < 0 ? 0 : lc;
          lim = lv < lc ? lv : lc;
        } else {
          lim = vis < cap ? vis : cap;
        }
      }
      int m = g_row < rows_total ? lim : 0x7FFFFFFF;
#pragma unroll
      for (int d = 1; d < 64; d <<= 1) {
        const int y = __shfl_xor(m, d, 64);
        m = y < m ? y : m;
      }
      lim_min = __builtin_amdgcn_readfirstlane(m);
    }
    // this item's query rows: the first item's staged at start-up (which then issues the first
    // ring steps), the others loaded into registers (no DMA step is issued between the previous
    // item's last steps and these loads, so they are the youngest loads in flight and waiting
    // for them at their first use leaves no ring step behind). Defined on every path here, the
    // rows of the previous item are dead through its finalize.
    if (k == kb) start_up();
    else load_q(k);
    if constexpr (kFp8) {
      // Q^T k-steps 34, 35 of the item to LDS (this wave's area; the score loops read them
      // back there, which frees 8 VGPRs in the step loop)
      *(bf16x8 __attribute__((address_space(3)))*)(lds + q_lds_addr(34)) = qreg[34];
      *(bf16x8 __attribute__((address_space(3)))*)(lds + q_lds_addr(35)) = qreg[35];
    }

    f32x16 o[16];
    float m_run = -INFINITY;   // reference max of the row (log2 domain, integer-valued once set)
    float m_seen = -INFINITY;  // largest row max seen in the segment
    float l_run = 0.f;
    bool window_exceeded = false;
    const int nsteps = sg.hh1 - sg.hh0;

    // ---- pipeline pieces
    // score operand t (k-step t)
    auto qk_read = [&](const QkAddr& ad, int t) -> bf16x8 {
      return lds_b128(lds + (ad.b[t & 3] + 128 * (t >> 2)));
    };
    // value operand t = 16q + c: Z^T[channels 32c ..][16 tokens of k-step q]
    auto pv_read = [&](const PvAddr& ad, int t) -> bf16x8 {
      const int q = t >> 4, c = t & 15;
      const bf16x4 lo = lds_tr16(lds + (ad.b[0][c & 1] + q * 16 * kRowBytes + 128 * (c >> 1)));
      const bf16x4 hi = lds_tr16(lds + (ad.b[1][c & 1] + q * 16 * kRowBytes + 128 * (c >> 1)));
      return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    };
    // Softmax of the scores s of step hh in small pieces, each about one MFMA's worth of
    // VALU, so that they can sit between the value MFMAs. The row's reference max is fixed
    // at its first finite score (rounded up to an integer) and never moves afterwards, so O
    // is never rescaled: P = 2^(s - ref) stays below 2^64 while the row max stays within
    // kWindow of the reference (no overflow in fp32 for any realistic length and magnitude);
    // a row that leaves the window marks the segment for a second pass with the segment's
    // maximum as the reference. Pieces: 0 waits for the scores, 1..4 take the max, 5 masks
    // (a masked step only) and updates the reference, 6..21 exponentiate one value each and
    // round P to bf16, 22 sums.
    // The row maximum is taken only where it is needed: on the segment's first step (which
    // sets the reference of every row that sees a key in the segment), on masked steps, and
    // on every step of a tracking pass. Elsewhere the only guard is the row sum: it bounds
    // every P, and the pass ends with a check that it stayed below 2^60.
    float sm_mx, sm_muse = 0.f, sm_psum;
    float sm_x = 0.f, sm_e = 0.f;   // skewed exp stages
    bool sm_do_max = true, sm_masked = false, track = false;
    auto softmax_piece = [&](f32x16& s, int hh, bool live, int piece, bf16x8* pk) {
      if (piece == 0) {
        mfma_result_wait(s);
        sm_masked = kStep * (hh + 1) > lim_min;   // (wave-uniform)
        sm_do_max = track || sm_masked || hh == sg.hh0;
      } else if (piece <= 4) {
        if (sm_do_max) {
          const int r0 = 4 * (piece - 1);
          float mx = piece == 1 ? -INFINITY : sm_mx;
#pragma unroll
          for (int r = r0; r < r0 + 4; ++r) mx = fmaxf(mx, s[r]);
          sm_mx = mx;
        }
      } else if (piece == 5) {
        if (sm_do_max) {
          if (sm_masked) {   // the sequence's last step, or causal rows
            const int key0 = kStep * hh + 4 * (lane >> 5);
            float mx = -INFINITY;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              s[r] = (key0 + 8 * (r >> 2) + (r & 3)) < lim ? s[r] : -INFINITY;
              mx = fmaxf(mx, s[r]);
            }
            sm_mx = mx;
          }
          const float mx = max_across_halves(sm_mx) * a.scale_log2;
          if (live) {
            m_seen = fmaxf(m_seen, mx);
            m_run = (m_run == -INFINITY && mx != -INFINITY) ? ceilf(mx) : m_run;
            window_exceeded = window_exceeded || (track && mx > m_run + kWindow);
          }
          sm_muse = (m_run == -INFINITY) ? 0.f : m_run;
        }
        sm_psum = 0.f;
      } else if (piece <= 23) {
        // three stages a piece apart (scaled logit of element k - 6, its exponential at
        // k - 7, sum and bf16 at k - 8), so that no piece is one dependent chain
        const int rf = piece - 6, re = piece - 7, ra = piece - 8;
        if (ra >= 0 && ra < 16) {
          sm_psum += sm_e;
          pk[ra >> 3][ra & 7] = (__bf16)sm_e;
        }
        if (re >= 0 && re < 16) sm_e = __builtin_amdgcn_exp2f(sm_x);
        if (rf < 16) sm_x = __builtin_fmaf(s[rf], a.scale_log2, -sm_muse);
      } else {
        const float psum = sum_across_halves(sm_psum);
        l_run = live ? l_run + psum : l_run;
      }
    };
    constexpr int kPieces = 25;
    // this wave's P tiles (k-steps 0, 1) into P buffer b: tile (row block, k-step q) is 1 KiB
    // at (2 row block + q) KiB, 16 B per lane, the A-operand layout
    auto p_store = [&](int b, const bf16x8* pk) {
      char __attribute__((address_space(3)))* dst = lds + (plane + b * kR32PBytes + wave * 2048);
      *reinterpret_cast<bf16x8 __attribute__((address_space(3)))*>(dst) = pk[0];
      *reinterpret_cast<bf16x8 __attribute__((address_space(3)))*>(dst + 1024) = pk[1];
    };

#pragma unroll 1
    for (int pass = 0; pass < 3; ++pass) {
      track = pass > 0;
#pragma unroll
      for (int c = 0; c < 16; ++c) o[c] = f32x16{};
      if (nsteps > 0) {
      bf16x8 pcur[2];   // P of the current step for this wave's rows (A operands, k-steps 0, 1)
      bf16x8 bq0[4];    // Z^T of the current step's k-step 0, this wave's channel tiles (B operands)
      uint32_t zc = (uint32_t)comp_slot * kBufBytes;
      // bf16: data of step 0 (steps 1 and 2 may stay in flight); fp8: steps 0 and 1 are in
      // their bf16 slots since the last region or fill (the barrier orders the previous
      // item's last LDS reads before the P writes below)
      if constexpr (!kFp8) wait_vmcnt<2 * kR32Dma>();
      barrier_lds();
      // scores and softmax of step 0; its P goes to P buffer 0
      {
        f32x16 s;
        bf16x8 qring[kR32QkRing];
        const QkAddr qa = qk_at(qk0, zc);
#pragma unroll
        for (int t = 0; t < kR32QkRing; ++t) qring[t] = qk_read(qa, t);
        bf16x8 qx[2];
#pragma unroll
        for (int t = 0; t < 36; ++t) {
          const bf16x8 cur = qring[t % kR32QkRing];
          if (t + kR32QkRing < 36) qring[t % kR32QkRing] = qk_read(qa, t + kR32QkRing);
          if (kFp8 && t >= 30 && t < 32) qx[t - 30] = q_lds(t + 4);
          if (t == 0) mfma_v0(s, cur, qreg[0]);
          else mfma_v(s, cur, (kFp8 && t >= 34) ? qx[t - 34] : qreg[t]);
        }
#pragma unroll
        for (int p = 0; p < kPieces; ++p) softmax_piece(s, sg.hh0, true, p, pcur);
        p_store(0, pcur);
        if constexpr (!kFp8) {   // (the fp8 step region reads its value operands itself)
          const PvAddr pa = pv_at(pv0, zc);
#pragma unroll
          for (int c = 0; c < 4; ++c) bq0[c] = pv_read(pa, c);
        }
      }
      if constexpr (!kFp8) wait_vmcnt<kR32Dma>();   // data of step 1, for the first region's scores
      barrier_lds();               // (and every wave's P of step 0)

      // Straight-line step body: the scores of step i+1 are computed also after the last
      // step (on whatever the next slot holds) and discarded, and a region past the end of
      // the worker's range issues zero-record loads, so that every region has the same
      // shape and the same DMA count.
#pragma unroll 1
      for (int i = 0; i < nsteps; ++i) {
        const int cs_next = kFp8 ? comp_slot ^ 1 : (comp_slot + 1 == kR32Slots ? 0 : comp_slot + 1);
        const uint32_t zn = (uint32_t)cs_next * kBufBytes;
        const bool live = i + 1 < nsteps;   // step i+1 belongs to this segment
        const StepRsrc rs = step_rsrc();
        const uint32_t lslot = kFp8 ? lds_u32 + kR8StBase + (uint32_t)load_slot * kR8StBytes
                                    : lds_u32 + (uint32_t)load_slot * kBufBytes;
        // fp8: the staged step i+2 (the slot after the one being loaded) is dequantised into
        // the bf16 slot of step i, this wave's 128 channels: tokens 0..15 while the scores are
        // computed (this wave read them before the last barrier), tokens 16..31 piece by
        // piece after the value operand reads of step i (LDS executes a wave's accesses in
        // order); the rope in the score phase (its last reader was the previous region)
        const uint32_t st_dq = kR8StBase + (uint32_t)(load_slot + 1 == kR8Stage ? 0 : load_slot + 1) * kR8StBytes;
        float f8_s = 0.f;
        F8Half f8_b;
        u32x2 f8_w[2];
        bf16x4 f8_lo;
        u32x4 f8_rp;
        // piece q of the dequantisation of half h: q = 0 the scale and bases, 1 + c the codes
        // of piece c, 5 + 2c the first 4 values of piece c, 6 + 2c the other 4 and the store
        auto f8_piece = [&](int h, int q) {
          if (q == 0) {
            f8_s = f8_scale(st_dq, h);
            f8_b = f8_half(st_dq, zc, h);
          } else if (q <= 4) {
            f8_w[(q - 1) & 1] = f8_codes(f8_b, q - 1);
          } else {
            const int c = (q - 5) >> 1;
            if (((q - 5) & 1) == 0) f8_lo = dequant4(f8_w[c & 1][0], f8_s);
            else f8_store(f8_b, c, f8_lo, dequant4(f8_w[c & 1][1], f8_s));
          }
        };
        const uint32_t pbuf = plane + (uint32_t)(i & 1) * kR32PBytes;   // P of step i (this lane)
        uint32_t voff = 0;        // source offset of the next DMA instruction (3 MFMAs ahead)
        f32x16 s;                 // scores of step i+1
        bf16x8 pnext[2];          // P of step i+1, this wave's rows
        // A operand of step i: P of row block (wave + g) % 4, k-step q (1 KiB per tile)
        auto a_read = [&](int g, int q) -> bf16x8 {
          const uint32_t rb = (uint32_t)((wave + g) & 3);
          return lds_b128(lds + (pbuf + rb * 2048u + (uint32_t)q * 1024u));
        };
        if constexpr (kFp8) {
          // 2) scores of step i+1 with the DMA instructions of step i+4 and half 0 of the
          //    dequantisation of step i+2 between them. Half 0 overwrites the k-step-0 rows of
          //    step i, so each Z^T tile of k-step 0 is read just before its piece is stored
          //    (LDS executes a wave's accesses in order); the P tiles of k-step 0 are read
          //    during the last score MFMAs
          bf16x8 aq0[2], bz0[4];   // (P tiles of k-step 0: two in flight)
          {
            const PvAddr pa = pv_at(pv0, zc);
            bf16x8 qring[kF8QkRing];
            const QkAddr qa = qk_at(qk0, zn);
#pragma unroll
            for (int t = 0; t < kF8QkRing; ++t) qring[t] = qk_read(qa, t);
            bf16x8 qx[2];
            uint32_t f8_sv = 0;
#pragma unroll
            for (int t = 0; t < 36; ++t) {
              const bf16x8 cur = qring[t % kF8QkRing];
              if (t + kF8QkRing < 36) qring[t % kF8QkRing] = qk_read(qa, t + kF8QkRing);
              if (t >= 30 && t < 32) qx[t - 30] = q_lds(t + 4);
              if (t == 33) aq0[0] = a_read(0, 0);
              if (t >= 18 && t < 26 && !(t & 1)) bz0[(t - 18) >> 1] = pv_read(pa, (t - 18) >> 1);
              if (t == 0) mfma_v0(s, cur, qreg[0]);
              else mfma_v(s, cur, t >= 34 ? qx[t - 34] : qreg[t]);
              // DMA instruction j at t = 2j + 1 (token-sparse: the row of the next one read right
              // after, two MFMAs ahead of its use)
              if (kSparse && t == 0) f8_sv = f8_row(0);
              if ((t & 1) == 1 && t < 12) {
                dma_f8(rs, lslot, t >> 1, f8_sv);
                if (kSparse && t < 11) f8_sv = f8_row((t >> 1) + 1);
              }
              if (t == 27) dma_rows((row_slot + 2) & 3);   // token-sparse: rows of step i+6
              if (t == 14) f8_piece(0, 0);
              if (t == 15) f8_piece(0, 1);
              if (t == 17) f8_piece(0, 2);
              if (t >= 19 && t < 27) f8_piece(0, t - 14);   // codes two pieces ahead of their conversion
              if (t == 20) f8_piece(0, 3);
              if (t == 22) f8_piece(0, 4);
              if (t == 8) f8_rp = f8_rope(st_dq);
              if (t == 11) f8_rope_store(zc, f8_rp);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          // 3) the 32 value MFMAs of step i (k-step 0 row block by row block, then k-step 1
          //    channel tile by channel tile) with the softmax of step i+1 and half 1 of the
          //    dequantisation between them (its stores after the last Z^T read of step i)
          {
            const PvAddr pa = pv_at(pv0, zc);
            bf16x8 bq1[3];   // ring of Z^T tiles of k-step 1
            bf16x8 aq1[4];   // P tiles of k-step 1
#pragma unroll
            for (int t = 0; t < 32; ++t) {
              if (t == 6) bq1[0] = pv_read(pa, 16 + 0);
              if (t >= 8 && t < 12) aq1[t - 8] = a_read(t - 8, 1);
              if (t == 12) bq1[1] = pv_read(pa, 16 + 1);
              if (t == 16) bq1[2] = pv_read(pa, 16 + 2);
              if (t == 20) bq1[0] = pv_read(pa, 16 + 3);
              if (t < 12 && t % 4 == 1) aq0[((t + 3) / 4) & 1] = a_read((t + 3) / 4, 0);
              if (t < 16) {
                const int g = t / 4, c = t % 4;
                mfma_a(o[4 * g + c], aq0[g & 1], bz0[c]);
              } else {
                const int c = (t - 16) / 4, g = (t - 16) % 4;
                mfma_a(o[4 * g + c], aq1[g], bq1[c % 3]);
              }
              if (t < kPieces) softmax_piece(s, sg.hh0 + i + 1, live, t, pnext);
              if (t == 22) f8_piece(1, 0);
              if (t == 23) f8_piece(1, 1);
              if (t == 24) f8_piece(1, 2);
              if (t >= 25) f8_piece(1, t - 20);
              if (t == 26) f8_piece(1, 3);
              if (t == 28) f8_piece(1, 4);
              __builtin_amdgcn_sched_barrier(0);
            }
          }
          f8_piece(1, 12);
          p_store((i + 1) & 1, pnext);
        } else {
        // 1) the first value MFMAs of step i: this wave's rows, k-step 0, its four channel
        //    tiles (operands in registers)
#pragma unroll
        for (int c = 0; c < kR32PvLead; ++c) {
          mfma_a(o[c], pcur[0], bq0[c]);
          __builtin_amdgcn_sched_barrier(0);
        }
        // 2) scores of step i+1 with the DMA instructions of the step being loaded; the P
        //    tiles of the other row blocks (k-step 0) are read during the last score MFMAs
        bf16x8 aq0[3];
        {
          bf16x8 qring[kR32QkRing];
          const QkAddr qa = qk_at(qk0, zn);
#pragma unroll
          for (int t = 0; t < kR32QkRing; ++t) qring[t] = qk_read(qa, t);
#pragma unroll
          for (int t = 0; t < 36; ++t) {
            const bf16x8 cur = qring[t % kR32QkRing];
            if (t + kR32QkRing < 36) qring[t % kR32QkRing] = qk_read(qa, t + kR32QkRing);
            if (t == 29) aq0[0] = a_read(1, 0);
            if (t == 31) aq0[1] = a_read(2, 0);
            if (t == 33) aq0[2] = a_read(3, 0);
            if (t == 0) mfma_v0(s, cur, qreg[0]);
            else mfma_v(s, cur, qreg[t]);
            if ((t & 3) == 0) voff = dma_voff(dmo, t >> 2);   // offset of the next DMA instruction
            if ((t & 3) == 3) issue32_rows(rs.kv, lslot, t >> 2, voff, wave);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        // 3) the remaining value MFMAs of step i, the softmax of step i+1 between them:
        //    k-step 0 for the other row blocks, then k-step 1 channel tile by channel tile
        {
          const PvAddr pa = pv_at(pv0, zc);
          bf16x8 bq1[4];   // Z^T tiles of k-step 1
          bf16x8 aq1[3];   // P tiles of k-step 1, the other row blocks
#pragma unroll
          for (int t = kR32PvLead; t < 32; ++t) {
            if (t == 5) bq1[0] = pv_read(pa, 16 + 0);
            if (t == 8) aq1[0] = a_read(1, 1);
            if (t == 9) aq1[1] = a_read(2, 1);
            if (t == 10) aq1[2] = a_read(3, 1);
            if (t == 7) bq1[1] = pv_read(pa, 16 + 1);
            if (t == 11) bq1[2] = pv_read(pa, 16 + 2);
            if (t == 13) bq1[3] = pv_read(pa, 16 + 3);
            if (t < 16) {
              const int g = 1 + (t - 4) / 4, c = (t - 4) % 4;
              mfma_a(o[4 * g + c], aq0[g - 1], bq0[c]);
            } else {
              const int c = (t - 16) / 4, g = (t - 16) % 4;
              mfma_a(o[4 * g + c], g == 0 ? pcur[1] : aq1[g == 0 ? 0 : g - 1], bq1[c]);
            }
            // one softmax piece after each value MFMA
            const int u = t - kR32PvLead;
            if (u < kPieces) softmax_piece(s, sg.hh0 + i + 1, live, u, pnext);
            // the first value operands of step i+1 once this step's k-step-0 MFMAs are done
            // (its rows were published at the last barrier), and the P of step i+1 once the
            // softmax has formed it, so that their LDS latency ends before the barrier
            if (t >= 17 && t <= 23 && (t & 1)) bq0[(t - 17) >> 1] = pv_read(pv_at(pv0, zn), (t - 17) >> 1);
            if (t == 29) p_store((i + 1) & 1, pnext);
            __builtin_amdgcn_sched_barrier(0);
          }
        }
        pcur[0] = pnext[0];
        pcur[1] = pnext[1];
        }
        // move the load cursor here: its scalar loads share the LDS counter, and the barrier
        // waits for that counter anyway
        advance();
        // everything but this region's DMA: the data of step i+2 (bf16) or i+3 (fp8)
        if constexpr (kFp8) wait_f8_steps<1, kSparse>(wave);
        else wait_vmcnt<kR32Dma>();
        barrier_lds();
        comp_slot = cs_next;
        zc = zn;
      }
      }
      // Did any row of the work-group leave the reference window? (vote through LDS)
      {
        int32_t __attribute__((address_space(3)))* vote =
            (int32_t __attribute__((address_space(3)))*)(lds + kPBase);
        // (a NaN sum counts as out of range)
        const bool lane_bad = track ? window_exceeded : !(l_run <= 0x1p60f);
        const bool wave_exceeded = __ballot(lane_bad) != 0;   // (all lanes take part)
        if (lane == 0) vote[wave] = wave_exceeded ? 1 : 0;
        barrier_lds();
        const bool again = (vote[0] | vote[1] | vote[2] | vote[3]) != 0;
        barrier_lds();   // (the votes are read before the area is reused)
        if (!again || pass == 2) break;
      }
      // Another pass over the segment. After the first: every row takes m + log2(l) rounded
      // up, which is at least its maximum, so no P exceeds 1; a row whose sum overflowed takes
      // its reference afresh, and the pass takes the maximum on every step with the window
      // check. After that (a tracking pass that left the window): the segment's maximum.
      // Wait for the loads in flight (the next item's first steps), then restart the load
      // cursor at the segment's first step in an empty ring.
      wait_vmcnt<0>();
      barrier_lds();
      if (pass == 0) {
        const bool ok = m_run != -INFINITY && l_run > 0.f && l_run <= 0x1p126f;
        m_run = ok ? ceilf(m_run + __log2f(l_run)) : -INFINITY;
      } else {
        m_run = (m_seen == -INFINITY) ? -INFINITY : ceilf(m_seen);
      }
      m_seen = -INFINITY;
      l_run = 0.f;
      window_exceeded = false;
      restart(lc, k);
      if constexpr (kSparse) {
        restart(pc, k);
        row_slot = 0;
      }
      load_slot = 0;
      comp_slot = 0;
      if constexpr (kFp8) {
        f8_fill(false);
      } else {
#pragma unroll 1
        for (int j = 0; j < kR32Slots - 1; ++j) issue_step();
      }
    }

    // ---- finalize: out = O / l and lse = m + log2(l), or, for items the plan split, the
    // unnormalised bf16 partial in register order plus (m, l). O tile 4g + c holds, in lane l
    // and register r, row 8(r/4) + 4(l/32) + r%4 of row block (wave + g) % 4 and channel
    // 128 wave + 32c + l%32; a row's 1/l, m and lse come from the wave that owns its softmax
    // (rows 32 wave ..), its 1/l through LDS.
    {
      int l = lane;
      asm volatile("" : "+v"(l));
      const int32_t* itf = plan + plan_items_off() + kItemWords * k;
      const int f_seq = itf[kISeq], f_tile = itf[kITile], f_ns = itf[kINsplits];
      const bool split = f_ns > 1;
      const int slot = split ? itf[kISlot] + (worker - itf[kIOwner]) : 0;
      const int row0 = kRowsPerTile * f_tile + 32 * wave;   // the first row this wave owns
      float __attribute__((address_space(3)))* inv_s = (float __attribute__((address_space(3)))*)(lds + kPBase + 64);
      // out row of register r of a tile of row block rb, and its column base for this lane
      auto out_row = [&](int rb, int r, bool& ok) -> float* {
        const int grow = kRowsPerTile * f_tile + 32 * rb + 8 * (r >> 2) + 4 * (l >> 5) + (r & 3);
        ok = grow < rows_total;
        const int jt = ok ? grow / a.heads : 0, hd = ok ? grow - jt * a.heads : 0;
        return out_ptr + ((int64_t)(f_seq * a.s_q + jt) * a.heads + hd) * kLat + 128 * wave + (l & 31);
      };
      if (!split) {
        if (l < 32) inv_s[32 * wave + l] = l_run > 0.f ? 1.f / l_run : 0.f;
        barrier_lds();   // every row's 1/l from the wave that owns it
      }
      mfma_results_settle();
      if (split) {
        char* part = reinterpret_cast<char*>(ws) + (int64_t)slot * kSlotBytes;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rb = (wave + g) & 3;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            bf16x8 v0, v1;
#pragma unroll
            for (int r = 0; r < 8; ++r) {   // unnormalised: the merge divides by the denominator
              v0[r] = (__bf16)o[4 * g + c][r];
              v1[r] = (__bf16)o[4 * g + c][8 + r];
            }
            // fragment (row block, channel tile 4 wave + c, lane)
            char* dst = part + 32 * (int64_t)((rb * 16 + 4 * wave + c) * 64 + l);
            *reinterpret_cast<bf16x8*>(dst) = v0;
            *reinterpret_cast<bf16x8*>(dst + 16) = v1;
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int rb = (wave + g) & 3;
          f32x4 inv4[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            inv4[j] = *(const f32x4 __attribute__((address_space(3)))*)(inv_s + 32 * rb + 8 * j + 4 * (l >> 5));
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            bool ok;
            float* dst = out_row(rb, r, ok);
            const float sc = inv4[r >> 2][r & 3];
#pragma unroll
            for (int c = 0; c < 4; ++c) {
              const float v = o[4 * g + c][r] * sc;
              if (ok) dst[32 * c] = v;
            }
            __builtin_amdgcn_sched_barrier(0);
          }
        }
      }
      const int grow = row0 + (l & 31);
      const int row = 32 * wave + (l & 31);
      if (split) {
        // the partial's reference max (log2 units; -inf for a row with no visible key) and
        // softmax denominator
        if (l < 32) {
          float* stat = reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (int64_t)slot * kSlotBytes + kSlotPartBytes);
          const bool any = grow < rows_total && l_run > 0.f;
          stat[row] = any ? m_run : -INFINITY;
          stat[kRowsPerTile + row] = any ? l_run : 0.f;
        }
      } else if (l < 32 && grow < rows_total) {
        const float m = (m_run == -INFINITY) ? 0.f : m_run;
        const float lse_v = l_run > 0.f ? (m + __log2f(l_run)) * 0.6931471805599453f : -INFINITY;
        const int jt = grow / a.heads, hd = grow - jt * a.heads;
        lse_ptr[(int64_t)(f_seq * a.s_q + jt) * a.heads + hd] = lse_v;
      }
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  report();
}

// Merge the partials of split items written by decode_rows32_kernel. Part k of a row holds
// O_k (unnormalised, relative to its reference max m_k, log2 units) and its denominator l_k:
// with M = max_k m_k and a_k = 2^(m_k - M), out = sum_k a_k O_k / sum_k a_k l_k and
// lse = (M + log2 sum_k a_k l_k) ln 2 (parts with no visible key have m_k = -inf, weight 0).
// One block per (split item, 32-row group w, 128-channel quarter cq). Fragment (w, c, lane)
// of a part is 32 contiguous bytes: 16 bf16, value r at row 32w + 8(r/4) + 4(lane/32) + r%4
// and channel 32c + lane%32, so a block reads 8 contiguous KiB per part. The data loads of
// the first parts are issued before the weights are formed; the merged rows leave through
// LDS as 512-B row segments.
constexpr int kCmbThreads = 256;
constexpr int kCmbMaxSplits = 64;    // parts merged per pass over the weights (LDS: 2 x 8 KiB)
constexpr int kCmbBatch = 4;         // parts whose data is in flight together

__global__ __launch_bounds__(kCmbThreads) void combine_rows32_kernel(const int32_t* __restrict__ plan,
                                                                     const char* __restrict__ ws,
                                                                     float* __restrict__ out,
                                                                     float* __restrict__ lse, int batch, int s_q,
                                                                     int heads, int causal, int n_items, int workers,
                                                                     int32_t* __restrict__ status) {
  __shared__ __attribute__((aligned(16))) float wts[kCmbMaxSplits][32];   // [part][row]: m_k, then weights
  __shared__ float dens[kCmbMaxSplits][32];                               // [part][row]: l_k
  __shared__ float tile_out[32][128 + 4];
  __shared__ __attribute__((aligned(16))) float row_resc[32];
  __shared__ __attribute__((aligned(16))) float row_t[32];
  __shared__ float row_m[32];
  // The header (one 16-word load) is checked before this block's split record is read: a plan
  // built for other arguments may sit in a smaller buffer, so no offset derived from the call's
  // arguments is read until the header matches them. (The record area holds n_items entries,
  // so the read is then in bounds for every block of the grid.)
  const i32x16 hd = load_plan_header(plan);
  if (!plan_header_matches(hd, batch, s_q, heads, causal, workers, n_items)) {
    if (status != nullptr && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)
      __hip_atomic_fetch_or(status, (int)kDevPlanMismatch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if ((int)blockIdx.x >= hd[kHSplitItems]) return;
  const int32_t* sr = plan + plan_split_off(n_items, workers) + kSplitWords * blockIdx.x;
  const int seq = sr[kSSeq], tile = sr[kSTile], ns_all = sr[kSNsplits], slot0 = sr[kSSlot];
  const int rows_total = s_q * heads;
  const int w = blockIdx.y, cq = blockIdx.z;
  if (kRowsPerTile * tile + 32 * w >= rows_total) return;
  const int tid = threadIdx.x;
  const int c = 4 * cq + (tid >> 6), ln = tid & 63, h = ln >> 5;
  const int64_t frag = 32 * (int64_t)((w * 16 + c) * 64 + ln);
  // this thread's rows: 8j + 4h + v for register r = 4j + v
  float acc[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  float m_old = -INFINITY, t_old = 0.f;   // per row, kept by threads tid < 32
  for (int s0 = 0; s0 < ns_all; s0 += kCmbMaxSplits) {
    const int ns = ns_all - s0 < kCmbMaxSplits ? ns_all - s0 : kCmbMaxSplits;
    // data of the first parts in flight while the weights are formed
    bf16x8 v[kCmbBatch][2];
#pragma unroll
    for (int b = 0; b < kCmbBatch; ++b)
      if (b < ns) {
        const char* p = ws + (int64_t)(slot0 + s0 + b) * kSlotBytes + frag;
        v[b][0] = *reinterpret_cast<const bf16x8*>(p);
        v[b][1] = *reinterpret_cast<const bf16x8*>(p + 16);
      }
    __syncthreads();
    for (int idx = tid; idx < 32 * ns; idx += kCmbThreads) {
      const int rr = idx & 31, sp = idx >> 5;
      const float* stat = reinterpret_cast<const float*>(ws + (int64_t)(slot0 + s0 + sp) * kSlotBytes + kSlotPartBytes);
      wts[sp][rr] = stat[32 * w + rr];
      dens[sp][rr] = stat[kRowsPerTile + 32 * w + rr];
    }
    __syncthreads();
    if (tid < 32) {
      float m = m_old;
      for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, wts[sp][tid]);
      const float safe = m == -INFINITY ? 0.f : m;
      const float resc = m_old == -INFINITY ? 0.f : exp2f(m_old - safe);
      float tot = t_old * resc;
      for (int sp = 0; sp < ns; ++sp) {
        const float mk = wts[sp][tid];
        const float wgt = mk == -INFINITY ? 0.f : exp2f(mk - safe);
        wts[sp][tid] = wgt;
        tot += wgt * dens[sp][tid];
      }
      m_old = m;
      t_old = tot;
      row_resc[tid] = resc;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 rs4 = *reinterpret_cast<const f32x4*>(&row_resc[8 * j + 4 * h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[4 * j + e] *= rs4[e];
    }
    for (int b0 = 0; b0 < ns; b0 += kCmbBatch) {
      if (b0 > 0) {
#pragma unroll
        for (int b = 0; b < kCmbBatch; ++b)
          if (b0 + b < ns) {
            const char* p = ws + (int64_t)(slot0 + s0 + b0 + b) * kSlotBytes + frag;
            v[b][0] = *reinterpret_cast<const bf16x8*>(p);
            v[b][1] = *reinterpret_cast<const bf16x8*>(p + 16);
          }
      }
#pragma unroll
      for (int b = 0; b < kCmbBatch; ++b)
        if (b0 + b < ns) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const f32x4 w4 = *reinterpret_cast<const f32x4*>(&wts[b0 + b][8 * j + 4 * h]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int r = 4 * j + e;
              acc[r] += w4[e] * (float)v[b][r >> 3][r & 7];
            }
          }
        }
    }
  }
  if (tid < 32) {
    row_t[tid] = t_old;
    row_m[tid] = m_old;
  }
  __syncthreads();
  {
    const int cl = 32 * (c - 4 * cq) + (ln & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f32x4 t4 = *reinterpret_cast<const f32x4*>(&row_t[8 * j + 4 * h]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float t = t4[e];
        tile_out[8 * j + 4 * h + e][cl] = acc[4 * j + e] * (t > 0.f ? 1.f / t : 0.f);
      }
    }
  }
  __syncthreads();
  // 32 rows x 128 channels: 32 float4 per row
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int idx = tid + kCmbThreads * j;
    const int rr = idx >> 5, c4 = (idx & 31) * 4;
    const int grow = kRowsPerTile * tile + 32 * w + rr;
    if (grow >= rows_total) continue;
    const int jt = grow / heads, hd = grow - jt * heads;
    const int64_t orow = (int64_t)(seq * s_q + jt) * heads + hd;
    *reinterpret_cast<f32x4*>(out + orow * kLat + 128 * cq + c4) = *reinterpret_cast<const f32x4*>(&tile_out[rr][c4]);
    if (cq == 0 && c4 == 0) {
      const float t = row_t[rr];
      lse[orow] = t > 0.f ? (row_m[rr] + __log2f(t)) * 0.6931471805599453f : -INFINITY;
    }
  }
}

template <bool kFp8, bool kSparse>
hipError_t launch_rows32(const DecodeArgs& a, const int32_t* srows, int srow_stride, hipStream_t stream) {
  constexpr int lds_bytes = kSparse ? kR8SparseLdsTotal : (kFp8 ? kR8LdsTotal : kR32LdsTotal);
  static thread_local int configured = -1;   // the LDS opt-in is per device
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)decode_rows32_kernel<kFp8, kSparse>,
                            hipFuncAttributeMaxDynamicSharedMemorySize, lds_bytes);
    if (e != hipSuccess) return e;
    configured = dev;
  }
  hipLaunchKernelGGL((decode_rows32_kernel<kFp8, kSparse>), dim3(a.workers), dim3(kR32Threads), lds_bytes, stream,
                     reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const char*>(a.kv), a.kv_scales,
                     a.block_table, a.plan, a.ws, a.out, a.lse, srows, srow_stride, a.status, scalars_of(a));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_rows32(const DecodeArgs& a, bool fp8, hipStream_t stream) {
  return fp8 ? launch_rows32<true, false>(a, nullptr, 0, stream) : launch_rows32<false, false>(a, nullptr, 0, stream);
}

hipError_t launch_decode_sparse_fp8(const DecodeArgs& a, const int32_t* rows, int row_stride, hipStream_t stream) {
  return launch_rows32<true, true>(a, rows, row_stride, stream);
}

hipError_t launch_combine_rows32(const DecodeArgs& a, hipStream_t stream) {
  const int n_items = a.batch * tiles_per_seq(a.s_q, a.heads);
  const int max_split = a.workers < n_items ? a.workers : n_items;   // split items <= both
  hipLaunchKernelGGL(combine_rows32_kernel, dim3(max_split, kRowsPerTile / 32, 4), dim3(kCmbThreads), 0, stream,
                     a.plan, reinterpret_cast<const char*>(a.ws), a.out, a.lse, a.batch, a.s_q, a.heads, a.causal,
                     n_items, a.workers, a.status);
  return hipGetLastError();
}

}  // namespace mla
