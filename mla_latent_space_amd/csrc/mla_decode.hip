// Latent-space MLA decode over an fp8 (OCP e4m3fn) cache, for gfx950 (MI355X).
//
// Page "Mla Analysis", section "Absorption Trick (FlashMLA)": scores are Qz . Z^T with the
// absorbed 576-wide queries, and the value is the latent row itself, so one pass over the
// paged latent cache gives O_latent = softmax(scale Qz Z^T) Z[:, :512] and a log-sum-exp
// per (token, head). With an fp8 cache each cached value is code * scale[token][tile]
// (page "FlashMLA", its fp8 cache support), dequantised once per step into a bf16 slot.
//
// Work-group = 8 waves (two per SIMD) = one persistent worker of the split plan, one per
// compute unit; it walks its contiguous run of (item, page) pairs in 32-token steps.
//  * Each half page (codes + rope, then its scales) is staged in LDS as loaded by LDS-DMA
//    buffer loads (buffer_load_dwordx4 ... lds: 1 KiB per wave instruction); the record
//    count stops at the last visible token, so masked tail rows arrive as zeros. Between
//    the two barriers of a step the work-group dequantises the oldest staged step into a
//    bf16 slot whose rows are XOR-swizzled in 16-B chunks (chunk ^= (token >> 1) & 7).
//  * Scores: wave w owns query rows 16w..16w+15 of the 128-row tile and computes
//    S^T = Z Q^T with v_mfma_f32_16x16x32_bf16: A = 16 tokens x 32 channels read from LDS
//    (ds_read_b128), B = Q^T held in 72 VGPRs for the whole segment.
//  * Online softmax in the S^T layout: each lane owns one query row and 8 of the 32
//    tokens, so row max / row sum are lane-local plus permlane16/32 swaps. The running
//    max is only moved when it grows by more than 2^8 (lazy rescale), so the accumulator
//    is rarely rescaled; the softmax of step i+1 is interleaved with the value MFMAs of
//    step i.
//  * P (bf16) goes through LDS in the MFMA B-operand layout; value products are split
//    by channels: wave w owns O^T[64w .. 64w+63][all 128 rows] (128 accumulator VGPRs),
//    A = Z^T via ds_read_b64_tr_b16 (transposing LDS read), B = P^T from LDS, with
//    v_mfma_f32_32x32x16_bf16.
//  * Finalize writes out/lse directly, or a normalised bf16 partial + lse into the
//    workspace for items the plan split; combine_kernel merges those by log-sum-exp.
#include "mla_device.h"

namespace mla {
namespace {

constexpr int kThreads = 512;                  // 8 waves, two per SIMD
constexpr int kNBuf = 4;                       // LDS ring depth
constexpr int kPRowBytes = 80;                 // P exchange row: 32 bf16 + 16 B pad (bank spread)

// LDS layout. bf16 cache: a ring of kNBuf slots of 32 bf16 rows, read in place. fp8 cache:
// a ring of kF8Slots staging slots (codes, rope, scales as loaded) and two bf16 slots that
// each step is dequantised into once, so the score/value code is shared with the bf16 path.
template <bool kFp8>
struct Lds {
  static constexpr int kWork = kFp8 ? 2 : kNBuf;                      // bf16 slots
  static constexpr int kOffF8 = kWork * kBufBytes;                    // fp8 staging ring
  static constexpr int kOffP = kOffF8 + (kFp8 ? kF8Slots * kF8SlotBytes : 0);   // P: [128 rows][32 tokens] bf16
  static constexpr int kOffAlpha = kOffP + kRowsPerTile * kPRowBytes;  // 128 floats: per-row rescale of a step
  static constexpr int kOffStat = kOffAlpha + 512;                    // 128 floats m, 128 floats l
  static constexpr int kBytes = kOffStat + 1024;
  static_assert(kBytes <= 160 * 1024, "LDS budget");
  // LDS-DMA instructions per step: waves below kLong issue kBase + 1, the others kBase
  static constexpr int kDmaBase = kFp8 ? kF8DmaInstr / 8 : kDmaInstr / 8;
  static constexpr int kLong = kFp8 ? kF8DmaInstr % 8 : kDmaInstr % 8;
  static constexpr int kIssueEvery = 36 / (kDmaBase + 1);   // score tiles between two DMA instructions
};

__device__ __forceinline__ int swz(int u) { return (u >> 1) & 7; }

// Per-lane source offsets of this wave's LDS-DMA instructions. Instruction i (1 KiB,
// 64 lanes x 16 B, lane-linear in LDS) is issued by wave i % 8; LDS chunk position
// p = 72u + pc holds logical chunk ch = pc ^ swz(u) of token u.
// Only full-rate 24-bit multiplies: with x = p * 1821, u = floor(p / 72) = x >> 17 and
// p mod 72 = ((x mod 2^17) * 72) >> 17, exactly for every p < 2304 (a step's 36 x 64 chunk
// positions; both products stay below 2^24).
__device__ __forceinline__ uint32_t dma_voff(int wave, int n, int lane) {
  const uint32_t p = 64u * (uint32_t)(wave + 8 * n) + (uint32_t)lane;
  const uint32_t x = __umul24(p, 1821u);
  const uint32_t u = x >> 17;
  const uint32_t pc = __umul24(x & 0x1FFFFu, 72u) >> 17;
  const uint32_t ch = (pc & ~7u) | ((pc & 7u) ^ (uint32_t)swz((int)u));
  return __umul24(u, (uint32_t)kRowBytes) + 16u * ch;
}

// One of this wave's LDS-DMA instructions of a step: instruction i = wave + 8n. The per-lane
// offset is recomputed at every issue from an opaque copy of the lane id: kept live across
// the loop it gets spilled, and a scratch reload waits vmcnt(0), which would drain the ring.
// bf16: 36 instructions of 1 KiB into the swizzled slot. fp8: 20 instructions copy the
// step's 20 KiB of codes+rope as they are, the 21st (lanes 0..31) its 512 B of scales.
template <bool kFp8>
__device__ __forceinline__ void issue_one(const StepRsrc& rs, uint32_t lds_slot, int n, int lane, int wave) {
  const int i = wave + 8 * n;
  int l = lane;
  asm volatile("" : "+v"(l));
  if constexpr (!kFp8) {
    if (i >= kDmaInstr) return;
    lds_dma_x4(lds_slot + 1024u * (uint32_t)i, dma_voff(wave, n, l), rs.kv);
  } else {
    if (i >= kF8DmaInstr) return;
    if (i < kF8DmaInstr - 1) {
      lds_dma_x4(lds_slot + 1024u * (uint32_t)i, 1024u * (uint32_t)i + 16u * (uint32_t)l, rs.kv);
    } else if (l < kStep) {
      lds_dma_x4(lds_slot + (uint32_t)kF8StepBytes, 16u * (uint32_t)l, rs.sc);
    }
  }
}

template <bool kFp8>
__device__ __forceinline__ void issue_step(const StepRsrc& rs, uint32_t lds_slot, int lane, int wave) {
#pragma unroll
  for (int n = 0; n < Lds<kFp8>::kDmaBase + 1; ++n) issue_one<kFp8>(rs, lds_slot, n, lane, wave);
}

// Dequantise one fp8 step from its staging slot into a bf16 slot (same row layout and
// swizzle as a bf16 cache step): thread t handles token t/16 and latent channels
// 32(t%16) .. +31, value = bf16(e4m3(code) * scale[token][tile]), plus 4 rope channels
// copied as they are. Zero-filled rows (past the visible tokens) stay zero.
__device__ __forceinline__ void dequant_step(const char __attribute__((address_space(3)))* f8,
                                             char __attribute__((address_space(3)))* dst, int tid) {
  asm volatile("" : "+v"(tid));
  const int u = tid >> 4, cg = tid & 15;
  const char __attribute__((address_space(3)))* row = f8 + u * kF8Row;
  const u32x4 c0 = *(const u32x4 __attribute__((address_space(3)))*)(row + 32 * cg);
  const u32x4 c1 = *(const u32x4 __attribute__((address_space(3)))*)(row + 32 * cg + 16);
  const float sc = *(const float __attribute__((address_space(3)))*)(f8 + kF8StepBytes + 16 * u + 4 * (cg >> 2));
  const uint32_t rope_lo = *(const uint32_t __attribute__((address_space(3)))*)(row + kLat + 8 * cg);
  const uint32_t rope_hi = *(const uint32_t __attribute__((address_space(3)))*)(row + kLat + 8 * cg + 4);
  uint32_t w[8] = {c0[0], c0[1], c0[2], c0[3], c1[0], c1[1], c1[2], c1[3]};
  bf16x2 o[16];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], false);
    const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[j], true);
    o[2 * j][0] = (__bf16)(lo[0] * sc);
    o[2 * j][1] = (__bf16)(lo[1] * sc);
    o[2 * j + 1][0] = (__bf16)(hi[0] * sc);
    o[2 * j + 1][1] = (__bf16)(hi[1] * sc);
  }
  char __attribute__((address_space(3)))* drow = dst + u * kRowBytes;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int ch = 4 * cg + c;   // logical 16-B chunk of the 1152-B row
    u32x4 v;
    v[0] = __builtin_bit_cast(uint32_t, o[4 * c + 0]);
    v[1] = __builtin_bit_cast(uint32_t, o[4 * c + 1]);
    v[2] = __builtin_bit_cast(uint32_t, o[4 * c + 2]);
    v[3] = __builtin_bit_cast(uint32_t, o[4 * c + 3]);
    *(u32x4 __attribute__((address_space(3)))*)(drow + 16 * ((ch & ~7) | ((ch & 7) ^ swz(u)))) = v;
  }
  // rope: logical bytes 1024 + 8cg = chunk 64 + cg/2, half cg&1
  typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
  u32x2 r;
  r[0] = rope_lo;
  r[1] = rope_hi;
  *(u32x2 __attribute__((address_space(3)))*)(drow + 16 * (64 + ((cg >> 1) ^ swz(u))) + 8 * (cg & 1)) = r;
}

constexpr int kQkAhead = 4;   // score-operand reads in flight ahead of the MFMA consuming them
constexpr int kPvAhead = 2;   // P-operand reads in flight ahead of the value MFMAs

// LDS byte offset (inside a slot) of score tile t: token tile t%2, 32-channel k-step t/2
__device__ __forceinline__ int qk_off(const int* qk_b, int t) {
  const int ks = t >> 1, mt = t & 1;
  return mt * 16 * kRowBytes + qk_b[ks & 1] + 128 * (ks >> 1);
}

// Lanes l, l^16, l^32, l^48 hold the same query row (16x16 MFMA output layout).
__device__ __forceinline__ float max_across_quarters(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  u = __float_as_uint(x);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_across_quarters(float x) {
  unsigned u = __float_as_uint(x);
  auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  u = __float_as_uint(x);
  r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}


template <bool kFp8>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(
    const __bf16* __restrict__ q_ptr, const char* __restrict__ kv_ptr, const float* __restrict__ kv_scales,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ plan, float* __restrict__ ws, float* __restrict__ out_ptr,
    float* __restrict__ lse_ptr, Scalars a) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = xcd_worker();
  if (plan[kHMagic] != kPlanMagic || plan[kHWorkers] != (int)gridDim.x || plan[kHBatch] != a.batch ||
      plan[kHSq] != a.s_q || plan[kHHeads] != a.heads || plan[kHCausal] != a.causal)
    return;
  const int n_items = plan[kHItems];
  const int32_t* wr = plan + plan_workers_off(n_items) + kWorkerWords * worker;
  const int kb = wr[0], pb = wr[1], ke = wr[2], pe = wr[3];
  int k_last = pe > 0 ? ke : ke - 1;
  k_last = k_last < n_items - 1 ? k_last : n_items - 1;
  if (kb >= n_items || k_last < kb) return;

  // ---- per-lane LDS addressing (byte offsets inside a ring slot), rebuilt from an opaque
  // lane id at the start of each use so that it does not occupy registers across the loop
  // scores, A = Z[16 tokens x 32 channels]: lane reads token l%16, chunk 4ks + l/16
  // chunk ch = 4ks + g (g = lane>>4) sits at (ch & ~7) | ((ch & 7) ^ swz(token)); swz(u) == swz(u+16)
  auto qk_addr = [&](int* qk_b) {
    int l = lane;
    asm volatile("" : "+v"(l));
    const int tok = l & 15, g = l >> 4;
#pragma unroll
    for (int x = 0; x < 2; ++x) qk_b[x] = tok * kRowBytes + 16 * ((4 * x + g) ^ swz(tok));
  };
  // values, A = Z^T via transposing reads: lane j of 16-lane group G reads token
  // 16q + 8(G>>1) + 4e + (j>>2), channels 64w + 32mt + 16(G&1) + 4(j&3) .. +3
  auto pv_addr = [&](int (*pv_base)[2]) {   // [token half e][channel tile mt]
    int l = lane;
    asm volatile("" : "+v"(l));
    const int G = l >> 4, j = l & 15;
    const int u0 = 8 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int u = 4 * e + u0;                                  // token in the 16-token k-step
        const int ch = 8 * wave + 4 * mt + 2 * (G & 1) + ((j & 3) >> 1);   // 16-B chunk index
        pv_base[e][mt] = u * kRowBytes + 16 * ((ch & ~7) | ((ch & 7) ^ swz(u))) + 8 * (j & 1);
      }
  };
  using L = Lds<kFp8>;
  char __attribute__((address_space(3)))* pbuf = lds + L::kOffP;
  float __attribute__((address_space(3)))* alpha_s = (float __attribute__((address_space(3)))*)(lds + L::kOffAlpha);
  float __attribute__((address_space(3)))* stat_m = (float __attribute__((address_space(3)))*)(lds + L::kOffStat);
  float __attribute__((address_space(3)))* stat_l = stat_m + kRowsPerTile;

  const int rows_total = a.s_q * a.heads;
  // Q^T B-operand (16x16x32) of item k: lane holds query row 16*wave + (lane & 15) of the
  // item's tile, channels 32ks + 8(lane>>4) .. +7. The next item's rows are loaded right
  // after the current item's finalize.
  bf16x8 qreg[18];
  int q_item = -1;
  auto load_q = [&](int k) {
    int l = lane;   // opaque: a hoisted per-lane address would be spilled
    asm volatile("" : "+v"(l));
    const int32_t* it = plan + plan_items_off() + kItemWords * k;
    const int g_row = kRowsPerTile * it[kITile] + 16 * wave + (l & 15);
    const bool ok = g_row < rows_total;
    const int jt = ok ? g_row / a.heads : 0;
    const int hd = ok ? g_row - jt * a.heads : 0;
    // rows past the last query row (a partial tile) compute with a copy of the tile's first
    // row: every output column of the MFMAs depends on its own row only, and the finalize
    // writes no such row
    const __bf16* qrow = q_ptr + ((int64_t)(it[kISeq] * a.s_q + jt) * a.heads + hd) * kDqk + 8 * (l >> 4);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qreg[ks] = *reinterpret_cast<const bf16x8*>(qrow + 32 * ks);
    q_item = k;
  };
  load_q(kb);

  // ---- load cursor; the first kLoadSlots-1 (bf16) or kLoadSlots (fp8) steps are issued
  // up front, then one step per compute region (its DMA instructions spread between the
  // score MFMAs)
  constexpr int kLoadSlots = kFp8 ? kF8Slots : kNBuf;
  constexpr int kLoadBase = kFp8 ? L::kOffF8 : 0;
  constexpr int kLoadSlotBytes = kFp8 ? kF8SlotBytes : kBufBytes;
  LoadCursor lc;
  cursor_enter(lc, plan, kb, kb, pb, ke, pe);
  auto settle = [&]() {
    while (lc.k <= k_last && lc.hh >= lc.hh1) {
      if (lc.k == k_last) {
        lc.k = k_last + 1;
        break;
      }
      cursor_enter(lc, plan, lc.k + 1, kb, pb, ke, pe);
    }
  };
  settle();
  if (lc.k <= k_last) cursor_fetch(lc, a, block_table);
  int load_slot = 0;
  int issued_ahead = 0;   // steps issued whose data the compute loop has not consumed yet
  auto advance = [&]() {
    ++issued_ahead;
    load_slot = load_slot + 1 == kLoadSlots ? 0 : load_slot + 1;
    ++lc.hh;
    settle();
    if (lc.k <= k_last) cursor_fetch(lc, a, block_table);
  };
  const uint32_t lds_u32 = (uint32_t)(uintptr_t)lds;
#pragma unroll 1
  for (int i = 0; i < (kFp8 ? kF8Slots : kNBuf - 1); ++i) {
    if (lc.k <= k_last) {
      issue_step<kFp8>(cursor_rsrc<kFp8>(lc, a, kv_ptr, kv_scales), lds_u32 + kLoadBase + load_slot * kLoadSlotBytes,
                       lane, wave);
      advance();
    }
  }

  int comp_slot = 0;   // bf16 slot of the segment's current step
  int conv_slot = 0;   // fp8: staging slot of the next step to dequantise

#pragma unroll 1
  for (int k = kb; k <= k_last; ++k) {
    const Seg sg = seg_of(plan, k, kb, pb, ke, pe);
    const int32_t* it = plan + plan_items_off() + kItemWords * k;

    // ---- number of keys visible to this lane's query row (16*wave + (lane & 15))
    int lim = 0;
    {
      const int g_row = kRowsPerTile * it[kITile] + 16 * wave + (lane & 15);
      if (g_row < rows_total) {
        int t = seqlens[it[kISeq]];
        t = t < 0 ? 0 : t;
        const int cap = a.max_pages * kPage;
        t = t > cap ? cap : t;
        lim = t;
        if (a.causal) {
          lim = t - a.s_q + 1 + g_row / a.heads;
          lim = lim < 0 ? 0 : (lim > t ? t : lim);
        }
      }
    }
    if (q_item != k) load_q(k);   // (after an item with no steps)

    f32x16 oacc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) oacc[mt][nt] = f32x16{};
    float m_run = -INFINITY;   // log2 domain
    float l_run = 0.f;
    const int nsteps = sg.hh1 - sg.hh0;

    // --- pipeline pieces -------------------------------------------------------------
    // scores of one step: S^T[32 tokens x 16 rows] as two 16x16 tiles; 36 tiles
    // t = (k-step t/2, token tile t%2), operand reads kQkAhead tiles ahead of their MFMA
    auto scores = [&](const char __attribute__((address_space(3)))* zb, f32x4* sacc, bool load, const StepRsrc& rs,
                      uint32_t slot) {
      sacc[0] = f32x4{};
      sacc[1] = f32x4{};
      int qk_b[2];
      qk_addr(qk_b);
      bf16x8 aring[kQkAhead];
#pragma unroll
      for (int t = 0; t < kQkAhead; ++t) aring[t] = lds_b128(zb + qk_off(qk_b, t));
#pragma unroll
      for (int t = 0; t < 36; ++t) {
        const bf16x8 cur = aring[t % kQkAhead];
        if (t + kQkAhead < 36) aring[t % kQkAhead] = lds_b128(zb + qk_off(qk_b, t + kQkAhead));
        sacc[t & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cur, qreg[t >> 1], sacc[t & 1], 0, 0, 0);
        if (t % L::kIssueEvery == 0 && load) issue_one<kFp8>(rs, slot, t / L::kIssueEvery, lane, wave);
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // mask + online softmax (log2 domain) of step hh; lane: row my_row, tokens
    // 16mt + 4(lane>>4) + v. Returns P as bf16 and the row's rescale factor. Branch-free
    // (the lazy rescale is a select), so it can be scheduled among the value MFMAs; with
    // live == false it leaves the running state untouched.
    auto softmax = [&](const f32x4* sacc, int hh, bool live, bf16x4* pk, float* alpha_out) {
      const int key0 = kStep * hh + 4 * (lane >> 4);
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const float sv = sacc[mt][v] * a.scale_log2;
          x[4 * mt + v] = (key0 + 16 * mt + v) < lim ? sv : -INFINITY;
          mx = fmaxf(mx, x[4 * mt + v]);
        }
      mx = max_across_quarters(mx);
      // move the reference max only when it grows by more than 2^kTau (O is still 0 while
      // the reference is -inf, so no rescale is needed then)
      const bool move = live && (mx > m_run + kTau);
      const float alpha = (move && m_run != -INFINITY) ? exp2f(m_run - mx) : 1.f;
      const float m_new = move ? mx : m_run;
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      float psum = 0.f;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i] - m_use);
        psum += p;
        pk[i >> 2][i & 3] = (__bf16)p;
      }
      psum = sum_across_quarters(psum);
      const float l_new = alpha * l_run + psum;
      m_run = m_new;
      l_run = live ? l_new : l_run;
      *alpha_out = alpha;
    };
    // addresses recomputed from an opaque lane id: kept live they would be spilled, and a
    // scratch reload inside the step loop waits vmcnt(0) (draining the DMA ring)
    auto publish = [&](const bf16x4* pk, float alpha) {
      int l = lane;
      asm volatile("" : "+v"(l));
      const int row = 16 * wave + (l & 15);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        *(bf16x4 __attribute__((address_space(3)))*)(pbuf + row * kPRowBytes + 2 * (16 * mt + 4 * (l >> 4))) = pk[mt];
      if (l < 16) alpha_s[row] = alpha;
    };
    // O^T[64 channels of this wave][128 rows] = alpha O^T + Z^T P^T for one step; the
    // softmax of the next step (VALU) is issued among these MFMAs
    auto rescale = [&]() {
      float al[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) al[nt] = alpha_s[32 * nt + (lane & 31)];
      const bool any = __ballot(al[0] != 1.f || al[1] != 1.f || al[2] != 1.f || al[3] != 1.f) != 0;
      if (any) {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) oacc[mt][nt] *= al[nt];
      }
    };
    auto values_and_softmax = [&](const char __attribute__((address_space(3)))* zb, const f32x4* sacc, int hh_next,
                                  bool live, bf16x4* pk, float* alpha_out) {
      // the value MFMAs get issue priority over the score tiles of the SIMD's other wave
      __builtin_amdgcn_s_setprio(1);
      // 8 (k-step q, row tile nt) pairs, 2 MFMAs each; P operands one pair ahead, the
      // transposed Z^T operands of k-step 1 read during k-step 0
      const char __attribute__((address_space(3)))* prow = pbuf + (lane & 31) * kPRowBytes + 16 * (lane >> 5);
      int pv_base[2][2];
      pv_addr(pv_base);
      bf16x8 av[2][2];
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const bf16x4 lo = lds_tr16(zb + pv_base[0][mt]);
        const bf16x4 hi = lds_tr16(zb + pv_base[1][mt]);
        av[0][mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      }
      // P operands kPvAhead pairs ahead of their MFMAs
      bf16x8 pring[kPvAhead];
#pragma unroll
      for (int j = 0; j < kPvAhead; ++j) pring[j] = lds_b128(prow + (j & 3) * 32 * kPRowBytes + 32 * (j >> 2));
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int q = j >> 2, nt = j & 3;
        const bf16x8 bp = pring[j % kPvAhead];
        if (j + kPvAhead < 8)
          pring[j % kPvAhead] = lds_b128(prow + ((j + kPvAhead) & 3) * 32 * kPRowBytes + 32 * ((j + kPvAhead) >> 2));
        if (j == 1) {
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
            const bf16x4 lo = lds_tr16(zb + kRowBytes * 16 + pv_base[0][mt]);
            const bf16x4 hi = lds_tr16(zb + kRowBytes * 16 + pv_base[1][mt]);
            av[1][mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          }
        }
#pragma unroll
        for (int mt = 0; mt < 2; ++mt)
          oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[q][mt], bp, oacc[mt][nt], 0, 0, 0);
      }
      softmax(sacc, hh_next, live, pk, alpha_out);
      // interleave: each value MFMA is followed by a few VALU (softmax) and one LDS read
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);   // VALU
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // wait until this wave's DMA of the oldest unconsumed step has landed (younger
    // steps stay in flight)
    auto consume = [&]() {
      --issued_ahead;
      if (wave < L::kLong) {
        if (issued_ahead >= 2) wait_vmcnt<2 * (L::kDmaBase + 1)>();
        else if (issued_ahead == 1) wait_vmcnt<L::kDmaBase + 1>();
        else wait_vmcnt<0>();
      } else {
        if (issued_ahead >= 2) wait_vmcnt<2 * L::kDmaBase>();
        else if (issued_ahead == 1) wait_vmcnt<L::kDmaBase>();
        else wait_vmcnt<0>();
      }
    };
    // fp8: dequantise the oldest staged step into bf16 slot ws
    auto dequant = [&](int wslot) {
      dequant_step(lds + L::kOffF8 + conv_slot * kF8SlotBytes, lds + wslot * kBufBytes, (int)threadIdx.x);
      conv_slot = conv_slot + 1 == kF8Slots ? 0 : conv_slot + 1;
    };
    // the step issued in a compute region goes into the slot freed by the barrier before it
    auto load_next = [&](bool& load, StepRsrc& rs, uint32_t& slot) {
      load = lc.k <= k_last;
      if (load) rs = cursor_rsrc<kFp8>(lc, a, kv_ptr, kv_scales);
      slot = lds_u32 + kLoadBase + load_slot * kLoadSlotBytes;
    };

    // --- segment pipeline: after barrier B2(i), one region computes the scores of step
    // i+1 and the value product of step i, then the softmax of step i+1 (its VALU work
    // overlaps the value MFMAs still in flight), and issues the loads of a step kNBuf-1
    // ahead into the slot freed at B1(i). Between B1(i+1) and B2(i+1) P/alpha of step i+1
    // are published and the data of step i+2 is awaited.
    if (nsteps > 0) {
      f32x4 sacc[2];
      bf16x4 pk[2];
      float alpha = 1.f;
      const StepRsrc no_rs = {};
      const char __attribute__((address_space(3)))* zcur = lds + comp_slot * kBufBytes;
      if constexpr (!kFp8) {
        consume();                     // data of step 0
        barrier_lds();                 // ... visible; previous segment fully done
        scores(zcur, sacc, false, no_rs, 0u);
        softmax(sacc, sg.hh0, true, pk, &alpha);
        publish(pk, alpha);
        if (nsteps > 1) consume();     // data of step 1
        barrier_lds();                 // B2(0)
      } else {
        consume();                     // staged data of steps 0 and 1
        if (nsteps > 1) consume();
        barrier_lds();
        dequant(comp_slot);
        if (nsteps > 1) dequant(comp_slot ^ 1);
        barrier_lds();
        scores(zcur, sacc, false, no_rs, 0u);
        softmax(sacc, sg.hh0, true, pk, &alpha);
        publish(pk, alpha);
        barrier_lds();                 // B2(0)
      }
#pragma unroll 1
      for (int i = 0; i < nsteps; ++i) {
        const int cs_next = comp_slot + 1 == L::kWork ? 0 : comp_slot + 1;
        const char __attribute__((address_space(3)))* znext = lds + cs_next * kBufBytes;
        const bool more = i + 1 < nsteps;
        bool load;
        StepRsrc rs;
        uint32_t lslot;
        load_next(load, rs, lslot);
        if (more) {
          scores(znext, sacc, load, rs, lslot);
        } else if (load) {
          issue_step<kFp8>(rs, lslot, lane, wave);
        }
        if (load) advance();
        rescale();
        values_and_softmax(zcur, sacc, sg.hh0 + i + 1, more, pk, &alpha);
        if (more) {
          if constexpr (!kFp8) {
            barrier_lds();             // B1(i+1): P(i), alpha(i) and step i's slot are free
            publish(pk, alpha);
            if (i + 2 < nsteps) consume();   // data of step i+2
            barrier_lds();             // B2(i+1)
          } else {
            if (i + 2 < nsteps) consume();   // staged data of step i+2
            barrier_lds();             // B1(i+1): P(i), alpha(i) and step i's bf16 slot are free
            publish(pk, alpha);
            if (i + 2 < nsteps) dequant(comp_slot);
            barrier_lds();             // B2(i+1)
          }
        }
        comp_slot = cs_next;
        zcur = znext;
      }
    }

    // ---- finalize: exchange (m, l) per row, write out/lse or a partial. Addresses are
    // rebuilt here from an opaque lane id and the plan record (kept live across the step
    // loop they would be spilled, and a scratch reload waits for every load in flight).
    {
      int l = lane;
      asm volatile("" : "+v"(l));
      const int32_t* itf = plan + plan_items_off() + kItemWords * k;
      const int f_seq = itf[kISeq], f_tile = itf[kITile];
      const bool split = itf[kINsplits] > 1;
      const int slot = split ? itf[kISlot] + (worker - itf[kIOwner]) : 0;
      const int mrow = 16 * wave + (l & 15);
      if (l < 16) {
        stat_m[mrow] = m_run;
        stat_l[mrow] = l_run;
      }
      barrier_lds();
      if (split) {
        // partial: bf16, each store one 512-B run in register order (see combine_kernel)
        char* part = reinterpret_cast<char*>(ws) + (int64_t)slot * kSlotBytes;
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const float lsum = stat_l[32 * nt + (l & 31)];
          const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              bf16x4 v;
              v[0] = (__bf16)(oacc[mt][nt][4 * g + 0] * inv);
              v[1] = (__bf16)(oacc[mt][nt][4 * g + 1] * inv);
              v[2] = (__bf16)(oacc[mt][nt][4 * g + 2] * inv);
              v[3] = (__bf16)(oacc[mt][nt][4 * g + 3] * inv);
              const int frag = (((wave * 4 + nt) * 2 + mt) * 4 + g) * 64 + l;
              *reinterpret_cast<bf16x4*>(part + 8 * (int64_t)frag) = v;
            }
        }
      } else {
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const int row = 32 * nt + (l & 31);
          const int grow = kRowsPerTile * f_tile + row;
          if (grow >= rows_total) continue;
          const float lsum = stat_l[row];
          const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
          const int jt = grow / a.heads, hd = grow - jt * a.heads;
          float* dst = out_ptr + ((int64_t)(f_seq * a.s_q + jt) * a.heads + hd) * kLat;
#pragma unroll
          for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
            for (int g = 0; g < 4; ++g) {
              const int c = 64 * wave + 32 * mt + 8 * g + 4 * (l >> 5);
              f32x4 v;
              v[0] = oacc[mt][nt][4 * g + 0] * inv;
              v[1] = oacc[mt][nt][4 * g + 1] * inv;
              v[2] = oacc[mt][nt][4 * g + 2] * inv;
              v[3] = oacc[mt][nt][4 * g + 3] * inv;
              *reinterpret_cast<f32x4*>(dst + c) = v;
            }
          }
        }
      }
      const int grow = kRowsPerTile * f_tile + mrow;
      if (l < 16 && grow < rows_total) {
        const float m = (m_run == -INFINITY) ? 0.f : m_run;
        const float lse_v = l_run > 0.f ? (m + __log2f(l_run)) * 0.6931471805599453f : -INFINITY;
        const int jt = grow / a.heads, hd = grow - jt * a.heads;
        if (split) reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + (int64_t)slot * kSlotBytes + kSlotPartBytes)[mrow] = lse_v;
        else lse_ptr[(int64_t)(f_seq * a.s_q + jt) * a.heads + hd] = lse_v;
      }
      barrier_lds();
    }
    // the next item's query rows: the youngest loads in flight, so waiting for them (at
    // their first use) leaves no ring step behind
    if (k < k_last) load_q(k + 1);
  }
}

// Merge the partials of split items: lse = log sum_k e^{lse_k}, out = sum_k e^{lse_k - lse} O_k
// (max-shifted; parts with lse = -inf carry no weight). One block per (split item, 32-row
// group nt). A partial is stored in the decode kernel's register order: value
// (row 32nt + (lane & 31), channel 64w + 32mt + 8g + 4(lane >> 5) + e) of a slot sits at
// bf16 index 4 * ((((w * 4 + nt) * 2 + mt) * 4 + g) * 64 + lane) + e, so a block reads each
// part as 8 contiguous 4-KiB runs. The merged rows go through LDS to leave as whole rows.
constexpr int kCombMaxSplits = 256;
constexpr int kCombThreads = 256;

__global__ __launch_bounds__(kCombThreads) void combine_kernel(const int32_t* __restrict__ plan,
                                                               const char* __restrict__ ws, float* __restrict__ out,
                                                               float* __restrict__ lse, int s_q, int heads) {
  __shared__ float wts[32][kCombMaxSplits];
  __shared__ float tile_out[32][kLat + 4];   // +4: rows start on different banks
  __shared__ float row_m[32], row_t[32];
  if (plan[kHMagic] != kPlanMagic) return;
  const int n_split = plan[kHSplitItems];
  const int n_items = plan[kHItems];
  if ((int)blockIdx.x >= n_split) return;
  const int32_t* sr = plan + plan_split_off(n_items, plan[kHWorkers]) + kSplitWords * blockIdx.x;
  const int seq = sr[kSSeq], tile = sr[kSTile], ns_all = sr[kSNsplits], slot0 = sr[kSSlot];
  const int rows_total = s_q * heads;
  const int nt = blockIdx.y;
  if (kRowsPerTile * tile + 32 * nt >= rows_total) return;
  const int tid = threadIdx.x;
  // this thread's 16 fragments: p = tid + 256 j -> (w, mt, g, lane)
  f32x4 acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_old = -INFINITY;   // per row, kept by threads tid < 32
  float t_old = 0.f;
  for (int s0 = 0; s0 < ns_all; s0 += kCombMaxSplits) {
    const int ns = ns_all - s0 < kCombMaxSplits ? ns_all - s0 : kCombMaxSplits;
    __syncthreads();
    for (int idx = tid; idx < 32 * ns; idx += kCombThreads) {
      const int r = idx / ns, sp = idx - r * ns;
      wts[r][sp] = reinterpret_cast<const float*>(ws + (int64_t)(slot0 + s0 + sp) * kSlotBytes + kSlotPartBytes)[32 * nt + r];
    }
    __syncthreads();
    // per row: new running max, weights relative to it, rescale of the earlier chunks
    if (tid < 32) {
      float m = m_old;
      for (int sp = 0; sp < ns; ++sp) m = fmaxf(m, wts[tid][sp]);
      const float safe = m == -INFINITY ? 0.f : m;
      const float resc = m_old == -INFINITY ? 0.f : __expf(m_old - safe);
      float tot = t_old * resc;
      for (int sp = 0; sp < ns; ++sp) {
        const float l = wts[tid][sp];
        const float wgt = l == -INFINITY ? 0.f : __expf(l - safe);
        wts[tid][sp] = wgt;
        tot += wgt;
      }
      m_old = m;
      t_old = tot;
      row_m[tid] = resc;   // (rescale of the accumulators, read below)
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) acc[j] *= row_m[(tid + 256 * j) & 31];
    for (int sp = 0; sp < ns; ++sp) {
      const __bf16* part = reinterpret_cast<const __bf16*>(ws + (int64_t)(slot0 + s0 + sp) * kSlotBytes);
      bf16x4 v[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const int p = tid + 256 * j;
        const int lane = p & 63, g = (p >> 6) & 3, mt = (p >> 8) & 1, w = p >> 9;
        const int frag = (((w * 4 + nt) * 2 + mt) * 4 + g) * 64 + lane;
        v[j] = *reinterpret_cast<const bf16x4*>(part + 4 * (int64_t)frag);
      }
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float wgt = wts[(tid + 256 * j) & 31][sp];
        acc[j][0] += wgt * (float)v[j][0];
        acc[j][1] += wgt * (float)v[j][1];
        acc[j][2] += wgt * (float)v[j][2];
        acc[j][3] += wgt * (float)v[j][3];
      }
    }
  }
  if (tid < 32) {
    row_t[tid] = t_old;
    row_m[tid] = m_old;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int p = tid + 256 * j;
    const int lane = p & 63, g = (p >> 6) & 3, mt = (p >> 8) & 1, w = p >> 9;
    const int r = lane & 31, c = 64 * w + 32 * mt + 8 * g + 4 * (lane >> 5);
    const float t = row_t[r];
    const float inv = t > 0.f ? 1.f / t : 0.f;
    *reinterpret_cast<f32x4*>(&tile_out[r][c]) = acc[j] * inv;
  }
  __syncthreads();
  // whole rows out: 32 rows x 128 float4
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const int idx = tid + 256 * j;
    const int r = idx >> 7, c4 = (idx & 127) * 4;
    const int grow = kRowsPerTile * tile + 32 * nt + r;
    if (grow >= rows_total) continue;
    const int jt = grow / heads, hd = grow - jt * heads;
    const int64_t orow = (int64_t)(seq * s_q + jt) * heads + hd;
    *reinterpret_cast<f32x4*>(out + orow * kLat + c4) = *reinterpret_cast<const f32x4*>(&tile_out[r][c4]);
    if (c4 == 0) {
      const float t = row_t[r];
      lse[orow] = t > 0.f ? row_m[r] + __logf(t) : -INFINITY;
    }
  }
}

template <bool kFp8>
hipError_t launch_decode(const DecodeArgs& a, hipStream_t stream) {
  // the LDS opt-in is per device; remember it per device id
  static thread_local int configured = -1;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (configured != dev) {
    e = hipFuncSetAttribute((const void*)decode_kernel<kFp8>, hipFuncAttributeMaxDynamicSharedMemorySize,
                            Lds<kFp8>::kBytes);
    if (e != hipSuccess) return e;
    configured = dev;
  }
  hipLaunchKernelGGL(decode_kernel<kFp8>, dim3(a.workers), dim3(kThreads), Lds<kFp8>::kBytes, stream,
                     reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const char*>(a.kv), a.kv_scales,
                     a.block_table, a.seqlens, a.plan, a.ws, a.out, a.lse, scalars_of(a));
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) { return launch_decode<true>(a, stream); }

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const int max_split = a.workers;   // split items <= active workers - 1
  hipLaunchKernelGGL(combine_kernel, dim3(max_split, kRowsPerTile / 32), dim3(kCombThreads), 0, stream, a.plan,
                     reinterpret_cast<const char*>(a.ws), a.out, a.lse, a.s_q, a.heads);
  return hipGetLastError();
}

}  // namespace mla
