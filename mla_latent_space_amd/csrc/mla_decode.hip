// Latent-space MLA decode kernels for gfx950 (MI355X).
//
// Page "Mla Analysis", section "Absorption Trick (FlashMLA)": scores are Qz . Z^T with the
// absorbed 576-wide queries, and the value is the latent row itself, so one pass over the
// paged latent cache gives O_latent = softmax(scale Qz Z^T) Z[:, :512] and a log-sum-exp
// per (token, head). Section "Cost Models": 2bhst(2k+p) FLOPs over w(bhs(2k+p) + bt(k+p))
// bytes, about 228 FLOP/byte at s=1 -- on MI355X (ridge ~315 FLOP/byte for bf16) the s=1
// decode is bound by HBM, so the design streams each cached token row from HBM exactly
// once per 128-row tile and keeps the matrix cores busy underneath.
//
// Work-group = 4 waves = one persistent worker of the split plan, one per compute unit.
//  * LDS ring of 4 steps x 32 tokens x 1152 B, filled by LDS-DMA buffer loads (16 B per
//    lane, coalesced). The buffer descriptor's record count stops at the last visible
//    token, so masked tail slots arrive as zeros (poisoned slots never reach the MFMAs).
//    Rows are XOR-swizzled in 16-B chunks (chunk ^= (token >> 1) & 7) so that both LDS
//    read patterns below are free of bank conflicts.
//  * Scores: wave w owns query rows 32w..32w+31 of the tile and computes S^T = Z Q^T with
//    v_mfma_f32_32x32x16_bf16: A = 32 tokens x 16 channels read from LDS (ds_read_b128),
//    B = Q^T held in 144 VGPRs for the whole sequence segment.
//  * Online softmax in the S^T layout: each lane owns one query row and 16 of the 32
//    tokens, so row max / row sum are lane-local plus one permlane32 swap. The running
//    max is only moved when it grows by more than 2^8 (lazy rescale), so the accumulator
//    is rarely rescaled.
//  * P (bf16) goes through LDS already in the MFMA B-operand layout; value products are
//    split by channels: wave w owns O^T[128w .. 128w+127][all 128 rows] (256 acc regs),
//    A = Z^T via ds_read_b64_tr_b16 (transposing LDS read), B = P^T from LDS.
//  * Finalize writes out/lse directly, or a normalised partial + lse into the workspace
//    for items the plan split; the combine kernel merges those by log-sum-exp.
#include "mla_internal.h"

namespace mla {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(2))) float f32x2;
typedef __attribute__((ext_vector_type(4))) short i16x4;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4;
#define LDSP(T) __attribute__((address_space(3))) T*

constexpr int kThreads = 512;                  // 8 waves, two per SIMD
constexpr int kStep = 32;                      // tokens per pipeline step
constexpr int kNBuf = 4;                       // LDS ring depth
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kBufBytes = kStep * kRowBytes;   // 36864
constexpr int kDmaInstr = kBufBytes / 1024;    // 36 LDS-DMA instructions (1 KiB each) per step
constexpr int kDmaBase = kDmaInstr / 8;        // 4 per wave ...
constexpr int kDmaWavesLong = kDmaInstr % 8;   // ... and one more for waves 0..3
constexpr int kPRowBytes = 80;                 // P exchange row: 32 bf16 + 16 B pad (bank spread)
constexpr int kOffP = kNBuf * kBufBytes;       // P exchange: [128 rows][32 tokens] bf16
constexpr int kOffAlpha = kOffP + kRowsPerTile * kPRowBytes;  // 128 floats: per-row rescale of this step
constexpr int kOffFlag = kOffAlpha + 512;      // 8 ints: a wave rescaled this step
constexpr int kOffStat = kOffFlag + 32;        // 128 floats m, 128 floats l
constexpr int kLdsBytes = kOffStat + 1024;
static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
constexpr float kTau = 8.0f;                   // lazy rescale threshold (log2 units)
constexpr uint32_t kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit format, gfx9 family

__device__ __forceinline__ int swz(int u) { return (u >> 1) & 7; }

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Scalar kernel arguments (the pointers travel as separate __restrict__ parameters so the
// compiler can prove the plan and block table are never written and use scalar loads).
struct Scalars {
  int64_t num_pages;
  int max_pages, batch, s_q, heads, causal;
  float scale_log2;
};

inline Scalars scalars_of(const DecodeArgs& d) {
  Scalars s;
  s.num_pages = d.num_pages;
  s.max_pages = d.max_pages;
  s.batch = d.batch;
  s.s_q = d.s_q;
  s.heads = d.heads;
  s.causal = d.causal;
  s.scale_log2 = d.scale_log2;
  return s;
}

typedef __attribute__((ext_vector_type(4))) int i32x4;

// LDS-DMA: 64 lanes x 16 B from the buffer (byte offset voff per lane; offsets at or past
// num_records read as zero) into LDS at m0 + 16 * lane. Written as inline asm so that the
// compiler does not track it as a pending LDS write: it would otherwise wait vmcnt(0)
// before unrelated LDS reads and drain the prefetch ring. The kernel orders these loads
// itself with wait_vmcnt + barrier_lds. No register outputs (nothing is left in flight
// in a VGPR).
__device__ __forceinline__ void lds_dma_x4(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile(
      "s_mov_b32 m0, %0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds"
      :
      : "s"(__builtin_amdgcn_readfirstlane(lds_addr)), "v"(voff), "s"(rsrc)
      : "memory", "m0");
}

// Work-group barrier for LDS traffic only. __syncthreads() also orders the LDS-DMA loads
// still in flight (it waits vmcnt(0)), which would drain the prefetch ring at every
// barrier; here each wave waits for exactly the DMA steps it needs (wait_vmcnt) and this
// barrier only waits for its own ds_read/ds_write traffic. The empty asm statements keep
// the compiler from moving LDS accesses across the barrier.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(15 | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0) only
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Steps (32-token halves of pages) of item k that this worker processes.
struct Seg { int k, hh0, hh1; };

__device__ __forceinline__ Seg seg_of(const int32_t* plan, int k, int kb, int pb, int ke, int pe) {
  const int32_t* it = plan + plan_items_off() + kItemWords * k;
  const int vis = it[kIVis], pages = it[kIPages];
  const int lo = (k == kb) ? pb : 0;
  const int hi = (k == ke) ? pe : pages;
  const int nhalf = (vis + kStep - 1) / kStep;
  int h0 = 2 * lo, h1 = 2 * hi < nhalf ? 2 * hi : nhalf;
  if (h1 < h0) h1 = h0;
  Seg s; s.k = k; s.hh0 = h0; s.hh1 = h1;
  return s;
}

// Load cursor: walks the worker's steps in order, kNBuf-1 steps ahead of the compute loop.
struct LoadCursor {
  int k, hh, hh1;   // current item, next step to load, end step of that item
};

template <bool kFp8>
struct Loader;

template <>
struct Loader<false> {
  // Issue this wave's share of the 36 LDS-DMA loads of step (item k, half hh) into a ring slot.
  __device__ __forceinline__ static void issue(const Scalars& a, const char* __restrict__ kv,
                                               const int32_t* __restrict__ block_table,
                                               const int32_t* __restrict__ plan, int k, int hh,
                                               char __attribute__((address_space(3)))* lds_slot, int lane,
                                               int wave) {
    const int32_t* it = plan + plan_items_off() + kItemWords * k;
    const int seq = it[kISeq], vis = it[kIVis];
    const int pg = hh >> 1;
    int pid = -1;
    if (pg < a.max_pages) pid = block_table[(int64_t)seq * a.max_pages + pg];
    int valid = vis - kStep * hh;
    valid = valid > kStep ? kStep : valid;
    const bool ok = pid >= 0 && (int64_t)pid < a.num_pages && valid > 0;
    const char* base = kv +
                       (ok ? ((int64_t)pid * (kPage * kRowBytes) + (int64_t)(hh & 1) * kBufBytes) : 0);
    const uint64_t addr = reinterpret_cast<uint64_t>(base);
    i32x4 rsrc;
    rsrc[0] = (int)(uint32_t)addr;
    rsrc[1] = (int)((uint32_t)(addr >> 32) & 0xFFFF);   // stride 0
    rsrc[2] = ok ? valid * kRowBytes : 0;               // num_records: bytes past it read as 0
    rsrc[3] = (int)kRsrcWord3;
    const uint32_t lds_base = (uint32_t)(uintptr_t)lds_slot;
    // Instruction i (1 KiB, 64 lanes x 16 B, lane-linear in LDS) is issued by wave i % 8.
    // LDS chunk position p = 72u + pc holds logical chunk ch = pc ^ swz(u) of token u.
#pragma unroll
    for (int n = 0; n < kDmaBase + 1; ++n) {
      const int i = wave + 8 * n;
      if (n == kDmaBase && wave >= kDmaWavesLong) break;
      const int p = 64 * i + lane;
      const int u = p / 72, pc = p - 72 * u;
      const int ch = (pc & ~7) | ((pc & 7) ^ swz(u));
      const uint32_t voff = (uint32_t)(u * kRowBytes + 16 * ch);
      lds_dma_x4(lds_base + 1024u * (uint32_t)i, voff, rsrc);
    }
  }
};

__device__ __forceinline__ bf16x8 lds_b128(const char __attribute__((address_space(3)))* p) {
  u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)p;
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x4 lds_tr16(const char __attribute__((address_space(3)))* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP(i16x4))(p));
  return __builtin_bit_cast(bf16x4, v);
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
__global__ __launch_bounds__(kThreads, 1) void decode_kernel(
    const __bf16* __restrict__ q_ptr, const char* __restrict__ kv_ptr, const float* __restrict__ kv_scales,
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seqlens,
    const int32_t* __restrict__ plan, float* __restrict__ ws, float* __restrict__ out_ptr,
    float* __restrict__ lse_ptr, Scalars a) {
  extern __shared__ __attribute__((aligned(1024))) char smem_raw[];
  char __attribute__((address_space(3)))* lds = (char __attribute__((address_space(3)))*)smem_raw;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int worker = blockIdx.x;
  if (plan[kHMagic] != kPlanMagic || plan[kHWorkers] != (int)gridDim.x || plan[kHBatch] != a.batch ||
      plan[kHSq] != a.s_q || plan[kHHeads] != a.heads || plan[kHCausal] != a.causal)
    return;
  const int n_items = plan[kHItems];
  const int32_t* wr = plan + plan_workers_off(n_items) + kWorkerWords * worker;
  const int kb = wr[0], pb = wr[1], ke = wr[2], pe = wr[3];
  int k_last = pe > 0 ? ke : ke - 1;
  k_last = k_last < n_items - 1 ? k_last : n_items - 1;
  if (kb >= n_items || k_last < kb) return;

  // ---- per-lane LDS addressing (byte offsets inside a ring slot)
  // scores, A = Z[16 tokens x 32 channels]: lane reads token l%16, chunk 4ks + l/16
  // chunk ch = 4ks + g (g = lane>>4) sits at (ch & ~7) | ((ch & 7) ^ swz(token)); swz(u) == swz(u+16)
  int qk_b[2];
  {
    const int tok = lane & 15, g = lane >> 4;
#pragma unroll
    for (int x = 0; x < 2; ++x) qk_b[x] = tok * kRowBytes + 16 * ((4 * x + g) ^ swz(tok));
  }
  // values, A = Z^T via transposing reads: lane j of 16-lane group G reads token
  // 16q + 8(G>>1) + 4e + (j>>2), channels 64w + 32mt + 16(G&1) + 4(j&3) .. +3
  int pv_base[2][2];   // [token half e][channel tile mt]
  {
    const int G = lane >> 4, j = lane & 15;
    const int u0 = 8 * (G >> 1) + (j >> 2);
#pragma unroll
    for (int e = 0; e < 2; ++e)
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int u = 4 * e + u0;                                  // token in the 16-token k-step
        const int ch = 8 * wave + 4 * mt + 2 * (G & 1) + ((j & 3) >> 1);   // 16-B chunk index
        pv_base[e][mt] = u * kRowBytes + 16 * ((ch & ~7) | ((ch & 7) ^ swz(u))) + 8 * (j & 1);
      }
  }
  char __attribute__((address_space(3)))* pbuf = lds + kOffP;
  float __attribute__((address_space(3)))* alpha_s = (float __attribute__((address_space(3)))*)(lds + kOffAlpha);
  int __attribute__((address_space(3)))* flag_s = (int __attribute__((address_space(3)))*)(lds + kOffFlag);
  float __attribute__((address_space(3)))* stat_m = (float __attribute__((address_space(3)))*)(lds + kOffStat);
  float __attribute__((address_space(3)))* stat_l = stat_m + kRowsPerTile;

  // ---- prologue: issue the first kNBuf-1 steps
  auto settle = [&](LoadCursor& c) {
    while (c.k <= k_last && c.hh >= c.hh1) {
      ++c.k;
      if (c.k > k_last) break;
      const Seg s = seg_of(plan, c.k, kb, pb, ke, pe);
      c.hh = s.hh0; c.hh1 = s.hh1;
    }
  };
  LoadCursor lc;
  {
    const Seg s0 = seg_of(plan, kb, kb, pb, ke, pe);
    lc.k = kb; lc.hh = s0.hh0; lc.hh1 = s0.hh1;
  }
  settle(lc);
  int load_slot = 0;
  int issued_ahead = 0;   // steps issued whose data the compute loop has not consumed yet
#pragma unroll 1
  for (int i = 0; i < kNBuf - 1; ++i) {
    if (lc.k <= k_last) {
      Loader<kFp8>::issue(a, kv_ptr, block_table, plan, lc.k, lc.hh, lds + load_slot * kBufBytes, lane, wave);
      ++issued_ahead;
      load_slot = (load_slot + 1) & (kNBuf - 1);
      ++lc.hh;
      settle(lc);
    }
  }

  int comp_slot = 0;
  const int rows_total = a.s_q * a.heads;

#pragma unroll 1
  for (int k = kb; k <= k_last; ++k) {
    const Seg sg = seg_of(plan, k, kb, pb, ke, pe);
    const int32_t* it = plan + plan_items_off() + kItemWords * k;
    const int seq = it[kISeq], tile = it[kITile];
    const int nsplits = it[kINsplits], slot_base = it[kISlot], owner = it[kIOwner];

    // ---- this lane's query row for scores: row 16*wave + (lane & 15)
    const int my_row = 16 * wave + (lane & 15);
    const int g_row = kRowsPerTile * tile + my_row;
    const bool row_ok = g_row < rows_total;
    const int j_tok = row_ok ? g_row / a.heads : 0;
    const int head = row_ok ? g_row - j_tok * a.heads : 0;
    int lim = 0;
    if (row_ok) {
      int t = seqlens[seq];
      t = t < 0 ? 0 : t;
      const int cap = a.max_pages * kPage;
      t = t > cap ? cap : t;
      lim = t;
      if (a.causal) {
        lim = t - a.s_q + 1 + j_tok;
        lim = lim < 0 ? 0 : (lim > t ? t : lim);
      }
    }
    // Q^T B-operand (16x16x32): lane holds row (lane&15), channels 32ks + 8(lane>>4) .. +7
    bf16x8 qreg[18];
    {
      const __bf16* qrow = q_ptr +
                           ((int64_t)(seq * a.s_q + j_tok) * a.heads + head) * kDqk + 8 * (lane >> 4);
#pragma unroll
      for (int ks = 0; ks < 18; ++ks)
        qreg[ks] = row_ok ? *reinterpret_cast<const bf16x8*>(qrow + 32 * ks) : bf16x8{};
    }
    wait_vmcnt<0>();

    f32x16 oacc[2][4];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) oacc[mt][nt] = f32x16{};
    float m_run = -INFINITY;   // log2 domain
    float l_run = 0.f;

#pragma unroll 1
    for (int hh = sg.hh0; hh < sg.hh1; ++hh) {
      // wait for this step's data (later steps stay in flight), then make it visible
      --issued_ahead;
      if (wave < kDmaWavesLong) {
        if (issued_ahead >= 2) wait_vmcnt<2 * (kDmaBase + 1)>();
        else if (issued_ahead == 1) wait_vmcnt<kDmaBase + 1>();
        else wait_vmcnt<0>();
      } else {
        if (issued_ahead >= 2) wait_vmcnt<2 * kDmaBase>();
        else if (issued_ahead == 1) wait_vmcnt<kDmaBase>();
        else wait_vmcnt<0>();
      }
      barrier_lds();
      // refill the slot freed by the previous step
      if (lc.k <= k_last) {
        Loader<kFp8>::issue(a, kv_ptr, block_table, plan, lc.k, lc.hh, lds + load_slot * kBufBytes, lane, wave);
        ++issued_ahead;
        load_slot = (load_slot + 1) & (kNBuf - 1);
        ++lc.hh;
        settle(lc);
      }
      const char __attribute__((address_space(3)))* zb = lds + comp_slot * kBufBytes;

      // ---- scores S^T[32 tokens x 16 rows] as two 16x16 tiles
      f32x4 sacc[2] = {f32x4{}, f32x4{}};
#pragma unroll
      for (int ks = 0; ks < 18; ks += 2) {
        bf16x8 av[2][2];
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            av[e][mt] = lds_b128(zb + mt * 16 * kRowBytes + qk_b[(ks + e) & 1] + 128 * ((ks + e) >> 1));
#pragma unroll
        for (int e = 0; e < 2; ++e)
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            sacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[e][mt], qreg[ks + e], sacc[mt], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      // ---- mask + online softmax (log2 domain); lane: row my_row, tokens 16mt + 4(lane>>4) + v
      const int key0 = kStep * hh + 4 * (lane >> 4);
      float x[8];
      float mx = -INFINITY;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int key = key0 + 16 * mt + v;
          const float sv = sacc[mt][v] * a.scale_log2;
          x[4 * mt + v] = key < lim ? sv : -INFINITY;
          mx = fmaxf(mx, x[4 * mt + v]);
        }
      mx = max_across_quarters(mx);
      float alpha = 1.f;
      bool rescaled = false;
      if (mx > m_run + kTau) {
        alpha = (m_run == -INFINITY) ? 0.f : exp2f(m_run - mx);
        rescaled = m_run != -INFINITY;
        m_run = mx;
      }
      const float m_use = (m_run == -INFINITY) ? 0.f : m_run;
      float psum = 0.f;
      bf16x4 pk[2];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float p = __builtin_amdgcn_exp2f(x[i] - m_use);
        psum += p;
        pk[i >> 2][i & 3] = (__bf16)p;
      }
      psum = sum_across_quarters(psum);
      l_run = alpha * l_run + psum;
      // publish P as [row][token] (80-byte rows), alpha and the rescale flag
#pragma unroll
      for (int mt = 0; mt < 2; ++mt)
        *(bf16x4 __attribute__((address_space(3)))*)(pbuf + my_row * kPRowBytes + 2 * (16 * mt + 4 * (lane >> 4))) =
            pk[mt];
      const uint64_t any = __ballot(rescaled);
      if (lane < 16) alpha_s[my_row] = rescaled ? alpha : 1.f;
      if (lane == 0) flag_s[wave] = any != 0;
      barrier_lds();

      // ---- O^T[64 channels of this wave][128 rows] += Z^T P^T
      {
        const u32x4 f0 = *(const u32x4 __attribute__((address_space(3)))*)flag_s;
        const u32x4 f1 = *(const u32x4 __attribute__((address_space(3)))*)(flag_s + 4);
        if ((f0[0] | f0[1] | f0[2] | f0[3] | f1[0] | f1[1] | f1[2] | f1[3]) != 0) {
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) {
            const float al = alpha_s[32 * nt + (lane & 31)];
#pragma unroll
            for (int mt = 0; mt < 2; ++mt) oacc[mt][nt] *= al;
          }
        }
      }
#pragma unroll
      for (int q = 0; q < 2; ++q) {
        bf16x8 av[2];
#pragma unroll
        for (int mt = 0; mt < 2; ++mt) {
          const bf16x4 lo = lds_tr16(zb + kRowBytes * 16 * q + pv_base[0][mt]);
          const bf16x4 hi = lds_tr16(zb + kRowBytes * 16 * q + pv_base[1][mt]);
          av[mt] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        }
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {
          const bf16x8 bp = lds_b128(pbuf + (32 * nt + (lane & 31)) * kPRowBytes + 2 * (16 * q + 8 * (lane >> 5)));
#pragma unroll
          for (int mt = 0; mt < 2; ++mt)
            oacc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], bp, oacc[mt][nt], 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      comp_slot = (comp_slot + 1) & (kNBuf - 1);
    }

    // ---- finalize: exchange (m, l) per row, write out/lse or a partial
    if (lane < 16) {
      stat_m[my_row] = m_run;
      stat_l[my_row] = l_run;
    }
    barrier_lds();
    const bool split = nsplits > 1;
    const int slot = split ? slot_base + (worker - owner) : 0;
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) {
      const int row = 32 * nt + (lane & 31);
      const int grow = kRowsPerTile * tile + row;
      if (grow >= rows_total) continue;
      const float l = stat_l[row];
      const float inv = l > 0.f ? 1.f / l : 0.f;
      const int jt = grow / a.heads, hd = grow - jt * a.heads;
      float* dst = split ? (ws + (int64_t)slot * kSlotFloats + (int64_t)row * kLat)
                         : (out_ptr + ((int64_t)(seq * a.s_q + jt) * a.heads + hd) * kLat);
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int c = 64 * wave + 32 * mt + 8 * g + 4 * (lane >> 5);
          f32x4 v;
          v[0] = oacc[mt][nt][4 * g + 0] * inv;
          v[1] = oacc[mt][nt][4 * g + 1] * inv;
          v[2] = oacc[mt][nt][4 * g + 2] * inv;
          v[3] = oacc[mt][nt][4 * g + 3] * inv;
          *reinterpret_cast<f32x4*>(dst + c) = v;
        }
      }
    }
    if (lane < 16 && row_ok) {
      const float l = l_run;
      const float m = (m_run == -INFINITY) ? 0.f : m_run;
      const float lse_v = l > 0.f ? (m + __log2f(l)) * 0.6931471805599453f : -INFINITY;
      if (split) ws[(int64_t)slot * kSlotFloats + (int64_t)kRowsPerTile * kLat + my_row] = lse_v;
      else lse_ptr[(int64_t)(seq * a.s_q + j_tok) * a.heads + head] = lse_v;
    }
    barrier_lds();
  }
}

// Merge the partials of split items: lse = log sum_k e^{lse_k}, out = sum_k e^{lse_k - lse} O_k.
__global__ __launch_bounds__(256) void combine_kernel(const int32_t* __restrict__ plan,
                                                      const float* __restrict__ ws, float* __restrict__ out,
                                                      float* __restrict__ lse, int s_q, int heads) {
  if (plan[kHMagic] != kPlanMagic) return;
  const int n_split = plan[kHSplitItems];
  const int n_items = plan[kHItems];
  if ((int)blockIdx.x >= n_split) return;
  const int k = plan[plan_split_off(n_items, plan[kHWorkers]) + blockIdx.x];
  const int32_t* it = plan + plan_items_off() + kItemWords * k;
  const int seq = it[kISeq], tile = it[kITile], ns = it[kINsplits], slot0 = it[kISlot];
  const int rows_total = s_q * heads;
  const int sub = threadIdx.x >> 7;        // two rows per pass
  const int c4 = (threadIdx.x & 127) * 4;  // channel quad
  const int rows_per_block = kRowsPerTile / gridDim.y;
  for (int r = blockIdx.y * rows_per_block + sub; r < (int)(blockIdx.y + 1) * rows_per_block; r += 2) {
    const int grow = kRowsPerTile * tile + r;
    if (grow >= rows_total) continue;
    float m = -INFINITY;
    for (int s = 0; s < ns; ++s) {
      const float l = ws[(int64_t)(slot0 + s) * kSlotFloats + (int64_t)kRowsPerTile * kLat + r];
      m = fmaxf(m, l);
    }
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float tot = 0.f;
    if (m != -INFINITY) {
      for (int s = 0; s < ns; ++s) {
        const float* base = ws + (int64_t)(slot0 + s) * kSlotFloats;
        const float l = base[(int64_t)kRowsPerTile * kLat + r];
        const float wgt = (l == -INFINITY) ? 0.f : __expf(l - m);
        tot += wgt;
        if (wgt != 0.f) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(base + (int64_t)r * kLat + c4);
          acc += wgt * v;
        }
      }
    }
    const int jt = grow / heads, hd = grow - jt * heads;
    const int64_t orow = (int64_t)(seq * s_q + jt) * heads + hd;
    const float inv = tot > 0.f ? 1.f / tot : 0.f;
    *reinterpret_cast<f32x4*>(out + orow * kLat + c4) = acc * inv;
    if (c4 == 0) lse[orow] = tot > 0.f ? m + __logf(tot) : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeArgs& a, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)decode_kernel<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                                     kLdsBytes);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_kernel<false>, dim3(a.workers), dim3(kThreads), kLdsBytes, stream,
                     reinterpret_cast<const __bf16*>(a.q), reinterpret_cast<const char*>(a.kv), a.kv_scales,
                     a.block_table, a.seqlens, a.plan, a.ws, a.out, a.lse, scalars_of(a));
  return hipGetLastError();
}

hipError_t launch_decode_fp8(const DecodeArgs& a, hipStream_t stream) {
  (void)a; (void)stream;
  return hipErrorNotSupported;
}

hipError_t launch_combine(const DecodeArgs& a, hipStream_t stream) {
  const int max_split = a.workers;   // split items <= active workers - 1
  hipLaunchKernelGGL(combine_kernel, dim3(max_split, 8), dim3(256), 0, stream, a.plan, a.ws, a.out, a.lse, a.s_q,
                     a.heads);
  return hipGetLastError();
}

}  // namespace mla
