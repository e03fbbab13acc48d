// Device-side pieces shared by the decode kernels: vector types, kernel scalars, the
// split-plan walk (segments and the load cursor), buffer descriptors of a cached half
// page, LDS-DMA issue, LDS-only barriers and waits, LDS operand reads.
#pragma once
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
typedef __attribute__((ext_vector_type(2))) unsigned u32x2;
#define LDSP(T) __attribute__((address_space(3))) T*

constexpr int kStep = 32;                      // tokens per pipeline step
constexpr int kRowBytes = kDqk * 2;            // 1152
constexpr int kBufBytes = kStep * kRowBytes;   // 36864
constexpr int kDmaInstr = kBufBytes / 1024;    // 36 LDS-DMA instructions (1 KiB each) per step
// fp8 cache (OCP e4m3fn): a cached row is 512 codes + 64 bf16 rope channels (640 B), with
// one f32 scale per 128-channel tile of the 512 latent channels in a separate array.
constexpr int kF8Row = kLat + 2 * kRope;       // 640

constexpr uint32_t kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit format, gfx9 family

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
// itself with wait_vmcnt + barrier_lds. The LDS address is an operand bound to m0, so the
// compiler sets m0 itself and knows it is in use; the instruction has no register outputs
// (nothing is left in flight in a VGPR).
__device__ __forceinline__ void lds_dma_x4(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)));
}

// The same for data read once per call (cache rows): with the non-temporal hint the 302 MB
// a dsv3 call streams do not displace what the work-groups share through L2 (query rows,
// the plan). Measured on the dsv3 decode: 97.6 -> 93.9 us per call; the same hint on the
// shared query staging, on the split partials or in the combine kernel gained nothing.
__device__ __forceinline__ void lds_dma_x4_stream(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen nt lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)));
}

// The same with 64 lanes x 4 B (LDS at m0 + 4 * lane).
__device__ __forceinline__ void lds_dma_x1(uint32_t lds_addr, uint32_t voff, i32x4 rsrc) {
  asm volatile("buffer_load_dword %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr)));
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

// Load cursor: walks the worker's steps in order, ahead of the compute loop. The fields of
// the current item are cached and the page id of the cursor's step is fetched when the
// cursor moves, one compute region before its descriptor is needed, so the scalar load's
// latency is covered by the barriers in between.
struct LoadCursor {
  int k, hh, hh1;   // current item, next step to load, end step of that item
  int seq, vis;     // fields of item k
  int pid;          // page id of step hh (-1: none)
};

__device__ __forceinline__ void cursor_fetch(LoadCursor& c, const Scalars& a, const int32_t* __restrict__ block_table) {
  const int pg = c.hh >> 1;
  c.pid = pg < a.max_pages ? block_table[(int64_t)c.seq * a.max_pages + pg] : -1;
}

__device__ __forceinline__ void cursor_enter(LoadCursor& c, const int32_t* __restrict__ plan, int k, int kb, int pb,
                                             int ke, int pe) {
  const int32_t* it = plan + plan_items_off() + kItemWords * k;
  const Seg sg = seg_of(plan, k, kb, pb, ke, pe);
  c.k = k;
  c.seq = it[kISeq];
  c.vis = it[kIVis];
  c.hh = sg.hh0;
  c.hh1 = sg.hh1;
}

// Buffer descriptors of the cursor's step (32 tokens = half of a 64-token page): base at
// the step's first row, record count at the last visible token, so rows past it read as
// zeros. A page id outside [0, num_pages) gives 0 records (all zeros). For an fp8 cache the
// second descriptor covers the step's scales. (Uniform by construction; readfirstlane tells
// the compiler so, keeping them in SGPRs.)
struct StepRsrc {
  i32x4 kv, sc;
};

__device__ __forceinline__ i32x4 make_rsrc(uint64_t addr, int bytes) {
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((int)(uint32_t)addr);
  r[1] = __builtin_amdgcn_readfirstlane((int)((uint32_t)(addr >> 32) & 0xFFFF));   // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(bytes);                                    // num_records
  r[3] = (int)kRsrcWord3;
  return r;
}

template <bool kFp8>
__device__ __forceinline__ StepRsrc cursor_rsrc(const LoadCursor& c, const Scalars& a, const char* __restrict__ kv,
                                                const float* __restrict__ scales, int& dev_err) {
  int valid = c.vis - kStep * c.hh;
  valid = valid > kStep ? kStep : valid;
  const bool in_range = c.pid >= 0 && (int64_t)c.pid < a.num_pages;
  const bool ok = in_range && valid > 0;
  // a page the step needs whose block-table entry lies outside the cache (entries past
  // max_pages are a length above capacity, reported on its own)
  if (valid > 0 && !in_range && (c.hh >> 1) < a.max_pages) dev_err |= kDevPageOutOfRange;
  StepRsrc r;
  if constexpr (!kFp8) {
    const uint64_t addr = reinterpret_cast<uint64_t>(kv) +
                          (ok ? ((uint64_t)c.pid * (kPage * kRowBytes) + (uint64_t)(c.hh & 1) * kBufBytes) : 0);
    r.kv = make_rsrc(addr, ok ? valid * kRowBytes : 0);
    r.sc = r.kv;
  } else {
    const uint64_t tok0 = ok ? (uint64_t)c.pid * kPage + (uint64_t)(c.hh & 1) * kStep : 0;
    r.kv = make_rsrc(reinterpret_cast<uint64_t>(kv) + tok0 * kF8Row, ok ? valid * kF8Row : 0);
    r.sc = make_rsrc(reinterpret_cast<uint64_t>(scales) + tok0 * 16, ok ? valid * 16 : 0);
  }
  return r;
}

__device__ __forceinline__ bf16x8 lds_b128(const char __attribute__((address_space(3)))* p) {
  u32x4 v = *(const u32x4 __attribute__((address_space(3)))*)p;
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x4 lds_tr16(const char __attribute__((address_space(3)))* p) {
  i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDSP(i16x4))(p));
  return __builtin_bit_cast(bf16x4, v);
}


// Work-groups are dealt to the 8 XCDs round-robin (consecutive blocks on consecutive XCDs;
// which XCD block 0 lands on varies between launches). Plan workers are numbered so that
// consecutive ones (the parts of one split item, which all load the item's queries) are
// blocks of one residue class and so share an XCD and its L2: worker = (blocks of lower
// residues) + b / 8. This only places work; nothing relies on it for correctness.
constexpr int kXcds = 8;
__device__ __forceinline__ int xcd_worker() {
  const int b = blockIdx.x, n = gridDim.x, x = b % kXcds;
  int before = 0;
  for (int y = 0; y < x; ++y) before += (n - y + kXcds - 1) / kXcds;
  return before + b / kXcds;
}

typedef __attribute__((ext_vector_type(16))) int i32x16;

// The plan header (16 words) in one scalar load: written as a chain of ||, the header check
// compiles to one scalar load, compare and branch per word.
__device__ __forceinline__ i32x16 load_plan_header(const int32_t* __restrict__ plan) {
  return *reinterpret_cast<const i32x16*>(plan);
}
// The header's identity words against the call's arguments.
__device__ __forceinline__ bool plan_header_matches(const i32x16& h, int batch, int s_q, int heads, int causal,
                                                    int workers, int n_items) {
  const int d = (h[kHMagic] ^ kPlanMagic) | (h[kHVersion] ^ kPlanVersion) | (h[kHBatch] ^ batch) |
                (h[kHSq] ^ s_q) | (h[kHHeads] ^ heads) | (h[kHCausal] ^ causal) | (h[kHWorkers] ^ workers) |
                (h[kHItems] ^ n_items);
  return d == 0;
}

}  // namespace
}  // namespace mla
