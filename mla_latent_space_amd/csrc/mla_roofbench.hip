// Measured roofline denominators (page "Mla Analysis", section "Cost Models": a decode call is
// bound by the larger of its bytes over the memory bandwidth and its FLOPs over the matrix
// peak). Two kernels, each doing nothing but the one thing it measures:
//  - stream_read_kernel: each work-group reads its own contiguous share of the buffer, 64 KiB
//    per round (every lane eight non-temporal 16-B loads in flight, a wave 1 KiB per load),
//    XOR-folding what it reads so that no load is dead. (Measured on MI355X over 2 GiB: 6.7 TB/s
//    this way against 5.9 TB/s for a grid-wide stride, the same loads otherwise.)
//  - mfma_loop_kernel: every wave issues rounds of four independent v_mfma_f32_32x32x16_bf16
//    (four accumulators, so one MFMA never waits for the previous one's result), with the
//    shader-clock and 100-MHz counters read at the start and end of the first wave.
// This library is separate from libmla; nothing in the decode path calls it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "mla_roofbench.h"

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(16))) float f32x16;

constexpr int kRbThreads = 512;   // stream read: threads per work-group
constexpr int kRbUnroll = 8;      // loads in flight per lane
constexpr int kMfLds = 96 * 1024; // MFMA loop: LDS per work-group, so that each CU holds one

__global__ __launch_bounds__(kRbThreads) void stream_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                                 u32x4* __restrict__ sink) {
  // work-group b: words [b per, (b + 1) per); round r: lane t reads words base + u T + t, u < 8
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t w0 = (int64_t)blockIdx.x * per;
  const int64_t w1 = w0 + per < n16 ? w0 + per : n16;
  u32x4 acc = {0u, 0u, 0u, 0u};
  int64_t i = w0 + threadIdx.x;
  for (; i + (kRbUnroll - 1) * kRbThreads < w1; i += kRbUnroll * kRbThreads) {
    u32x4 v[kRbUnroll];
#pragma unroll
    for (int u = 0; u < kRbUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * kRbThreads);
#pragma unroll
    for (int u = 0; u < kRbUnroll; ++u) acc ^= v[u];
  }
  for (; i < w1; i += kRbThreads) acc ^= __builtin_nontemporal_load(src + i);
  sink[(int64_t)blockIdx.x * kRbThreads + threadIdx.x] = acc;
}

__global__ __launch_bounds__(512) void mfma_loop_kernel(int iters, float* __restrict__ sink,
                                                        uint64_t* __restrict__ clocks) {
  uint64_t t0 = 0, r0 = 0;
  if (threadIdx.x < 64) {
    t0 = __builtin_amdgcn_s_memtime();
    r0 = __builtin_amdgcn_s_memrealtime();
  }
  bf16x8 one;
#pragma unroll
  for (int e = 0; e < 8; ++e) one[e] = (__bf16)1.0f;
  f32x16 acc[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) acc[k] = f32x16{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 4; ++k) acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(one, one, acc[k], 0, 0, 0);
  }
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
    sink[4 * g + k] = s;
  }
  if (threadIdx.x == 0) {
    const uint64_t t1 = __builtin_amdgcn_s_memtime(), r1 = __builtin_amdgcn_s_memrealtime();
    uint64_t* c = clocks + 4 * blockIdx.x;
    c[0] = t0;
    c[1] = t1;
    c[2] = r0;
    c[3] = r1;
  }
}

}  // namespace

extern "C" int32_t mla_rb_stream_read(const void* src, int64_t bytes, void* sink, int32_t blocks, void* stream) {
  if (src == nullptr || sink == nullptr || bytes <= 0 || bytes % 16 != 0 || blocks < 1 || blocks > 65536 ||
      (reinterpret_cast<uintptr_t>(src) & 15) != 0 || (reinterpret_cast<uintptr_t>(sink) & 15) != 0)
    return 1;
  hipLaunchKernelGGL(stream_read_kernel, dim3(blocks), dim3(kRbThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), bytes / 16, static_cast<u32x4*>(sink));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

extern "C" int32_t mla_rb_mfma_bf16_loop(int32_t blocks, int32_t waves_per_simd, int32_t iters, float* sink,
                                         uint64_t* clocks, void* stream) {
  if (sink == nullptr || clocks == nullptr || blocks < 1 || blocks > 4096 || (waves_per_simd != 1 && waves_per_simd != 2) ||
      iters < 1 || iters > (1 << 20))
    return 1;
  static thread_local int configured = -1;   // the LDS opt-in is per device
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 4;
  if (configured != dev) {
    if (hipFuncSetAttribute((const void*)mfma_loop_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, kMfLds) !=
        hipSuccess)
      return 4;
    configured = dev;
  }
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(256 * waves_per_simd), kMfLds,
                     static_cast<hipStream_t>(stream), iters, sink, clocks);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}
