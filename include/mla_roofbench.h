/*
 * mla_roofbench -- measured roofline denominators for the decode kernels of libmla on the
 * device they run on (AMD Instinct MI355X, gfx950). C ABI, a library of its own
 * (libmla_roofbench.so): nothing in libmla calls it.
 *
 * Page "Mla Analysis", section "Cost Models": the bound of a decode call is the larger of its
 * bytes over the memory bandwidth and its FLOPs over the matrix peak. The published MI355X
 * figures (8 TB/s of HBM, 2.5 PFLOP/s of dense bf16 MFMA at the 2.4 GHz peak clock) are the
 * headline denominators. These two calls measure what the device delivers instead:
 *  - mla_rb_stream_read: how fast a plain read stream moves a buffer from memory into
 *    registers (the reachable memory bandwidth);
 *  - mla_rb_mfma_bf16_loop: how fast chains of v_mfma_f32_32x32x16_bf16 run with nothing
 *    else to do, and at which shader clock (the reachable matrix peak).
 *
 * Conventions: every pointer is caller-owned device memory unless the argument says host; the
 * calls allocate nothing and enqueue their work on `stream` (a hipStream_t; NULL = the default
 * stream). A call that returns 0 has enqueued its kernel; time it with events on the same
 * stream. Every host-checkable error is returned before anything is enqueued: 1 for an invalid
 * argument, 4 for a failed launch (the codes of libmla's status enum).
 */
#ifndef MLA_ROOFBENCH_H
#define MLA_ROOFBENCH_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads src[0 .. bytes) once, 16 B per lane and load, with the non-temporal hint, eight loads
 * in flight per lane. blocks work-groups of 512 threads each read a contiguous share of the
 * buffer (ceil(bytes / 16 / blocks) words, the last one less), 64 KiB per round, consecutive
 * lanes on consecutive 16-B words (a wave reads 1 KiB per load). Thread g of the grid writes
 * to sink[g] (16 B) the XOR of the words it read, so that the loads cannot be dropped: the
 * XOR of all sink words is the XOR of all 16-B words of src.
 *   src    device, 16-B aligned, `bytes` readable; bytes > 0 and a multiple of 16.
 *   sink   device, 16 * 512 * blocks bytes, overwritten.
 *   blocks 1 .. 65536.
 * The memory traffic of one call is `bytes` read plus the sink write. */
int32_t mla_rb_stream_read(const void* src, int64_t bytes, void* sink, int32_t blocks, void* stream);

/* blocks work-groups of 256 * waves_per_simd threads, each holding 96 KiB of LDS so that no
 * two share a compute unit: with 256 blocks every CU runs 4 * waves_per_simd waves. Each wave
 * issues iters rounds of four independent v_mfma_f32_32x32x16_bf16 (four accumulators; all
 * operands 1.0, so each element of an accumulator ends at 16 * iters). That is
 * blocks * 4 * waves_per_simd * iters * 4 * 32768 FLOPs per call.
 *   sink   device, 4 * 256 * waves_per_simd * blocks floats: word 4g + a is the sum of the 16
 *          elements that thread g holds of accumulator a (256 * iters, exact in fp32 for
 *          iters <= 2^16).
 *   clocks device, 4 * blocks uint64: per block, the shader-clock counter (s_memtime) and the
 *          100-MHz reference counter (s_memrealtime) at its first wave's start and end, in
 *          the order (shader start, shader end, ref start, ref end). The shader clock over the
 *          block's run is (shader end - start) / (ref end - start) * 100 MHz.
 *   blocks 1 .. 4096; waves_per_simd 1 or 2; iters 1 .. 2^20. */
int32_t mla_rb_mfma_bf16_loop(int32_t blocks, int32_t waves_per_simd, int32_t iters, float* sink, uint64_t* clocks,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MLA_ROOFBENCH_H */
