/*
 * rfp4_bench.h -- C ABI of librfp4_bench.so, a measurement aid beside librfp4.so (not
 * part of the ROCmFP4 method): a plain streaming read of device memory, the ceiling
 * that the memory-bound decode GEMV is measured against ("Feasibility Report: Porting
 * ROCmFP4 to Atlas", "Why AMD is Different from NVIDIA": on AMD the bottleneck is
 * memory bandwidth), and a dense bf16 matrix-core loop, the sustained rate that the
 * prefill GEMM (the page's "Kernel System" w4a16 GEMM) is measured against.
 */
#ifndef RFP4_BENCH_H
#define RFP4_BENCH_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes at device pointer `p` (16-byte aligned, bytes a multiple of 16)
 * once, with 16-byte loads, `unroll` loads in flight per lane (1, 2, 4 or 8) and a grid
 * of `wgs_per_cu` 256-thread workgroups per CU (1..32), each workgroup reading
 * consecutive 4 KiB runs; the XOR of everything read is folded into a value that is
 * written to `sink` (a device uint32) only if it equals a value the data never
 * produces, so the loads cannot be dropped and nothing else is written. Asynchronous on
 * `stream` (a hipStream_t, NULL = the null stream). Returns 0, or -1 for a bad argument
 * (checked before any HIP call), or the HIP error code of the launch. */
__attribute__((visibility("default"))) int rfp4bench_read(const void* p, size_t bytes, int unroll,
                                                          int wgs_per_cu, uint32_t* sink, void* stream);

/* Issues, on each of `wgs_per_cu` (1..8) workgroups per CU of `threads` (64, 128, 256 or
 * 512) threads, `iters` (>= 1) rounds of 8 v_mfma_f32_32x32x16_bf16 per wavefront into 8
 * independent accumulators, with operands that differ between consecutive instructions;
 * nothing is read from memory, and `sink` (a device uint32) is written only if the sums
 * take a value they never take. One launch performs CUs x wgs_per_cu x threads / 64 x
 * iters x 8 x 32768 flops. Asynchronous on `stream`. Returns 0, -1 for a bad argument
 * (checked before any HIP call), or the HIP error code of the launch. */
__attribute__((visibility("default"))) int rfp4bench_mfma(int wgs_per_cu, int threads, int iters, uint32_t* sink,
                                                          void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RFP4_BENCH_H */
