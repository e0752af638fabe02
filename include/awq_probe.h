/*
 * awq_probe.h - measurement kernels that give the W4A16 benchmark its measured ceilings
 * (libawq_probe_gfx950.so; not part of the product path).
 *
 * Decode time is the bytes a layer moves divided by the bandwidth reached
 * (edgesiliconlab ?p=2015, section "The Mathematics of Memory Bandwidth Saturation").
 * Beside the specification peak the benchmark reports what a read-only kernel with the
 * decode kernel's access pattern reaches on the same number of bytes, the cost of one
 * empty launch, and how many ALU instructions issue beside a matrix instruction. Return codes: 0 ok, 1 invalid argument, 3 misaligned, 5 launch
 * rejected by the HIP runtime.
 */
#ifndef AWQ_PROBE_H_
#define AWQ_PROBE_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Number of launch shapes awq_probe_stream_read accepts (0 .. n - 1). */
int awq_probe_shapes(void);

/*
 * Read `bytes` bytes of `buf` (device, 16-byte aligned, 0 < bytes < 2^31) once, with
 * 16-byte non-temporal loads per lane, 1 KiB per wavefront load, all of a wavefront's
 * loads in flight at once. Launch shape: 0 = 512 threads and 32 KiB per workgroup,
 * 1 = 256 threads and 16 KiB, 2 = 1024 threads and 64 KiB, 3 = 256 threads and 64 KiB.
 * sink: device, one uint32, written only if the data XOR to a fixed constant (keeps
 * the loads alive). Asynchronous on `stream`.
 */
int awq_probe_stream_read(const void* buf, size_t bytes, int shape, uint32_t* sink,
                          hipStream_t stream);

/* One empty kernel (one workgroup of 64 threads) on `stream`. */
int awq_probe_empty(hipStream_t stream);

/*
 * Matrix-core / ALU co-issue (the prefill kernel dequantizes weights with ALU
 * instructions while the matrix cores multiply: edgesiliconlab ?p=2015, section "Kernel
 * Execution: Marlin vs. ExLlamaV2 INT4 GEMM Micro-Architecture", item 3). `blocks`
 * workgroups of 256 threads (1 .. 4096; 256 = one wavefront per SIMD on every CU, 512 =
 * two) each run `iters` iterations of 8 independent 16 x 16 x 32 binary16 matrix
 * instructions, each followed by `alu` (0 .. 4) packed binary16 multiplies. out: device,
 * blocks * 256 floats, overwritten. Asynchronous on `stream`.
 */
int awq_probe_mfma_alu(float* out, int alu, int blocks, int iters, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_PROBE_H_ */
