/* Machine-peak probes (libksa_probe.so): the measured ceilings that the
 * benchmark reports its rooflines against, beside the published MI355X peaks.
 * Measurement only; nothing here is part of the attention path, and the
 * attention library (libksa.so) neither contains nor calls these.
 *
 * All pointers are device pointers, owned by the caller; every call is
 * asynchronous on `stream`.  Return value: 0 = launched, -1 = invalid
 * argument (nothing launched), otherwise the hipError_t of the launch.
 */
#ifndef KSA_PROBE_H_
#define KSA_PROBE_H_

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 matrix-core issue loop: `blocks` workgroups of 256 threads (two per
 * SIMD at most), each wave issuing `iters` (even) x 4 independent
 * v_mfma_f32_32x32x16_bf16 on register operands.  operands: NULL (values
 * derived from the lane index, identical every iteration) or a 16-byte
 * aligned device buffer of ksa_probe_mfma_bf16_operand_bytes(blocks) bytes
 * of bf16 data, from which every lane takes 8 operand pairs and cycles
 * through them.  sink: [blocks * 256] fp32, written once per thread (keeps
 * the loop live).  The FLOP count of one launch is
 * ksa_probe_mfma_bf16_flops(blocks, iters). */
int32_t ksa_probe_mfma_bf16(int32_t blocks, int32_t iters, const void* operands, float* sink,
                            hipStream_t stream);
double ksa_probe_mfma_bf16_flops(int32_t blocks, int32_t iters);
size_t ksa_probe_mfma_bf16_operand_bytes(int32_t blocks);

/* Streaming read of `bytes` (a multiple of 16, 16-byte aligned) from src
 * with 16-byte non-temporal loads, grid-stride over `blocks` workgroups of
 * 256 threads.  sink: [blocks * 256] uint32, one XOR fold per thread. */
int32_t ksa_probe_hbm_read(const void* src, size_t bytes, int32_t blocks, uint32_t* sink, hipStream_t stream);

/* Streaming copy of `bytes` (a multiple of 16; src and dst 16-byte aligned,
 * not overlapping) with 16-byte loads and stores. */
int32_t ksa_probe_hbm_copy(const void* src, void* dst, size_t bytes, int32_t blocks, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KSA_PROBE_H_ */
