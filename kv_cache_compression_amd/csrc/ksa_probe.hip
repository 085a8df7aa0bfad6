// Machine-peak probes for the benchmark's rooflines (libksa_probe.so):
//   - a bf16 MFMA issue loop (v_mfma_f32_32x32x16_bf16, register operands,
//     four independent accumulation chains per wave, two waves per SIMD), the
//     sustained matrix rate of the chip under the same launch shape as the
//     prefill kernels.  The operands either derive from the lane index (the
//     same values every iteration) or cycle through eight operand pairs
//     loaded from a buffer of the caller's data: the matrix cores draw more
//     power, and the clock drops, when the operand bits toggle as they do on
//     real tensors;
//   - a streaming HBM read (16-byte non-temporal loads, eight in flight per
//     thread), the access pattern of the split-K decode;
//   - a streaming HBM copy (16-byte loads and stores).
// None of these is part of the attention path; they only measure the GPU.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/ksa_probe.h"

namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kChains = 4;
constexpr int kUnroll = 8;

constexpr int kPairs = 8;  // operand pairs cycled through when loaded from data

__global__ void __launch_bounds__(kThreads, 2) probe_mfma_kernel(int32_t iters, const bf16x8_t* __restrict__ opnd,
                                                                float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  bf16x8_t a[kPairs], b[kPairs];
  if (opnd != nullptr) {
    // 2 kPairs operands of 16 bytes per lane, distinct per wave
    const bf16x8_t* p = opnd + (static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x) * (2 * kPairs);
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      a[i] = p[2 * i];
      b[i] = p[2 * i + 1];
    }
  } else {
#pragma unroll
    for (int i = 0; i < kPairs; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        a[i][j] = static_cast<__bf16>(0.001f * static_cast<float>(lane + j));
        b[i][j] = static_cast<__bf16>(0.001f * static_cast<float>(j - lane));
      }
  }
  f32x16_t acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[c][r] = 0.f;
  for (int it = 0; it < iters; it += 2) {
#pragma unroll
    for (int u = 0; u < 2 * kChains; ++u) {
      const int c = u % kChains;
      const int pr = u % kPairs;
      acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[pr], b[pr], acc[c], 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[c][r];
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = s;
}

__global__ void __launch_bounds__(kThreads) probe_read_kernel(const u32x4_t* __restrict__ src, size_t n16,
                                                             uint32_t* __restrict__ sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  uint32_t x = 0;
  for (; i + (kUnroll - 1) * stride < n16; i += kUnroll * stride) {
    u32x4_t v[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) x ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  for (; i < n16; i += stride) {
    const u32x4_t v = __builtin_nontemporal_load(src + i);
    x ^= v.x ^ v.y ^ v.z ^ v.w;
  }
  sink[static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x] = x;
}

__global__ void __launch_bounds__(kThreads) probe_copy_kernel(const u32x4_t* __restrict__ src,
                                                             u32x4_t* __restrict__ dst, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * kThreads;
  size_t i = static_cast<size_t>(blockIdx.x) * kThreads + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    u32x4_t v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < 4; ++u) __builtin_nontemporal_store(v[u], dst + i + u * stride);
  }
  for (; i < n16; i += stride) __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

int32_t status_of(hipError_t e) { return e == hipSuccess ? 0 : static_cast<int32_t>(e); }

}  // namespace

extern "C" {

__attribute__((visibility("default"))) double ksa_probe_mfma_bf16_flops(int32_t blocks, int32_t iters) {
  // 4 waves per block, kChains MFMAs of 2 * 32 * 32 * 16 FLOP per iteration
  return static_cast<double>(blocks) * (kThreads / 64) * iters * kChains * 2.0 * 32 * 32 * 16;
}

__attribute__((visibility("default"))) size_t ksa_probe_mfma_bf16_operand_bytes(int32_t blocks) {
  return blocks <= 0 ? 0 : static_cast<size_t>(blocks) * kThreads * 2 * kPairs * sizeof(bf16x8_t);
}

__attribute__((visibility("default"))) int32_t ksa_probe_mfma_bf16(int32_t blocks, int32_t iters,
                                                                   const void* operands, float* sink,
                                                                   hipStream_t stream) {
  if (blocks <= 0 || iters <= 0 || iters % 2 != 0 || sink == nullptr ||
      reinterpret_cast<uintptr_t>(operands) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream, iters,
                     static_cast<const bf16x8_t*>(operands), sink);
  return status_of(hipGetLastError());
}

__attribute__((visibility("default"))) int32_t ksa_probe_hbm_read(const void* src, size_t bytes, int32_t blocks,
                                                                  uint32_t* sink, hipStream_t stream) {
  if (src == nullptr || sink == nullptr || blocks <= 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(probe_read_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), bytes / 16, sink);
  return status_of(hipGetLastError());
}

__attribute__((visibility("default"))) int32_t ksa_probe_hbm_copy(const void* src, void* dst, size_t bytes,
                                                                  int32_t blocks, hipStream_t stream) {
  if (src == nullptr || dst == nullptr || blocks <= 0 || bytes % 16 != 0 ||
      reinterpret_cast<uintptr_t>(src) % 16 != 0 || reinterpret_cast<uintptr_t>(dst) % 16 != 0)
    return -1;
  hipLaunchKernelGGL(probe_copy_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kThreads), 0, stream,
                     static_cast<const u32x4_t*>(src), static_cast<u32x4_t*>(dst), bytes / 16);
  return status_of(hipGetLastError());
}

}  // extern "C"
