// Device-side helpers shared by the KSA kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ksa.h"

namespace ksa {

typedef uint16_t bf16_t;  // raw bfloat16 storage
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float bf16_to_f32(bf16_t x) {
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}

// Round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(bf16_t, b);
}

// Pack two floats into one dword of two bf16 (lo = a, hi = b), RNE.
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  return static_cast<uint32_t>(f32_to_bf16(a)) | (static_cast<uint32_t>(f32_to_bf16(b)) << 16);
}

template <typename T>
__device__ __forceinline__ float load_f32(const T* p);
template <>
__device__ __forceinline__ float load_f32<float>(const float* p) {
  return *p;
}
template <>
__device__ __forceinline__ float load_f32<bf16_t>(const bf16_t* p) {
  return bf16_to_f32(*p);
}

template <typename T>
__device__ __forceinline__ void store_f32(T* p, float v);
template <>
__device__ __forceinline__ void store_f32<float>(float* p, float v) {
  *p = v;
}
template <>
__device__ __forceinline__ void store_f32<bf16_t>(bf16_t* p, float v) {
  *p = f32_to_bf16(v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// x combined with the value of the lane 32 away, on the vector ALU:
// v_permlane32_swap trades lanes 32..63 of one copy of x with lanes 0..31 of
// another, so every lane holds both halves' values and computes
// op(x[low lane], x[high lane]) in the same order.
__device__ __forceinline__ float with_upper_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float with_upper_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
// The same for the lane 16 away within each half wave: v_permlane16_swap
// trades the odd 16-lane rows of one copy with the even rows of another.
__device__ __forceinline__ float with_row_pair_max(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float with_row_pair_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Augmented row of text token t (Eq. 1): every complete chunk before it adds
// one summary row.
__device__ __forceinline__ int64_t text_row(int64_t t, int32_t k) { return t + t / k; }
// Augmented row of summary s_j: last row of chunk j.
__device__ __forceinline__ int64_t summary_row(int64_t j, int32_t k) {
  return j * (k + 1) + k;
}

// Position id of augmented row a for n text tokens and chunk size k
// (Sec. 2.2.1: text keeps its text index, a summary takes the id of its
// chunk's last text token).
__device__ __forceinline__ int64_t augmented_position(int64_t a, int64_t n, int32_t k) {
  const int64_t M = n / k;
  if (a < M * (k + 1)) {
    const int64_t c = a / (k + 1);
    const int64_t o = a - c * (k + 1);
    return c * k + (o < k ? o : k - 1);  // summary: the chunk's last text position
  }
  return M * k + (a - M * (k + 1));  // trailing partial chunk
}

}  // namespace ksa
