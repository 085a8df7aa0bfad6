// Helpers of the bf16 MFMA kernels with 128-wide heads (gfx950, wave64):
// swizzled LDS row layout, transposing LDS reads, bf16 packing, and the
// fast floor(t / k) used to map text indices to Eq. 1 rows.
#pragma once

#include "ksa_common.h"

namespace ksa {
namespace mfma {

constexpr int D = 128;
constexpr int ROW_BYTES = D * 2;  // 256 B per (row, head)

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

// 16-byte chunk c (0..15) of LDS row `row` is stored at chunk c ^ swz(row),
// swz(row) = 4 (row % 4) + (row / 4) % 4, a bijection on 16 consecutive rows:
//   - MFMA operand reads (16 lanes = 16 rows, one logical chunk) land on 16
//     different chunk positions, i.e. all 64 banks once;
//   - transposing reads (per 32 lanes: 4 rows x 4 consecutive chunks
//     4q .. 4q+3) flip the chunk's two upper bits by row % 4, so the 16
//     (row, chunk) pairs also take 16 different positions.
// The DMA writes stay linear (lane l writes bytes 16 l ..): the global side
// fetches the chunk that belongs there.
__device__ __forceinline__ int lds_swz(int row) { return ((row & 3) << 2) | ((row >> 2) & 3); }
__device__ __forceinline__ int lds_off(int row, int chunk) {
  return row * ROW_BYTES + ((chunk ^ lds_swz(row)) << 4);
}

// ds_read_b64_tr_b16: in each group of 16 lanes, lane 4 rr + c4 names row
// rr and columns 4 c4 .. 4 c4 + 3 of a 4 x 16 bf16 block; lane i receives
// column i (4 values, rows 0..3).
__device__ __forceinline__ bf16x4_t lds_read_tr(const char* base, int byte_off) {
  auto p = (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)(base) + byte_off);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Takes the word by value: __builtin_bit_cast applied directly to a vector
// element (v.y) reads element 0 with this compiler.
__device__ __forceinline__ bf16x2_t as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2_t, w); }

// Cross-lane reductions on the vector ALU (no LDS round trip):
//   - sum16: the sum over each group of 16 lanes, in every lane of the
//     group, by DPP: quad swaps (xor 1, xor 2), then the mirrored half-row
//     (quad q gets quad 1 - q) and the mirrored row (half h gets half 1 - h);
//   - with_upper_half_max / with_upper_half_sum (ksa_common.h) for the lane
//     32 away.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_mov<0xB1>(x);   // quad_perm [1, 0, 3, 2]
  x += dpp_mov<0x4E>(x);   // quad_perm [2, 3, 0, 1]
  x += dpp_mov<0x141>(x);  // row_half_mirror
  x += dpp_mov<0x140>(x);  // row_mirror
  return x;
}

// floor(t / d) = (umulhi(t, m) + t) >> l for 0 <= t < 2^31.
inline void fast_div(uint32_t d, uint32_t* m, uint32_t* l) {
  uint32_t s = 0;
  while ((uint64_t(1) << s) < d) ++s;
  *l = s;
  *m = static_cast<uint32_t>(((uint64_t(1) << 32) * ((uint64_t(1) << s) - d)) / d + 1);
}
__device__ __forceinline__ int32_t fast_div_apply(int32_t t, uint32_t m, uint32_t l) {
  return static_cast<int32_t>((__umulhi(static_cast<uint32_t>(t), m) + static_cast<uint32_t>(t)) >> l);
}

}  // namespace mfma
}  // namespace ksa
