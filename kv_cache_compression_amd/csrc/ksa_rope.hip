// Half-split rotary embedding with the KSA position rule.
//
// "Kwai Summary Attention Technical Report", Sec. 2.2.1: text tokens keep
// their text index as position id (summaries consume none) and a summary
// token takes the id of its chunk's last text token.  RoPE is applied to Q
// and K before attention and before keys enter the cache (Sec. 2.3.1).
//
// One thread owns one rotation pair (f, f + rot_dim/2) of one row and walks
// every head of that row, so the fp64 angle and its sine/cosine are formed
// once per (row, f).
#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

template <typename T>
__global__ void __launch_bounds__(256) rope_kernel(RopeArgs a, T* __restrict__ x) {
  const int32_t half = a.rot_dim / 2;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.batch) * a.rows * half;
  if (tid >= total) return;
  const int32_t f = static_cast<int32_t>(tid % half);
  const int64_t br = tid / half;  // batch * rows + row
  const int64_t row = br % a.rows;
  const int64_t pos = a.positions ? a.positions[br] : augmented_position(row, a.n_text, a.chunk);
  const double inv_freq = pow(a.theta, -2.0 * static_cast<double>(f) / a.rot_dim);
  const double ang = static_cast<double>(pos) * inv_freq;
  double sn, cs;
  sincos(ang, &sn, &cs);
  T* base = x + br * a.heads * static_cast<int64_t>(a.head_dim) + a.rot_off + f;
  for (int32_t h = 0; h < a.heads; ++h) {
    T* p = base + static_cast<int64_t>(h) * a.head_dim;
    const double lo = load_f32(p);
    const double hi = load_f32(p + half);
    store_f32(p, static_cast<float>(lo * cs - hi * sn));
    store_f32(p + half, static_cast<float>(hi * cs + lo * sn));
  }
}

// bf16 with 8 | rot_dim / 2 and 8 | rot_off: one thread owns 8 consecutive
// pairs of one row (16-byte loads of each half) and walks every head; the
// rotation itself runs in fp32 (bf16 inputs are exact in fp32).
__global__ void __launch_bounds__(256) rope_bf16x8_kernel(RopeArgs a, bf16_t* __restrict__ x) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int32_t half = a.rot_dim / 2;
  const int32_t groups = half / 8;
  const int64_t tid = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t total = static_cast<int64_t>(a.batch) * a.rows * groups;
  if (tid >= total) return;
  const int32_t f0 = 8 * static_cast<int32_t>(tid % groups);
  const int64_t br = tid / groups;
  const int64_t row = br % a.rows;
  const int64_t pos = a.positions ? a.positions[br] : augmented_position(row, a.n_text, a.chunk);
  // angles in fp64 (frequencies by repeated ratio, reduced modulo 2 pi in
  // fp64); sine and cosine of the reduced angle in fp32 are far below the
  // bf16 rounding of the outputs
  const double ratio = pow(a.theta, -2.0 / a.rot_dim);
  double inv_freq = pow(a.theta, -2.0 * static_cast<double>(f0) / a.rot_dim);
  constexpr double kTwoPi = 6.283185307179586;
  float cs[8], sn[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const double ang = static_cast<double>(pos) * inv_freq;
    const double red = ang - kTwoPi * rint(ang / kTwoPi);
    sincosf(static_cast<float>(red), &sn[e], &cs[e]);
    inv_freq *= ratio;
  }
  bf16_t* base = x + br * a.heads * static_cast<int64_t>(a.head_dim) + a.rot_off + f0;
#pragma unroll 4
  for (int32_t h = 0; h < a.heads; ++h) {
    bf16_t* p = base + static_cast<int64_t>(h) * a.head_dim;
    const u32x4 lo = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    const u32x4 hi = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p + half));
    u32x4 olo, ohi;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float r_lo[2], r_hi[2];
#pragma unroll
      for (int e2 = 0; e2 < 2; ++e2) {
        const int e = 2 * w + e2;
        const float l = __uint_as_float(e2 ? (lo[w] & 0xffff0000u) : (lo[w] << 16));
        const float u = __uint_as_float(e2 ? (hi[w] & 0xffff0000u) : (hi[w] << 16));
        r_lo[e2] = l * cs[e] - u * sn[e];
        r_hi[e2] = u * cs[e] + l * sn[e];
      }
      olo[w] = pack_bf16x2(r_lo[0], r_lo[1]);
      ohi[w] = pack_bf16x2(r_hi[0], r_hi[1]);
    }
    *reinterpret_cast<u32x4*>(p) = olo;
    *reinterpret_cast<u32x4*>(p + half) = ohi;
  }
}

hipError_t launch_rope(const RopeArgs& a, void* x, int32_t dtype, hipStream_t s) {
  const int64_t total = static_cast<int64_t>(a.batch) * a.rows * (a.rot_dim / 2);
  if (total == 0) return hipSuccess;
  const int threads = 256;
  if (dtype == KSA_DTYPE_BF16 && (a.rot_dim / 2) % 8 == 0 && a.rot_off % 8 == 0 && a.head_dim % 8 == 0) {
    const int64_t blocks8 = (total / 8 + threads - 1) / threads;
    hipLaunchKernelGGL(rope_bf16x8_kernel, dim3(static_cast<uint32_t>(blocks8)), dim3(threads), 0, s, a,
                       static_cast<bf16_t*>(x));
    return hipGetLastError();
  }
  const int64_t blocks = (total + threads - 1) / threads;
  if (dtype == KSA_DTYPE_FP32) {
    hipLaunchKernelGGL(rope_kernel<float>, dim3(static_cast<uint32_t>(blocks)), dim3(threads), 0, s,
                       a, static_cast<float*>(x));
  } else {
    hipLaunchKernelGGL(rope_kernel<bf16_t>, dim3(static_cast<uint32_t>(blocks)), dim3(threads), 0,
                       s, a, static_cast<bf16_t*>(x));
  }
  return hipGetLastError();
}

}  // namespace ksa
