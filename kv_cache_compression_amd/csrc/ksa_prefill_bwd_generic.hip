// Generic backward of the KSA prefill attention, any dtype and head dims up
// to 1024: one wavefront per output row.
//
// The forward is masked softmax attention (Eq. 10 of "Kwai Summary
// Attention Technical Report") over the visible pairs of Sec. 2.2; its
// gradient touches exactly the same pairs.  With the forward's natural-log
// normaliser lse_i the probabilities are recomputed directly,
// p_ij = exp(scale q_i.k_j - lse_i), and with delta_i = dout_i . out_i
// (the row's sum of p_ij dP_ij):
//   dS_ij = p_ij (dout_i . v_j - delta_i)
//   dq_i  = scale sum_j dS_ij k_j       (one wave per query row, its keys)
//   dk_j  = scale sum_i dS_ij q_i       (one wave per key row, the queries
//   dv_j  =       sum_i p_ij dout_i      that see it, all heads of its group)
// Queries that see key row j:
//   summary s_j:  s_j itself, and (KSA) every text t_i with
//                 floor(i/k) - C - 1 >= j;
//   text t_x, chunk c = floor(x/k):  the summary s_c (if chunk c is
//                 complete) and text t_x .. t_{(c+C+1)k-1} (chunk window),
//                 or t_x .. t_{x+W-1} (token window).
#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

// delta[b, h, row] = sum_d dout * out, fp32.  One wave per (row, head).
template <typename T>
__global__ void __launch_bounds__(256) bwd_delta_kernel(int64_t rows, int32_t hq, int32_t dv, int64_t L,
                                                        const T* __restrict__ out,
                                                        const T* __restrict__ dout,
                                                        float* __restrict__ delta) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= rows * hq) return;
  const int64_t base = wave * dv;  // (b, row, h) row-major == wave order
  float acc = 0.f;
  for (int d = lane; d < dv; d += 64) acc += load_f32(out + base + d) * load_f32(dout + base + d);
  acc = wave_sum(acc);
  if (lane == 0) {
    const int h = static_cast<int>(wave % hq);
    const int64_t br = wave / hq;
    const int64_t b = br / L, row = br % L;
    delta[(b * hq + h) * L + row] = acc;
  }
}

// bf16 with Dv = 128: 16 lanes per (row, head), 8 elements per lane.
__global__ void __launch_bounds__(256) bwd_delta_d128_bf16_kernel(int64_t rows, int32_t hq, int64_t L,
                                                                  const bf16_t* __restrict__ out,
                                                                  const bf16_t* __restrict__ dout,
                                                                  float* __restrict__ delta) {
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  const bool ok = item < rows * hq;
  float acc = 0.f;
  if (ok) {
    const u32x4 o = *reinterpret_cast<const u32x4*>(out + item * 128 + 8 * c);
    const u32x4 g = *reinterpret_cast<const u32x4*>(dout + item * 128 + 8 * c);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc += __uint_as_float(o[e] << 16) * __uint_as_float(g[e] << 16);
      acc += __uint_as_float(o[e] & 0xffff0000u) * __uint_as_float(g[e] & 0xffff0000u);
    }
  }
  acc += __shfl_xor(acc, 8);
  acc += __shfl_xor(acc, 4);
  acc += __shfl_xor(acc, 2);
  acc += __shfl_xor(acc, 1);
  if (ok && c == 0) {
    const int h = static_cast<int>(item % hq);
    const int64_t br = item / hq;
    delta[(br / L * hq + h) * L + br % L] = acc;
  }
}

namespace {

template <typename T, int N>
__device__ __forceinline__ void load_vec(float (&x)[N], const T* p, int d_lim, int lane, float mul = 1.f) {
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int d = lane + 64 * e;
    x[e] = d < d_lim ? load_f32(p + d) * mul : 0.f;
  }
}

template <int N>
__device__ __forceinline__ float dot_wave(const float (&a)[N], const float (&b)[N]) {
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < N; ++e) s += a[e] * b[e];
  return wave_sum(s);
}

}  // namespace

// dq: one wave per (b, h, augmented row).
template <typename T, int N>
__global__ void __launch_bounds__(256) bwd_dq_generic_kernel(PrefillArgs a, const T* __restrict__ q,
                                                             const T* __restrict__ kx,
                                                             const T* __restrict__ vx,
                                                             const T* __restrict__ dout,
                                                             const float* __restrict__ lse,
                                                             const float* __restrict__ delta,
                                                             T* __restrict__ dq) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= static_cast<int64_t>(a.batch) * a.L * a.hq) return;
  const int h = static_cast<int>(wave % a.hq);
  const int64_t br = wave / a.hq;
  const int64_t row = br % a.L;
  const int b = static_cast<int>(br / a.L);
  const int kvh = h / (a.hq / a.hkv);
  const int64_t M = a.n_text / a.k;
  const int64_t ks = static_cast<int64_t>(a.hkv) * a.dqk, vs = static_cast<int64_t>(a.hkv) * a.dv;
  const T* kb = kx + static_cast<int64_t>(b) * a.L * ks + static_cast<int64_t>(kvh) * a.dqk;
  const T* vb = vx + static_cast<int64_t>(b) * a.L * vs + static_cast<int64_t>(kvh) * a.dv;
  const int64_t qoff = ((static_cast<int64_t>(b) * a.L + row) * a.hq + h);
  float qv[N], gv[N], acc[N];
  load_vec<T, N>(qv, q + qoff * a.dqk, a.dqk, lane);
  load_vec<T, N>(gv, dout + qoff * a.dv, a.dv, lane);
#pragma unroll
  for (int e = 0; e < N; ++e) acc[e] = 0.f;
  const int64_t srow = (static_cast<int64_t>(b) * a.hq + h) * a.L + row;
  const float lse2 = lse[srow] * kLog2e;
  const float dlt = delta[srow];
  const float sl = a.scale * kLog2e;
  auto step = [&](int64_t r) {
    float kv[N], vv[N];
    load_vec<T, N>(kv, kb + r * ks, a.dqk, lane);
    load_vec<T, N>(vv, vb + r * vs, a.dv, lane);
    const float p = fast_exp2(dot_wave<N>(qv, kv) * sl - lse2);
    const float ds = p * (dot_wave<N>(gv, vv) - dlt);
#pragma unroll
    for (int e = 0; e < N; ++e) acc[e] += ds * kv[e];
  };
  const int64_t c = row / (a.k + 1);
  const int64_t o = row - c * (a.k + 1);
  if (row < M * (a.k + 1) && o == a.k) {
    for (int64_t r = c * (a.k + 1); r <= row; ++r) step(r);
  } else {
    const int64_t i = row < M * (a.k + 1) ? c * a.k + o : M * a.k + (row - M * (a.k + 1));
    const int64_t ci = i / a.k;
    const int64_t ns = a.mode == KSA_MODE_KSA ? ci - a.C : 0;
    for (int64_t j = 0; j < ns; ++j) step(summary_row(j, a.k));
    int64_t t0 = ci - a.C > 0 ? (ci - a.C) * a.k : 0;
    if (a.mode == KSA_MODE_SWA) t0 = i - a.window_tokens + 1 > 0 ? i - a.window_tokens + 1 : 0;
    for (int64_t t = t0; t <= i; ++t) step(text_row(t, a.k));
  }
  T* dst = dq + qoff * a.dqk;
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int d = lane + 64 * e;
    if (d < a.dqk) store_f32(dst + d, acc[e] * a.scale);
  }
}

// dk, dv: one wave per (b, kv head, augmented key row), all heads of the group.
template <typename T, int N>
__global__ void __launch_bounds__(256) bwd_dkdv_generic_kernel(PrefillArgs a, const T* __restrict__ q,
                                                               const T* __restrict__ kx,
                                                               const T* __restrict__ vx,
                                                               const T* __restrict__ dout,
                                                               const float* __restrict__ lse,
                                                               const float* __restrict__ delta,
                                                               T* __restrict__ dk, T* __restrict__ dv) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= static_cast<int64_t>(a.batch) * a.L * a.hkv) return;
  const int kvh = static_cast<int>(wave % a.hkv);
  const int64_t br = wave / a.hkv;
  const int64_t r = br % a.L;
  const int b = static_cast<int>(br / a.L);
  const int g = a.hq / a.hkv;
  const int64_t M = a.n_text / a.k;
  const int64_t koff = (static_cast<int64_t>(b) * a.L + r) * a.hkv + kvh;
  float kv[N], vv[N], dka[N], dva[N];
  load_vec<T, N>(kv, kx + koff * a.dqk, a.dqk, lane);
  load_vec<T, N>(vv, vx + koff * a.dv, a.dv, lane);
#pragma unroll
  for (int e = 0; e < N; ++e) dka[e] = dva[e] = 0.f;
  const float sl = a.scale * kLog2e;
  for (int hh = 0; hh < g; ++hh) {
    const int h = kvh * g + hh;
    auto step = [&](int64_t qr) {
      const int64_t qoff = (static_cast<int64_t>(b) * a.L + qr) * a.hq + h;
      const int64_t srow = (static_cast<int64_t>(b) * a.hq + h) * a.L + qr;
      float qv[N], gv[N];
      load_vec<T, N>(qv, q + qoff * a.dqk, a.dqk, lane);
      load_vec<T, N>(gv, dout + qoff * a.dv, a.dv, lane);
      const float p = fast_exp2(dot_wave<N>(qv, kv) * sl - lse[srow] * kLog2e);
      const float ds = p * (dot_wave<N>(gv, vv) - delta[srow]);
#pragma unroll
      for (int e = 0; e < N; ++e) {
        dva[e] += p * gv[e];
        dka[e] += ds * qv[e];
      }
    };
    const int64_t c = r / (a.k + 1);
    const int64_t o = r - c * (a.k + 1);
    if (r < M * (a.k + 1) && o == a.k) {
      step(r);  // the summary itself
      if (a.mode == KSA_MODE_KSA)
        for (int64_t i = (c + a.C + 1) * a.k; i < a.n_text; ++i) step(text_row(i, a.k));
    } else {
      const int64_t x = r < M * (a.k + 1) ? c * a.k + o : M * a.k + (r - M * (a.k + 1));
      const int64_t cx = x / a.k;
      if (cx < M) step(summary_row(cx, a.k));
      int64_t hi = a.mode == KSA_MODE_SWA ? x + a.window_tokens - 1 : (cx + a.C + 1) * a.k - 1;
      if (hi > a.n_text - 1) hi = a.n_text - 1;
      for (int64_t i = x; i <= hi; ++i) step(text_row(i, a.k));
    }
  }
#pragma unroll
  for (int e = 0; e < N; ++e) {
    const int d = lane + 64 * e;
    if (d < a.dqk) store_f32(dk + koff * a.dqk + d, dka[e] * a.scale);
    if (d < a.dv) store_f32(dv + koff * a.dv + d, dva[e]);
  }
}

hipError_t launch_bwd_delta(const PrefillArgs& a, int32_t dtype, const void* out, const void* dout,
                            float* delta, hipStream_t s) {
  const int64_t rows = static_cast<int64_t>(a.batch) * a.L;
  const int64_t items = rows * a.hq;
  if (items == 0) return hipSuccess;
  if (dtype == KSA_DTYPE_BF16 && a.dv == 128) {
    hipLaunchKernelGGL(bwd_delta_d128_bf16_kernel, dim3(static_cast<uint32_t>((items + 15) / 16)), dim3(256),
                       0, s, rows, a.hq, a.L, static_cast<const bf16_t*>(out), static_cast<const bf16_t*>(dout),
                       delta);
  } else if (dtype == KSA_DTYPE_BF16) {
    hipLaunchKernelGGL(bwd_delta_kernel<bf16_t>, dim3(static_cast<uint32_t>((items + 3) / 4)), dim3(256), 0, s,
                       rows, a.hq, a.dv, a.L, static_cast<const bf16_t*>(out),
                       static_cast<const bf16_t*>(dout), delta);
  } else {
    hipLaunchKernelGGL(bwd_delta_kernel<float>, dim3(static_cast<uint32_t>((items + 3) / 4)), dim3(256), 0, s,
                       rows, a.hq, a.dv, a.L, static_cast<const float*>(out), static_cast<const float*>(dout),
                       delta);
  }
  return hipGetLastError();
}

template <typename T, int N>
static hipError_t launch_bwd_generic_t(const PrefillArgs& a, const void* q, const void* k, const void* v,
                                       const void* dout, const float* lse, const float* delta, void* dq,
                                       void* dk, void* dv, hipStream_t s) {
  const int64_t wq = static_cast<int64_t>(a.batch) * a.L * a.hq;
  const int64_t wk = static_cast<int64_t>(a.batch) * a.L * a.hkv;
  hipLaunchKernelGGL((bwd_dq_generic_kernel<T, N>), dim3(static_cast<uint32_t>((wq + 3) / 4)), dim3(256), 0, s,
                     a, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(dout), lse, delta, static_cast<T*>(dq));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dkdv_generic_kernel<T, N>), dim3(static_cast<uint32_t>((wk + 3) / 4)), dim3(256), 0,
                     s, a, static_cast<const T*>(q), static_cast<const T*>(k), static_cast<const T*>(v),
                     static_cast<const T*>(dout), lse, delta, static_cast<T*>(dk), static_cast<T*>(dv));
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_bwd_generic_d(const PrefillArgs& a, const void* q, const void* k, const void* v,
                                       const void* dout, const float* lse, const float* delta, void* dq,
                                       void* dk, void* dv, hipStream_t s) {
  const int d = a.dqk > a.dv ? a.dqk : a.dv;
  if (d <= 64) return launch_bwd_generic_t<T, 1>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
  if (d <= 128) return launch_bwd_generic_t<T, 2>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
  if (d <= 256) return launch_bwd_generic_t<T, 4>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
  if (d <= 576) return launch_bwd_generic_t<T, 9>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
  return launch_bwd_generic_t<T, 16>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
}

hipError_t launch_prefill_bwd_generic(const PrefillArgs& a, int32_t dtype, const void* q, const void* k,
                                      const void* v, const void* dout, const float* lse, const float* delta,
                                      void* dq, void* dk, void* dv, hipStream_t s) {
  if (static_cast<int64_t>(a.batch) * a.L == 0) return hipSuccess;
  if (dtype == KSA_DTYPE_FP32)
    return launch_bwd_generic_d<float>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
  return launch_bwd_generic_d<bf16_t>(a, q, k, v, dout, lse, delta, dq, dk, dv, s);
}

}  // namespace ksa
