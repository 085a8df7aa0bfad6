// Generic KSA prefill: one wavefront per (sequence, query head, augmented
// row), walking only the keys the row may see.
//
// Visible keys ("Kwai Summary Attention Technical Report", Sec. 2.2.1-2.2.2):
//   text t_i, c = floor(i/k):  summaries s_0 .. s_{c-C-1}  (Eq. 3, left term)
//                              text t_{max(0,(c-C)k)} .. t_i (Eq. 2 / Eq. 3 right term)
//   summary s_j:               its chunk's text and itself, which are the k+1
//                              consecutive augmented rows j(k+1) .. j(k+1)+k.
// No mask is formed: the two runs above are enumerated from chunk indices.
// The summary-free baseline modes drop the summary run (SCA) or also replace
// the text run by the last W tokens (SWA).
#include "ksa_attend_wave.h"
#include "ksa_internal.h"

namespace ksa {

template <typename T, int NQ, int NV>
__global__ void __launch_bounds__(256) prefill_generic_kernel(PrefillArgs a, int rows_kind,
                                                              const T* __restrict__ q,
                                                              const T* __restrict__ kx,
                                                              const T* __restrict__ vx,
                                                              T* __restrict__ out,
                                                              float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * (blockDim.x / 64) + (threadIdx.x >> 6);
  const int64_t M = a.n_text / a.k;
  const int64_t R = rows_kind == 1 ? M : a.L;
  const int64_t total = static_cast<int64_t>(a.batch) * R * a.hq;
  if (wave >= total) return;
  const int h = static_cast<int>(wave % a.hq);
  const int64_t br = wave / a.hq;
  const int64_t rr = br % R;
  const int b = static_cast<int>(br / R);
  const int64_t row = rows_kind == 1 ? summary_row(rr, a.k) : rr;
  const int kvh = h / (a.hq / a.hkv);
  const int64_t kstride = static_cast<int64_t>(a.hkv) * a.dqk;  // per augmented row
  const T* kbase = kx + static_cast<int64_t>(b) * a.L * kstride + static_cast<int64_t>(kvh) * a.dqk;
  const T* vbase;
  int64_t vstride;
  if (a.v_is_k_prefix) {
    vbase = kbase;
    vstride = kstride;
  } else {
    vstride = static_cast<int64_t>(a.hkv) * a.dv;
    vbase = vx + static_cast<int64_t>(b) * a.L * vstride + static_cast<int64_t>(kvh) * a.dv;
  }

  WaveAttnState<NQ, NV> st;
  const T* qrow = q + ((static_cast<int64_t>(b) * a.L + row) * a.hq + h) * a.dqk;
  wave_attn_init<T, NQ, NV>(st, qrow, a.dqk, a.scale * kLog2e, lane);
  if (a.rope_theta > 0.0) {
    // Sec. 2.2.1 rotary embedding of the query, half-split over all Dqk
    // columns: pair (f, f + Dqk/2) turns by pos * theta^(-2f/Dqk), in fp64,
    // rounded to T as a separate rotation pass would store it.
    const int half = a.dqk / 2;
    const double pos = static_cast<double>(augmented_position(row, a.n_text, a.k));
#pragma unroll
    for (int e = 0; e < NQ; ++e) {
      const int d = lane + 64 * e;
      if (d < a.dqk) {
        const int f = d < half ? d : d - half;
        double sn, cs;
        sincos(pos * pow(a.rope_theta, -2.0 * f / a.dqk), &sn, &cs);
        const double x = load_f32(qrow + d);
        const double y = load_f32(qrow + (d < half ? d + half : d - half));
        const double r = d < half ? x * cs - y * sn : x * cs + y * sn;
        T rt;
        store_f32(&rt, static_cast<float>(r));
        st.q[e] = load_f32(&rt) * (a.scale * kLog2e);
      }
    }
  }

  // Decode the row through the Eq. 1 layout.
  const int64_t c = row / (a.k + 1);
  const int64_t o = row - c * (a.k + 1);
  const bool is_summary = row < M * (a.k + 1) && o == a.k;
  if (is_summary) {
    for (int64_t r = c * (a.k + 1); r <= row; ++r)
      wave_attn_step<T, NQ, NV>(st, kbase + r * kstride, vbase + r * vstride, a.dqk, a.dv, lane);
  } else {
    const int64_t i = row < M * (a.k + 1) ? c * a.k + o : M * a.k + (row - M * (a.k + 1));
    const int64_t ci = i / a.k;
    // summaries that left the window (KSA only)
    const int64_t ns = a.mode == KSA_MODE_KSA ? ci - a.C : 0;
    for (int64_t j = 0; j < ns; ++j) {
      const int64_t r = summary_row(j, a.k);
      wave_attn_step<T, NQ, NV>(st, kbase + r * kstride, vbase + r * vstride, a.dqk, a.dv, lane);
    }
    int64_t t0 = ci - a.C > 0 ? (ci - a.C) * a.k : 0;  // chunk window (KSA, SCA)
    if (a.mode == KSA_MODE_SWA) t0 = i - a.window_tokens + 1 > 0 ? i - a.window_tokens + 1 : 0;
    for (int64_t t = t0; t <= i; ++t) {
      const int64_t r = text_row(t, a.k);
      wave_attn_step<T, NQ, NV>(st, kbase + r * kstride, vbase + r * vstride, a.dqk, a.dv, lane);
    }
  }
  T* orow = out + ((static_cast<int64_t>(b) * a.L + row) * a.hq + h) * a.dv;
  float* lrow = lse ? lse + (static_cast<int64_t>(b) * a.hq + h) * a.L + row : nullptr;
  wave_attn_finish<T, NQ, NV>(st, orow, a.dv, lrow, lane);
}

template <typename T, int N>
static hipError_t launch_generic_t(const PrefillArgs& a, int rows_kind, const void* q,
                                   const void* k, const void* v, void* out, float* lse,
                                   hipStream_t s) {
  const int64_t M = a.n_text / a.k;
  const int64_t R = rows_kind == 1 ? M : a.L;
  const int64_t waves = static_cast<int64_t>(a.batch) * R * a.hq;
  if (waves == 0) return hipSuccess;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((prefill_generic_kernel<T, N, N>), dim3(static_cast<uint32_t>(blocks)),
                     dim3(256), 0, s, a, rows_kind, static_cast<const T*>(q),
                     static_cast<const T*>(k), static_cast<const T*>(v), static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_generic_d(const PrefillArgs& a, int rows_kind, const void* q,
                                   const void* k, const void* v, void* out, float* lse,
                                   hipStream_t s) {
  const int d = a.dqk > a.dv ? a.dqk : a.dv;
  if (d <= 64) return launch_generic_t<T, 1>(a, rows_kind, q, k, v, out, lse, s);
  if (d <= 128) return launch_generic_t<T, 2>(a, rows_kind, q, k, v, out, lse, s);
  if (d <= 256) return launch_generic_t<T, 4>(a, rows_kind, q, k, v, out, lse, s);
  if (d <= 576) return launch_generic_t<T, 9>(a, rows_kind, q, k, v, out, lse, s);
  return launch_generic_t<T, 16>(a, rows_kind, q, k, v, out, lse, s);
}

hipError_t launch_prefill_generic(const PrefillArgs& a, int32_t dtype, int rows_kind, const void* q,
                                  const void* k, const void* v, void* out, float* lse,
                                  hipStream_t s) {
  if (dtype == KSA_DTYPE_FP32)
    return launch_generic_d<float>(a, rows_kind, q, k, v, out, lse, s);
  return launch_generic_d<bf16_t>(a, rows_kind, q, k, v, out, lse, s);
}

}  // namespace ksa
