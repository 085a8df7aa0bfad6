// One wavefront attends one query vector to a run of key rows with an
// online (streaming) softmax.  Lanes own strided slices of the head
// dimension: lane l holds elements l, l+64, l+128, ...  This is the
// correctness path used for every shape that has no tuned kernel and for
// the summary-query rows of the prefill (k+1 keys each).
#pragma once

#include "ksa_common.h"

namespace ksa {

template <int NQ, int NV>
struct WaveAttnState {
  float q[NQ];
  float o[NV];
  float m;  // running max, log2 domain
  float l;  // running sum of exp2(s - m)
};

template <typename T, int NQ, int NV>
__device__ __forceinline__ void wave_attn_init(WaveAttnState<NQ, NV>& st, const T* q, int dqk,
                                               float scale_log2, int lane) {
#pragma unroll
  for (int e = 0; e < NQ; ++e) {
    const int d = lane + 64 * e;
    st.q[e] = d < dqk ? load_f32(q + d) * scale_log2 : 0.f;
  }
#pragma unroll
  for (int e = 0; e < NV; ++e) st.o[e] = 0.f;
  st.m = kNegInf;
  st.l = 0.f;
}

// Consume one key/value row.
template <typename T, int NQ, int NV>
__device__ __forceinline__ void wave_attn_step(WaveAttnState<NQ, NV>& st, const T* krow,
                                               const T* vrow, int dqk, int dv, int lane) {
  float part = 0.f;
#pragma unroll
  for (int e = 0; e < NQ; ++e) {
    const int d = lane + 64 * e;
    if (d < dqk) part += st.q[e] * load_f32(krow + d);
  }
  const float s = wave_sum(part);
  const float m_new = fmaxf(st.m, s);
  const float alpha = fast_exp2(st.m - m_new);  // 0 on the first key
  const float p = fast_exp2(s - m_new);
  st.l = st.l * alpha + p;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int d = lane + 64 * e;
    const float vv = d < dv ? load_f32(vrow + d) : 0.f;
    st.o[e] = st.o[e] * alpha + p * vv;
  }
  st.m = m_new;
}

// Write O = o / l and, if requested, the natural-log LSE.  An empty run
// (l == 0) writes zeros and -inf.
template <typename T, int NQ, int NV>
__device__ __forceinline__ void wave_attn_finish(const WaveAttnState<NQ, NV>& st, T* out, int dv,
                                                 float* lse, int lane) {
  const float inv = st.l > 0.f ? 1.f / st.l : 0.f;
#pragma unroll
  for (int e = 0; e < NV; ++e) {
    const int d = lane + 64 * e;
    if (d < dv) store_f32(out + d, st.o[e] * inv);
  }
  if (lse && lane == 0) *lse = st.l > 0.f ? (st.m + log2f(st.l)) * kLn2 : kNegInf;
}

}  // namespace ksa
