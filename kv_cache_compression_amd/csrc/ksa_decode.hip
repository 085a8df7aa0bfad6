// KSA decode attention over the three-region cache.
//
// "Kwai Summary Attention Technical Report", Sec. 2.3.1 and Fig. 4: every
// decode read is one contiguous slice of the cache of a (sequence, kv head):
//   text query:    [filled part of the current chunk | ring | s_0 .. s_{m-C-1}]
//                  start = 1 + k - r,  length = r + min(m, C) k + max(0, m - C)
//   summary query: [scratch | whole current chunk]  start = 0, length = k + 1
// (slot order: scratch, current chunk filled right to left, ring of C chunks,
// summary buffer).  No gather, concatenation or mask is needed; decoding is
// bound by HBM bandwidth.
//
// Two paths:
//   * generic: one wavefront per (sequence, query head) streams the slice;
//   * bf16 Dqk = Dv = 128: split-K over the slice.  Each workgroup takes a
//     row range of one (sequence, kv head) for all query heads of the group:
//     Q.K^T on 16x16x32 bf16 MFMA with K rows loaded straight into the MFMA
//     operand layout, P.V on the vector ALU with one 16-byte V load per lane,
//     then a second kernel merges the per-split (max, sum, output) partials.
#include <mutex>

#include "ksa_attend_wave.h"
#include "ksa_internal.h"

namespace ksa {

typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

struct Slice {
  int64_t start;
  int64_t len;
  bool ok;
};

// kind: 0 text, 1 summary.  state = {m, r, -, err}.
__device__ __forceinline__ Slice decode_slice(const int32_t* st, int kind, int32_t k, int32_t C,
                                             int32_t max_summaries) {
  const int64_t m = st[0];
  const int64_t r = st[1];
  Slice s;
  if (kind == 0) {
    s.start = 1 + k - r;
    s.len = r + (m < C ? m : C) * k + (m > C ? m - C : 0);
    s.ok = r >= 0 && r <= k && m >= 0 && m <= max_summaries;
  } else {
    s.start = 0;
    s.len = k + 1;
    s.ok = r == 0 && m >= 1 && m <= max_summaries;  // the summary was just committed
  }
  if (!s.ok) s.len = 0;
  return s;
}

// ----------------------------------------------------------------- generic --

template <typename T, int NQ, int NV>
__global__ void __launch_bounds__(256) decode_generic_kernel(DecodeArgs a, const T* __restrict__ ck,
                                                             const T* __restrict__ cv,
                                                             int32_t* __restrict__ state,
                                                             const T* __restrict__ q,
                                                             const int32_t* __restrict__ kind,
                                                             T* __restrict__ out,
                                                             float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= static_cast<int64_t>(a.batch) * a.hq) return;
  const int h = static_cast<int>(wave % a.hq);
  const int b = static_cast<int>(wave / a.hq);
  const int kd = kind[b];
  if (kd < 0) return;
  const Slice sl = decode_slice(state + 4 * b, kd, a.k, a.C, a.max_summaries);
  if (!sl.ok && h == 0 && lane == 0) state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SUMMARY_READ;
  const int kvh = h / (a.hq / a.hkv);
  const int64_t seq = static_cast<int64_t>(b) * a.hkv + kvh;
  const T* kc = ck + seq * a.slots * a.dqk;
  const T* vc;
  int64_t vstride;
  if (a.v_is_k_prefix) {
    vc = kc;
    vstride = a.dqk;
  } else {
    vc = cv + seq * a.slots * a.dv;
    vstride = a.dv;
  }
  WaveAttnState<NQ, NV> st;
  wave_attn_init<T, NQ, NV>(st, q + (static_cast<int64_t>(b) * a.hq + h) * a.dqk, a.dqk,
                            a.scale * kLog2e, lane);
  for (int64_t r = sl.start; r < sl.start + sl.len; ++r)
    wave_attn_step<T, NQ, NV>(st, kc + r * a.dqk, vc + r * vstride, a.dqk, a.dv, lane);
  wave_attn_finish<T, NQ, NV>(st, out + (static_cast<int64_t>(b) * a.hq + h) * a.dv, a.dv,
                              lse ? lse + static_cast<int64_t>(b) * a.hq + h : nullptr, lane);
}

template <typename T, int N>
static hipError_t launch_decode_generic_t(const DecodeArgs& a, const void* ck, const void* cv,
                                          int32_t* state, const void* q, const int32_t* kind,
                                          void* out, float* lse, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(a.batch) * a.hq;
  hipLaunchKernelGGL((decode_generic_kernel<T, N, N>), dim3(static_cast<uint32_t>((waves + 3) / 4)),
                     dim3(256), 0, s, a, static_cast<const T*>(ck), static_cast<const T*>(cv),
                     state, static_cast<const T*>(q), kind, static_cast<T*>(out), lse);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_decode_generic(const DecodeArgs& a, const void* ck, const void* cv,
                                        int32_t* state, const void* q, const int32_t* kind,
                                        void* out, float* lse, hipStream_t s) {
  const int d = a.dqk > a.dv ? a.dqk : a.dv;
  if (d <= 64) return launch_decode_generic_t<T, 1>(a, ck, cv, state, q, kind, out, lse, s);
  if (d <= 128) return launch_decode_generic_t<T, 2>(a, ck, cv, state, q, kind, out, lse, s);
  if (d <= 256) return launch_decode_generic_t<T, 4>(a, ck, cv, state, q, kind, out, lse, s);
  if (d <= 576) return launch_decode_generic_t<T, 9>(a, ck, cv, state, q, kind, out, lse, s);
  return launch_decode_generic_t<T, 16>(a, ck, cv, state, q, kind, out, lse, s);
}

// ------------------------------------------------------ split-K, bf16 d128 --

constexpr int kDecWaves = 4;
constexpr int kDecTile = 16;     // rows per wave iteration
constexpr int kDecMaxSplits = 64;

// Rows handled by split `sp` of a slice of `len` rows cut into `ns` splits.
__device__ __forceinline__ void split_range(int64_t len, int ns, int sp, int64_t* r0, int64_t* r1) {
  int64_t per = (len + ns - 1) / ns;
  per = (per + kDecTile - 1) / kDecTile * kDecTile;
  *r0 = per * sp < len ? per * sp : len;
  *r1 = per * (sp + 1) < len ? per * (sp + 1) : len;
}

// Workspace record per (sequence, query head, split): {m (log2 domain), l, o[128]}.
template <int G>
__global__ void __launch_bounds__(256) decode_gqa_d128_split_kernel(
    DecodeArgs a, int nsplit, const bf16_t* __restrict__ ck, const bf16_t* __restrict__ cv,
    const int32_t* __restrict__ state, const bf16_t* __restrict__ q,
    const int32_t* __restrict__ kind, float* __restrict__ ws) {
  constexpr int D = 128;
  const int sp = blockIdx.x;
  const int kvh = blockIdx.y;
  const int b = blockIdx.z;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int kd = kind[b];
  if (kd < 0) return;  // uniform over the block
  const Slice sl = decode_slice(state + 4 * b, kd, a.k, a.C, a.max_summaries);
  int64_t r0, r1;
  split_range(sl.len, nsplit, sp, &r0, &r1);

  const int64_t seq = static_cast<int64_t>(b) * a.hkv + kvh;
  const bf16_t* kc = ck + (seq * a.slots + sl.start) * D;
  const bf16_t* vc = cv + (seq * a.slots + sl.start) * D;

  // Q^T as the B operand of Q.K^T: column n = head (lane % 16), k-slots
  // d = 32 ks + 8 (lane / 16) + j.
  const int col = lane & 15;
  const int grp = lane >> 4;
  bf16x8_t qop[4];
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    if (col < G) {
      const bf16_t* qp = q + (static_cast<int64_t>(b) * a.hq + kvh * G + col) * D + 32 * ks + 8 * grp;
      qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp);
    } else {
      qop[ks] = bf16x8_t{};
    }
  }
  const float sc = a.scale * kLog2e;

  // P and alpha exchange between the MFMA layout and the V layout.
  __shared__ float p_lds[kDecWaves][kDecTile][16];
  __shared__ float a_lds[kDecWaves][16];
  __shared__ float red_m[kDecWaves][G];
  __shared__ float red_l[kDecWaves][G];
  __shared__ float red_o[kDecWaves][G][D];

  float m_run = kNegInf;  // per head (lane % 16) in the MFMA layout
  float l_run = 0.f;      // partial over this lane's rows
  float o[G][8];          // V layout: d = 8 (lane % 16) + e, rows with row % 4 == lane / 16
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) o[h][e] = 0.f;

  // K and V rows of the next tile are loaded while the current one is used
  // (rows clamped into the range; a clamped row gets weight 0).  The slice is
  // read once per step: non-temporal loads (about 8% faster than cached ones
  // here, at the streaming-read rate).
  const int64_t stride = kDecWaves * kDecTile;
  auto load_k = [&](int64_t t, bf16x8_t* kop) {
    const int64_t kr = t + col < r1 ? t + col : r1 - 1;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
      kop[ks] = __builtin_bit_cast(bf16x8_t, __builtin_nontemporal_load(
                                                  reinterpret_cast<const u32x4_t*>(kc + kr * D + 32 * ks + 8 * grp)));
  };
  auto load_v = [&](int64_t t, uint4* vr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = t + grp + 4 * i;
      vr[i] = __builtin_bit_cast(uint4, __builtin_nontemporal_load(
                                            reinterpret_cast<const u32x4_t*>(vc + (row < r1 ? row : r1 - 1) * D + 8 * col)));
    }
  };
  int64_t t0 = r0 + static_cast<int64_t>(wave) * kDecTile;
  bf16x8_t kop_n[4];
  uint4 v_n[4];
  if (t0 < r1) {
    load_k(t0, kop_n);
    load_v(t0, v_n);
  }
  for (; t0 < r1; t0 += stride) {
    bf16x8_t kop[4];
    uint4 vr[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) kop[ks] = kop_n[ks];
#pragma unroll
    for (int i = 0; i < 4; ++i) vr[i] = v_n[i];
    if (t0 + stride < r1) {
      load_k(t0 + stride, kop_n);
      load_v(t0 + stride, v_n);
    }
    // ---- S = K Q^T for 16 rows (MFMA, A = K rows) ----
    f32x4_t s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) s = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kop[ks], qop[ks], s, 0, 0, 0);
    // C layout: lane holds head `col`, rows 4 grp + i.
    float sv[4];
    float tmax = kNegInf;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = t0 + 4 * grp + i;
      sv[i] = row < r1 ? s[i] * sc : kNegInf;
      tmax = fmaxf(tmax, sv[i]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float p = fast_exp2(sv[i] - m_use);
      psum += p;
      p_lds[wave][4 * grp + i][col] = p;
    }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (grp == 0) a_lds[wave][col] = alpha;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): LDS writes done
    __builtin_amdgcn_wave_barrier();

    // ---- O += P V (vector ALU, lane owns 8 d of rows grp, grp+4, ...) ----
    float al[G];
#pragma unroll
    for (int h = 0; h < G; ++h) al[h] = a_lds[wave][h];
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) o[h][e] *= al[h];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int rl = grp + 4 * i;
      const uint4 vraw = vr[i];
      float vv[8];
      vv[0] = __uint_as_float(vraw.x << 16);
      vv[1] = __uint_as_float(vraw.x & 0xffff0000u);
      vv[2] = __uint_as_float(vraw.y << 16);
      vv[3] = __uint_as_float(vraw.y & 0xffff0000u);
      vv[4] = __uint_as_float(vraw.z << 16);
      vv[5] = __uint_as_float(vraw.z & 0xffff0000u);
      vv[6] = __uint_as_float(vraw.w << 16);
      vv[7] = __uint_as_float(vraw.w & 0xffff0000u);
#pragma unroll
      for (int h = 0; h < G; ++h) {
        const float p = p_lds[wave][rl][h];  // 0 for rows past the range
#pragma unroll
        for (int e = 0; e < 8; ++e) o[h][e] += p * vv[e];
      }
    }
    __builtin_amdgcn_wave_barrier();  // p_lds reuse in the next tile
  }

  // ---- reduce within the wave ----
  // l: lanes of one head (col) hold partial sums of different rows.
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int h = 0; h < G; ++h)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float x = o[h][e];
      x += __shfl_xor(x, 16);
      x += __shfl_xor(x, 32);
      o[h][e] = x;
    }
  if (lane < G) {
    red_m[wave][lane] = m_run;
    red_l[wave][lane] = l_run;
  }
  if (grp == 0) {
#pragma unroll
    for (int h = 0; h < G; ++h)
#pragma unroll
      for (int e = 0; e < 8; ++e) red_o[wave][h][8 * col + e] = o[h][e];
  }
  __syncthreads();
  // ---- reduce across the waves and write the split's partial ----
  for (int idx = threadIdx.x; idx < G * (D + 2); idx += blockDim.x) {
    const int h = idx / (D + 2);
    const int c = idx % (D + 2);
    float mx = kNegInf;
#pragma unroll
    for (int w = 0; w < kDecWaves; ++w) mx = fmaxf(mx, red_m[w][h]);
    const float mu = mx == kNegInf ? 0.f : mx;
    float acc = 0.f;
    if (c == 0) {
      acc = mx;
    } else {
#pragma unroll
      for (int w = 0; w < kDecWaves; ++w) {
        const float wgt = fast_exp2(red_m[w][h] - mu);
        acc += wgt * (c == 1 ? red_l[w][h] : red_o[w][h][c - 2]);
      }
    }
    const int hq = kvh * G + h;
    ws[((static_cast<int64_t>(b) * a.hq + hq) * nsplit + sp) * (D + 2) + c] = acc;
  }
}

// Merge the split partials of one (sequence, query head) per workgroup.
template <typename T>
__global__ void __launch_bounds__(128) decode_merge_kernel(DecodeArgs a, int nsplit,
                                                           int32_t* __restrict__ state,
                                                           const int32_t* __restrict__ kind,
                                                           const float* __restrict__ ws,
                                                           T* __restrict__ out,
                                                           float* __restrict__ lse) {
  const int hq = blockIdx.x;
  const int b = blockIdx.y;
  if (kind[b] < 0) return;
  // error flag for a summary read that finds no freshly committed chunk (the
  // split kernel has read the state by now)
  if (hq == 0 && threadIdx.x == 0 && !decode_slice(state + 4 * b, kind[b], a.k, a.C, a.max_summaries).ok)
    state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SUMMARY_READ;
  const int D = a.dv;
  const float* rec = ws + (static_cast<int64_t>(b) * a.hq + hq) * nsplit * (D + 2);
  float mx = kNegInf;
  for (int s = 0; s < nsplit; ++s) mx = fmaxf(mx, rec[s * (D + 2)]);
  const float mu = mx == kNegInf ? 0.f : mx;
  float l = 0.f;
  for (int s = 0; s < nsplit; ++s) l += fast_exp2(rec[s * (D + 2)] - mu) * rec[s * (D + 2) + 1];
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = threadIdx.x; d < D; d += blockDim.x) {
    float acc = 0.f;
    for (int s = 0; s < nsplit; ++s) acc += fast_exp2(rec[s * (D + 2)] - mu) * rec[s * (D + 2) + 2 + d];
    store_f32(out + (static_cast<int64_t>(b) * a.hq + hq) * D + d, acc * inv);
  }
  if (lse && threadIdx.x == 0)
    lse[static_cast<int64_t>(b) * a.hq + hq] = l > 0.f ? (mx + log2f(l)) * kLn2 : kNegInf;
}

static bool gqa_fast_ok(const DecodeArgs& a, int32_t dtype) {
  const int g = a.hq / a.hkv;
  return dtype == KSA_DTYPE_BF16 && a.dqk == 128 && a.dv == 128 && !a.v_is_k_prefix &&
         (g == 1 || g == 2 || g == 4 || g == 8 || g == 16);
}

static int choose_splits(const DecodeArgs& a) {
  const int64_t cap = static_cast<int64_t>(a.k) + static_cast<int64_t>(a.C) * a.k + a.max_summaries + 1;
  const int64_t pairs = static_cast<int64_t>(a.batch) * a.hkv;
  int ns = static_cast<int>((2048 + pairs - 1) / pairs);  // about 8 workgroups per CU
  const int64_t by_len = (cap + 255) / 256;               // at least 256 rows each
  if (ns > by_len) ns = static_cast<int>(by_len);
  if (ns > kDecMaxSplits) ns = kDecMaxSplits;
  if (ns < 1) ns = 1;
  return ns;
}

size_t decode_workspace_bytes(const DecodeArgs& a) {
  // sized for either split-K path; the generic path needs none
  const size_t gqa = static_cast<size_t>(a.batch) * a.hq * kDecMaxSplits * (a.dv + 2) * sizeof(float);
  return a.v_is_k_prefix ? decode_mla_workspace_bytes(a) : gqa;
}

size_t decode_workspace_bytes_used(const DecodeArgs& a, int32_t dtype) {
  if (decode_mla_supported(a, dtype)) return decode_mla_workspace_bytes_used(a);
  if (!gqa_fast_ok(a, dtype)) return 0;
  return static_cast<size_t>(a.batch) * a.hq * choose_splits(a) * (a.dv + 2) * sizeof(float);
}

// ------------------------------------------------------- allocation-free --

// Scratch of the allocation-free decode (split partials and, for the MLA
// path, the cut): one copy per GPU, set up by the runtime when this code
// object is loaded and held until the process ends.  On the host `scratch`
// names a stand-in, not device memory: host code uses only the address
// decode_scratch() looks up.  Every call on a GPU shares that GPU's copy;
// each launch writes every record it later reads, so nothing needs clearing,
// but calls that overlap on one GPU race.
const size_t kDecodeScratchBytes = size_t(128) << 20;
static __device__ __align__(256) char scratch[size_t(128) << 20];

hipError_t decode_scratch(void** ptr) {
  constexpr int kMaxDev = 64;
  static std::mutex mu;
  static void* addr[kMaxDev] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

template <int G>
static hipError_t launch_gqa(const DecodeArgs& a, int ns, const void* ck, const void* cv,
                             const int32_t* state, const void* q, const int32_t* kind, float* ws,
                             hipStream_t s) {
  hipLaunchKernelGGL((decode_gqa_d128_split_kernel<G>), dim3(ns, a.hkv, a.batch), dim3(256), 0, s,
                     a, ns, static_cast<const bf16_t*>(ck), static_cast<const bf16_t*>(cv), state,
                     static_cast<const bf16_t*>(q), kind, ws);
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, int32_t dtype, const void* ck, const void* cv,
                         const int32_t* state, const void* q, const int32_t* kind, void* out,
                         float* lse, void* ws, hipStream_t s) {
  int32_t* st = const_cast<int32_t*>(state);
  if (decode_mla_supported(a, dtype)) return launch_decode_mla(a, ck, st, q, kind, out, lse, ws, s);
  if (!gqa_fast_ok(a, dtype)) {
    if (dtype == KSA_DTYPE_FP32)
      return launch_decode_generic<float>(a, ck, cv, st, q, kind, out, lse, s);
    return launch_decode_generic<bf16_t>(a, ck, cv, st, q, kind, out, lse, s);
  }
  hipError_t e = hipSuccess;
  const int ns = choose_splits(a);
  float* w = static_cast<float*>(ws);
  switch (a.hq / a.hkv) {
    case 1: e = launch_gqa<1>(a, ns, ck, cv, state, q, kind, w, s); break;
    case 2: e = launch_gqa<2>(a, ns, ck, cv, state, q, kind, w, s); break;
    case 4: e = launch_gqa<4>(a, ns, ck, cv, state, q, kind, w, s); break;
    case 8: e = launch_gqa<8>(a, ns, ck, cv, state, q, kind, w, s); break;
    default: e = launch_gqa<16>(a, ns, ck, cv, state, q, kind, w, s); break;
  }
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_merge_kernel<bf16_t>, dim3(a.hq, a.batch), dim3(128), 0, s, a, ns, st, kind,
                     w, static_cast<bf16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace ksa
