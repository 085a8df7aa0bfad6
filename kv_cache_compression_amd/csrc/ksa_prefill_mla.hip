// KSA prefill in the absorbed-MLA form for bf16: 128 query heads share one
// latent key/value head, keys are 576 wide (512 latent + 64 rotary) and
// values are the first 512 key columns.
//
// "Kwai Summary Attention Technical Report", Sec. 3.2, Eq. (6) and Table 1
// (summary compression composed with MLA) and Sec. 2.3 (block-sparse
// prefill): every augmented row attends, for all 128 heads, to the keys the
// Eq. (3) rule gives it: a text row t_i (chunk c) to the summaries
// s_0 .. s_{c-C-1} and the text t_{(c-C)k} .. t_i, a summary row s_j to the
// k + 1 rows of its chunk.
//
// One workgroup of 8 wavefronts per (sequence, augmented row) computes all
// 128 heads, so each key tile staged in LDS feeds 128 query rows; tiles of
// 32 keys walk the row's summary run, then its text run (only a run's last
// tile is partial), loaded straight into LDS, three buffers deep, with
// per-lane row addresses from the Eq. (1) map (summary j at row j(k+1)+k,
// text x at x + x/k).  Waves 2p and 2p+1 own heads 32p .. 32p+31: wave
// 2p+h forms the part of S^T = K Q^T over key columns 288h .. 288h+287 on
// 32x32x16 bf16 MFMA, the two parts are summed through LDS (the same sum in
// both waves), both run the same softmax, and wave 2p+h accumulates value
// columns 256h .. 256h+255 of O^T += V^T P^T, V^T read through
// ds_read_b64_tr_b16 from the same tile.  Each wave thus holds half of Q
// and of O, and reads half of each tile per 32 heads, which halves the LDS
// operand traffic of the full-width 16-head split (the limit there: 544 KB
// of operand reads per 32-key tile and CU).  The reference maximum moves
// only when a tile exceeds it by more than 2^8 (the accumulators are then
// rescaled in place).  Rows are taken longest first (text rows from the end
// of the sequence), summary rows last.
#include <type_traits>

#include "ksa_internal.h"
#include "ksa_mfma_common.h"

namespace ksa {

namespace {

using namespace mfma;

constexpr int DQK = 576, DV = 512;
constexpr int HQ = 128;
constexpr int TK = 32;                  // keys per tile
constexpr int GRB = DQK * 2;            // bytes per augmented row in HBM: 1152
constexpr int RB = GRB + 16;            // padded LDS row: 1168 bytes (73 chunks)
constexpr int RCH = RB / 16;            // 73
constexpr int TILE_LDS = 37 * 64 * 16;  // 37888 bytes >= 32 x 1168
constexpr int KPF = 4;                  // K operand reads issued this many MFMAs ahead
constexpr int VPF = 4;                  // V^T operand reads issued this many MFMAs ahead
constexpr int NBUF = 3;
constexpr float kLazy = 8.f;

typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

struct MlaPrefillArgs {
  int32_t batch, n, L, k, C, M;
  uint32_t divk_m, divk_l;
  float sl;
};

}  // namespace

__global__ void __launch_bounds__(512, 1) prefill_mla_kernel(MlaPrefillArgs a, const bf16_t* __restrict__ kx,
                                                             const bf16_t* __restrict__ q, bf16_t* __restrict__ out,
                                                             float* __restrict__ lse) {
  __shared__ __attribute__((aligned(16))) char lds0[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds1[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds2[TILE_LDS];
  // partial S^T exchange between the two waves of a pair: 16 values + 4
  // padding per lane
  __shared__ __attribute__((aligned(16))) float xs[8][64][20];
  char* const lds[NBUF] = {lds0, lds1, lds2};

  // row of this workgroup: text rows from the last backwards, then summaries
  const int b = blockIdx.x % a.batch;
  const int idx = blockIdx.x / a.batch;
  bool is_sum;
  int row, ns, sn, t0, x_last;  // summary run [0, sn), text run [t0, x_last]
  if (idx < a.n) {
    const int i = a.n - 1 - idx;
    const int c = fast_div_apply(i, a.divk_m, a.divk_l);
    is_sum = false;
    row = i + c;
    sn = c - a.C > 0 ? c - a.C : 0;
    t0 = c - a.C > 0 ? (c - a.C) * a.k : 0;
    x_last = i;
  } else {
    const int j = idx - a.n;
    is_sum = true;
    row = j * (a.k + 1) + a.k;
    sn = 0;
    t0 = j * (a.k + 1);  // the k + 1 contiguous rows of the chunk, as raw rows
    x_last = row;
  }
  sn = __builtin_amdgcn_readfirstlane(sn);
  t0 = __builtin_amdgcn_readfirstlane(t0);
  x_last = __builtin_amdgcn_readfirstlane(x_last);
  row = __builtin_amdgcn_readfirstlane(row);
  ns = (sn + TK - 1) / TK;
  const int ntile = ns + (x_last - t0 + TK) / TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1;  // heads 32 pair .. 32 pair + 31
  const int hf = wave & 1;     // key columns 288 hf .., value columns 256 hf ..
  const int half = lane >> 5;
  const int head = 32 * pair + (lane & 31);
  const int64_t qo = (static_cast<int64_t>(b) * a.L + row) * HQ + head;

  // Q^T (this wave's key-column half) as the B operand of S^T = K Q^T on
  // 32x32x16 MFMA: column = head (lane % 32), k-slots d = 288 hf + 16 ks + 8 half + j.
  bf16x8_t qop[18];
  {
    const bf16_t* qp = q + qo * DQK + 288 * hf + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
  }

  // Tile loads: chunk s = 64 (8 i + wave) + lane of a tile (i < 5,
  // 8 i + wave < 37) is tile row s / 73, 16-byte chunk s % 73 (chunk 72 is
  // LDS padding and reads 16 bytes past the row).
  const int nld = wave < 5 ? 5 : 4;
  auto trw = [&](int i) { return ((8 * i + wave) * 64 + lane) / RCH; };
  auto tch = [&](int i) { return 16 * (((8 * i + wave) * 64 + lane) % RCH); };
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(kx + static_cast<int64_t>(b) * a.L * DQK), static_cast<short>(0), a.L * GRB, 0x00020000);
  auto prefetch = [&](int t, char* buf) __attribute__((always_inline)) {
    // the per-lane row and chunk of each load are formed here, each time:
    // kept across the loop they are spilled, and a spill reload waits for
    // every tile copy in flight
    int ln = lane;
    asm volatile("" : "+v"(ln));
    auto trw = [&](int i) { return ((8 * i + wave) * 64 + ln) / RCH; };
    auto tch = [&](int i) { return 16 * (((8 * i + wave) * 64 + ln) % RCH); };
    int vo[5];
    if (t < ns) {
      const int j0 = t * TK;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int j = min(j0 + trw(i), sn - 1);
        vo[i] = (j * (a.k + 1) + a.k) * GRB + tch(i);
      }
    } else {
      const int x0 = t0 + (t - ns) * TK;
#pragma unroll
      for (int i = 0; i < 5; ++i) {
        const int x = min(x0 + trw(i), x_last);
        const int r = is_sum ? x : x + fast_div_apply(x, a.divk_m, a.divk_l);
        vo[i] = r * GRB + tch(i);
      }
    }
#pragma unroll
    for (int i = 0; i < 5; ++i)
      if (i < nld)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(buf + (8 * i + wave) * 1024), 16, vo[i], 0, 0, 0);
  };

  // O^T over this wave's 256 value columns in 8 blocks of 32: lane holds
  // head lane % 32, d = 256 hf + 32 db + 8 (r / 4) + 4 half + r % 4.
  f32x16_t oacc[8];
  float l_run = 0.f;
  float m_ref = kNegInf;
  const uint32_t one2 = 0x3f803f80u;
  // K operand: row = key lane % 32, bytes 576 hf + 32 ks + 16 half.
  const int krow_off = (lane & 31) * RB + 16 * half + 576 * hf;
  // V^T operand: in 16-lane group G, lane (4 rr + c4) reads key row
  // 4 (G / 2) + rr (+ 8 for the second half of the k-slots) and d =
  // 256 hf + 32 db + 16 (G % 2) + 4 c4; the transposing read gives lane i
  // V[4 keys][d = 256 hf + 32 db + i % 32].
  const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
  const int vrow_off = (4 * (G >> 1) + rr) * RB + 2 * (16 * (G & 1) + 4 * c4) + 512 * hf;

  auto tile_step = [&](auto cur_c, int t) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    if (t + 1 < ntile) {
      if (wave < 5)
        __builtin_amdgcn_s_waitcnt(0x0075);  // vmcnt(5) lgkmcnt(0)
      else
        __builtin_amdgcn_s_waitcnt(0x0074);  // vmcnt(4) lgkmcnt(0)
    } else {
      __builtin_amdgcn_s_waitcnt(0x0070);  // vmcnt(0) lgkmcnt(0)
    }
    wg_barrier();
    const char* kl = lds[cur];
    // ---- this wave's half of S^T = K Q^T (keys x heads, 32 x 32) ----
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
    bf16x8_t kring[KPF];
#pragma unroll
    for (int i = 0; i < KPF; ++i) kring[i] = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 32 * i);
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8_t kop = kring[ks % KPF];
      if (ks + KPF < 18) kring[ks % KPF] = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 32 * (ks + KPF));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; r += 4)
      *reinterpret_cast<f32x4_t*>(&xs[wave][lane][r]) = (f32x4_t){s[r], s[r + 1], s[r + 2], s[r + 3]};
    __builtin_amdgcn_s_waitcnt(0xc07f);  // exchange written (lgkmcnt(0)); loads stay in flight
    wg_barrier();
    {
      f32x4_t part[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) part[r] = *reinterpret_cast<const f32x4_t*>(&xs[wave ^ 1][lane][4 * r]);
      // the same sum in both waves of the pair: a + b == b + a exactly
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = hf == 0 ? s[r] + part[r >> 2][r & 3] : part[r >> 2][r & 3] + s[r];
    }
    // tile t + 2 goes into the buffer of tile t - 1 (released by the barrier
    // at the top of this step); issued after the exchange reads
    if (t + 2 < ntile) prefetch(t + 2, lds[(cur + 2) % NBUF]);
    // ---- softmax: lane = head, registers = keys 8 (r/4) + 4 half + r%4 ----
    const int valid = t < ns ? sn - t * TK : x_last - (t0 + (t - ns) * TK) + 1;
    if (valid < TK) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[r] = (8 * (r >> 2) + 4 * half + (r & 3)) < valid ? s[r] : kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int r = 0; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = with_upper_half_max(tmax) * a.sl;
    if (__any(tmax > m_ref + kLazy)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 8; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float nm = -m_ref;
    u32x4_t pw[2];
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const uint32_t w = pk_bf16(fast_exp2(fmaf(s[r], a.sl, nm)), fast_exp2(fmaf(s[r + 1], a.sl, nm)));
      pw[r >> 3][(r & 7) >> 1] = w;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                              __builtin_bit_cast(bf16x2_t, one2), l_run, false);
    }
    // ---- this wave's half of O^T += V^T P^T (V = first 512 key columns) ----
    {
      auto vread = [&](int i) __attribute__((always_inline)) {
        const int off = vrow_off + 16 * (i >> 3) * RB + 64 * (i & 7);
        const bf16x4_t lo = lds_read_tr(kl, off);
        const bf16x4_t hi = lds_read_tr(kl, off + 8 * RB);
        return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      };
      bf16x8_t vring[VPF];
#pragma unroll
      for (int i = 0; i < VPF; ++i) vring[i] = vread(i);
#pragma unroll
      for (int i = 0; i < 16; ++i) {  // i = 8 ks + db
        const bf16x8_t vop = vring[i % VPF];
        if (i + VPF < 16) vring[i % VPF] = vread(i + VPF);
        const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw[i >> 3]);
        oacc[i & 7] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[i & 7], 0, 0, 0);
      }
    }
  };
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  if (ntile > 0) prefetch(0, lds[0]);
  if (ntile > 1) prefetch(1, lds[1]);
  for (int t = 0; t < ntile; t += 3) {
    tile_step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntile) tile_step(std::integral_constant<int, 1>(), t + 1);
    if (t + 2 < ntile) tile_step(std::integral_constant<int, 2>(), t + 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS write in flight

  const float l_tot = with_upper_half_sum(l_run);
  const float inv = 1.f / l_tot;
  bf16_t* op = out + qo * DV + 256 * hf;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * db + 8 * qq + 4 * half;
      u32x2_t w;
      w.x = pk_bf16(oacc[db][4 * qq + 0] * inv, oacc[db][4 * qq + 1] * inv);
      w.y = pk_bf16(oacc[db][4 * qq + 2] * inv, oacc[db][4 * qq + 3] * inv);
      *reinterpret_cast<u32x2_t*>(op + d) = w;
    }
  if (lse && half == 0 && hf == 0)
    lse[(static_cast<int64_t>(b) * HQ + head) * a.L + row] = (m_ref + log2f(l_tot)) * kLn2;
}

bool prefill_mla_supported(const PrefillArgs& a, int32_t dtype) {
  return dtype == KSA_DTYPE_BF16 && a.v_is_k_prefix && a.dqk == DQK && a.dv == DV && a.hq == HQ && a.hkv == 1 &&
         a.mode == KSA_MODE_KSA && a.L * static_cast<int64_t>(GRB) + RB < (int64_t(1) << 31) &&
         static_cast<int64_t>(a.batch) * a.L < (int64_t(1) << 31);
}

hipError_t launch_prefill_mla(const PrefillArgs& p, const void* k, const void* q, void* out, float* lse,
                              hipStream_t s) {
  MlaPrefillArgs a;
  a.batch = p.batch;
  a.n = static_cast<int32_t>(p.n_text);
  a.L = static_cast<int32_t>(p.L);
  a.k = p.k;
  a.C = p.C;
  a.M = static_cast<int32_t>(p.n_text / p.k);
  fast_div(static_cast<uint32_t>(a.k), &a.divk_m, &a.divk_l);
  a.sl = p.scale * kLog2e;
  const int64_t blocks = static_cast<int64_t>(a.batch) * a.L;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_mla_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(512), 0, s, a,
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(q), static_cast<bf16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace ksa
