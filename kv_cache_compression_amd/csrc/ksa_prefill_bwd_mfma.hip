// Backward of the block-sparse KSA prefill for bf16, Dqk = Dv = 128, on
// gfx950 MFMA.
//
// The forward ("Kwai Summary Attention Technical Report", Sec. 2.3, Eq. 10)
// is softmax attention over the visible pairs of Eq. (3); the backward
// recomputes p_ij = exp(scale q_i.k_j - lse_i) from the forward's
// normaliser and, with delta_i = dout_i . out_i, forms
// dS_ij = p_ij (dout_i . v_j - delta_i).  Three kernels, no atomics:
//
// dq kernel (the forward's tiling: a workgroup owns 128 query rows of one
// kv head's group, 32 rows per wave, and walks the same two key runs in
// 64-key tiles):
//   S^T = K Q^T and dP^T = V dO^T on v_mfma_f32_32x32x16_bf16 (A = K / V
//   rows from LDS, B = Q / dO held in registers), dS^T in registers, then
//   dQ^T += K^T dS^T with K^T read through ds_read_b64_tr_b16.  Summary
//   query rows (k + 1 keys each) run in the first workgroups, one wave per
//   (sequence, kv head, summary).
//
// dkdv kernel (keys fixed, queries streamed): a workgroup owns 128 keys of
// one kv head, 32 per wave, held in registers as B operands; it walks the
// query tiles (64 rows of one query head) that see them, for every head of
// the group:
//   S = Q K^T and dP = dO V^T (A = Q / dO rows from LDS), P and dS in
//   registers, dV^T += dO^T P and dK^T += Q^T dS (A = dO^T / Q^T through
//   transposing LDS reads).
//   Text keys x (chunk c) are seen by text t_x .. t_{(c+C+1)k-1} (or the
//   token window) and by the summary s_c: one workgroup covers all of them
//   and writes dk, dv.  Summary keys s_j are seen by every text t_i with
//   floor(i/k) >= j + C + 1 (KSA only), a range that grows towards the start
//   of the sequence; it is cut into segments of equal length, one
//   workgroup per (128 summaries, segment), each writing fp32 partial sums.
// reduce kernel: one wave per (sequence, kv head, summary) adds the
// segments' partials and the summary query's own pair (s_j sees itself)
// and writes dk, dv of the summary rows.
#include <type_traits>

#include "ksa_internal.h"
#include "ksa_mfma_common.h"

namespace ksa {

namespace {

using namespace mfma;

constexpr int BN = 64;                      // keys (dq) or queries (dkdv) per tile
constexpr int TILE_BYTES = BN * ROW_BYTES;  // 16 KB
constexpr int KW = 128;                     // keys per dkdv workgroup
constexpr int SUM_R = 16;                   // key rows per pass of a summary query wave

struct BwdArgs {
  int32_t batch, n, L, k, C, hq, hkv, g, M;
  int32_t mode, W;
  uint32_t divk_m, divk_l;
  float sl;     // softmax scale * log2(e)
  float scale;  // softmax scale
  // dq kernel
  int32_t n_tiles, n_hg, n_sum_blocks;
  int32_t n_kv_blocks;  // dkdv workgroups, ahead of the dq ones in the grid
  // dkdv kernel
  int32_t n_sum_wg;  // summary-key workgroups (all sequences and heads)
  int32_t nt_sum;    // 128-summary tiles per head
  int32_t nu, qseg;  // query segments of the summary keys, their length
  int64_t part_stride_bh;  // floats of partials per (sequence, kv head)
};

__device__ __forceinline__ int32_t div_k(const BwdArgs& a, int32_t t) {
  return fast_div_apply(t, a.divk_m, a.divk_l);
}
__device__ __forceinline__ int32_t trow(const BwdArgs& a, int32_t t) { return t + div_k(a, t); }

// Number of 128-summary tiles whose first visible text query lies in
// segment u or before it (and before n): the tiles with a workgroup for u.
__device__ __forceinline__ int32_t seg_tiles(const BwdArgs& a, int32_t u) {
  const int32_t lim = min(a.n, (u + 1) * a.qseg) - 1;  // last query of the segment
  const int32_t top = div_k(a, lim) - a.C - 1;         // largest summary it sees
  if (top < 0) return 0;
  return min(a.nt_sum, top / KW + 1);
}

// ---------------------------------------------------------------------------
// Summary query rows: dq of s_j over its k + 1 keys.  Lane (hh, c) holds
// dims 8c .. 8c+7 of head hh of a group of four.
// ---------------------------------------------------------------------------
__device__ void summary_dq_wave(const BwdArgs& a, int64_t item, const bf16_t* __restrict__ q,
                                const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx,
                                const bf16_t* __restrict__ dout, const float* __restrict__ lse,
                                const float* __restrict__ delta, bf16_t* __restrict__ dq) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int hh = lane >> 4;
  const int j = static_cast<int>(item % a.M);
  const int kvh = static_cast<int>((item / a.M) % a.hkv);
  const int b = static_cast<int>(item / (static_cast<int64_t>(a.M) * a.hkv));
  const int r0 = j * (a.k + 1);
  const int nrows = a.k + 1;
  const int srow = r0 + a.k;
  const int64_t kvs = static_cast<int64_t>(a.hkv) * D;
  const bf16_t* kb = kx + static_cast<int64_t>(b) * a.L * kvs + kvh * D + 8 * c;
  const bf16_t* vb = vx + static_cast<int64_t>(b) * a.L * kvs + kvh * D + 8 * c;
  for (int hg = 0; hg < a.g; hg += 4) {
    const int hloc = hg + hh;
    const bool hval = hloc < a.g;
    const int h = kvh * a.g + (hval ? hloc : 0);
    const int64_t qo = (static_cast<int64_t>(b) * a.L + srow) * a.hq * D + static_cast<int64_t>(h) * D + 8 * c;
    const u32x4_t qw = *reinterpret_cast<const u32x4_t*>(q + qo);
    const u32x4_t gw = *reinterpret_cast<const u32x4_t*>(dout + qo);
    const int64_t so = (static_cast<int64_t>(b) * a.hq + h) * a.L + srow;
    const float lse2 = lse[so] * kLog2e;
    const float dl = delta[so];
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nrows; s0 += SUM_R) {
      u32x4_t kw[SUM_R], vw[SUM_R];
#pragma unroll
      for (int r = 0; r < SUM_R; ++r) {
        const int row = r0 + min(s0 + r, nrows - 1);
        kw[r] = *reinterpret_cast<const u32x4_t*>(kb + row * kvs);
        vw[r] = *reinterpret_cast<const u32x4_t*>(vb + row * kvs);
      }
#pragma unroll
      for (int r = 0; r < SUM_R; ++r) {
        float s = 0.f, dp = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw[e]), as_bf16x2(kw[r][e]), s, false);
          dp = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(gw[e]), as_bf16x2(vw[r][e]), dp, false);
        }
        s = sum16(s);
        dp = sum16(dp);
        const float p = fast_exp2(fmaf(s, a.sl, -lse2));
        const float ds = s0 + r < nrows ? p * (dp - dl) : 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += ds * bf_lo(kw[r][e]);
          acc[2 * e + 1] += ds * bf_hi(kw[r][e]);
        }
      }
    }
    if (hval) {
      u32x4_t w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = pk_bf16(acc[2 * e] * a.scale, acc[2 * e + 1] * a.scale);
      *reinterpret_cast<u32x4_t*>(dq + qo) = w;
    }
  }
}

}  // namespace

// ---------------------------------------------------------------------------
// dq of the text query rows.
// ---------------------------------------------------------------------------
template <int HPW>
__device__ __forceinline__ void bwd_dq_body(const BwdArgs& a, int blk, const bf16_t* __restrict__ q,
                                            const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx,
                                            const bf16_t* __restrict__ dout, const float* __restrict__ lse,
                                            const float* __restrict__ delta, bf16_t* __restrict__ dq, char* lds) {
  constexpr int PT = 32 * (4 / HPW);  // text positions per workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (blk < a.n_sum_blocks) {
    const int64_t item = static_cast<int64_t>(blk) * 4 + wave;
    if (item < static_cast<int64_t>(a.batch) * a.hkv * a.M)
      summary_dq_wave(a, item, q, kx, vx, dout, lse, delta, dq);
    return;
  }
  const int n_slots = a.batch * a.hkv * a.n_hg;
  const int bid = blk - a.n_sum_blocks;
  const int hslot = bid % n_slots;
  const int tile = a.n_tiles - 1 - bid / n_slots;  // longest first
  const int hg = hslot % a.n_hg;
  const int kvh = (hslot / a.n_hg) % a.hkv;
  const int b = hslot / (a.n_hg * a.hkv);
  const int h = kvh * a.g + hg * HPW + (wave % HPW);

  // Key runs of the workgroup (as in the forward).
  const int p0 = tile * PT;
  const int p_last = (p0 + PT < a.n ? p0 + PT : a.n) - 1;
  const int c_first = div_k(a, p0), c_last = div_k(a, p_last);
  const int sn = a.mode == KSA_MODE_KSA && c_last - a.C > 0 ? c_last - a.C : 0;
  const int t0 = a.mode == KSA_MODE_SWA ? (p0 - a.W + 1 > 0 ? p0 - a.W + 1 : 0)
                                        : (c_first - a.C > 0 ? (c_first - a.C) * a.k : 0);
  const int ns = (sn + BN - 1) / BN;
  const int n_total = ns + (p_last - t0 + BN) / BN;

  const int iw0 = p0 + 32 * (wave / HPW);
  const int iw1 = iw0 + 31 < a.n ? iw0 + 31 : a.n - 1;
  const bool wave_active = iw0 < a.n;
  const int qi = iw0 + (lane & 31);
  const bool q_valid = qi < a.n;
  const int ci = div_k(a, q_valid ? qi : 0);
  const int smax = q_valid ? ci - a.C - 1 : -1;
  auto text_lo = [&](int i, int c) {
    return a.mode == KSA_MODE_SWA ? (i - a.W + 1 > 0 ? i - a.W + 1 : 0) : (c - a.C > 0 ? (c - a.C) * a.k : 0);
  };
  const int tlo = q_valid ? text_lo(qi, ci) : 0x7fffffff;
  const int cw0 = div_k(a, wave_active ? iw0 : 0), cw1 = div_k(a, wave_active ? iw1 : 0);
  const int tlo_w1 = text_lo(wave_active ? iw1 : 0, cw1);

  // Q^T and dO^T as B operands: column = query (lane % 32), k-slots
  // d = 16 ks + 8 (lane / 32) + j.
  const int half = lane >> 5;
  const int qrow = trow(a, q_valid ? qi : 0);
  bf16x8_t qop[8], gop[8];
  {
    const int64_t o = (static_cast<int64_t>(b) * a.L + qrow) * a.hq * D + static_cast<int64_t>(h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qop[ks] = q_valid ? *reinterpret_cast<const bf16x8_t*>(q + o + 16 * ks) : bf16x8_t{};
      gop[ks] = q_valid ? *reinterpret_cast<const bf16x8_t*>(dout + o + 16 * ks) : bf16x8_t{};
    }
  }
  const int64_t so = (static_cast<int64_t>(b) * a.hq + h) * a.L + qrow;
  const float nlse2 = q_valid ? -lse[so] * kLog2e : 0.f;
  const float dl = q_valid ? delta[so] : 0.f;

  const int ld_chunk = tid & 15;
  const int ld_row = tid >> 4;
  const int kvs = a.hkv * D;
  const int RB = kvs * 2;
  const int64_t kv_base = static_cast<int64_t>(b) * a.L * kvs + kvh * D;
  const int kv_bytes = (a.L * kvs - kvh * D) * 2;
  const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(kx + kv_base), static_cast<short>(0), kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(vx + kv_base), static_cast<short>(0), kv_bytes, 0x00020000);
  const int chunk16 = 16 * (ld_chunk ^ lds_swz(ld_row));
  const int sum_step = (a.k + 1) * RB;
  const int s_c0 = ld_row * sum_step + a.k * RB + chunk16;
  char* const lds_k[2] = {lds, lds + TILE_BYTES};
  char* const lds_v[2] = {lds + 2 * TILE_BYTES, lds + 3 * TILE_BYTES};
  // rows past a run's end are masked or, past the sequence, read as zeros;
  // when k divides 64 a text tile starts 64 + 64/k rows after the previous
  int t_base[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    t_base[u] = static_cast<int>(__umul24(static_cast<uint32_t>(trow(a, t0 + ld_row + 16 * u)), RB)) + chunk16;
  const int t_step = (BN + BN / a.k) * RB;
  const bool k_div = (BN % a.k) == 0;
  auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, char* buf, int tt) {
    int vo[4];
    if (tt < ns) {
      const int sb = s_c0 + tt * BN * sum_step;
#pragma unroll
      for (int u = 0; u < 4; ++u) vo[u] = sb + 16 * u * sum_step;
    } else if (k_div) {
      const int d = (tt - ns) * t_step;
#pragma unroll
      for (int u = 0; u < 4; ++u) vo[u] = t_base[u] + d;
    } else {
      const int x0 = t0 + (tt - ns) * BN + ld_row;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        vo[u] = static_cast<int>(__umul24(static_cast<uint32_t>(trow(a, x0 + 16 * u)), RB)) + chunk16;
    }
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + (64 * wave + 256 * u) * 16), 16, vo[u], 0, 0, 0);
  };

  // Row-operand offsets (K / V rows lane % 32 (+32), chunk 2 ks + half) and
  // transposing offsets of K^T: in 16-lane group G, lane (4 rr + c4) points
  // at key row 16 ks + 8 rd + 4 (G / 2) + rr and d = 32 db + 16 (G % 2) + 4 c4.
  int koff0, toff[2][4];
  {
    const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
    koff0 = lds_off(lane & 31, half);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + 16 * (G & 1) + 4 * c4;
      const int row0 = 4 * (G >> 1) + rr;
      toff[0][db] = lds_off(row0, d >> 3) + 2 * (d & 7);
      toff[1][db] = lds_off(row0 + 8, d >> 3) + 2 * (d & 7);
    }
  }

  f32x16_t dqacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dqacc[db][r] = 0.f;

  auto iter = [&](auto cur_c, int tt) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    if (tt + 1 < n_total) {
      load_tile(rsrc_k, lds_k[cur ^ 1], tt + 1);
      load_tile(rsrc_v, lds_v[cur ^ 1], tt + 1);
    }
    const char* kl = lds_k[cur];
    const char* vl = lds_v[cur];
    // edge tiles: key of (kb2, r) = key0 + 32 kb2 + 8 (r / 4) + 4 half + r % 4
    const bool is_sum = tt < ns;
    const int key0 = is_sum ? tt * BN : t0 + (tt - ns) * BN;
    const bool full = is_sum ? key0 + BN - 1 <= cw0 - a.C - 1 : (key0 >= tlo_w1 && key0 + BN - 1 <= iw0);
    const int kbase = key0 + 4 * half;
    const int lo_r = (is_sum ? -1 : tlo) - kbase, hi_r = (is_sum ? smax : qi) - kbase;
    // the tile's two 32-key halves one after the other: S^T, dP^T and dS^T of
    // one half, then its dQ^T += K^T dS^T, so that one half's scores are live
    // at a time (the freed registers let the LDS operand reads run ahead)
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
      f32x16_t s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (koff0 ^ (ks << 5)) + 32 * ROW_BYTES * kb2;
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(kl + off);
        const bf16x8_t vop = *reinterpret_cast<const bf16x8_t*>(vl + off);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, gop[ks], dp, 0, 0, 0);
      }
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb2 + 8 * (r >> 2) + (r & 3);
          s[r] = (off >= lo_r && off <= hi_r) ? s[r] : kNegInf;
        }
      }
      // dS^T packed as the B operand of dQ^T += K^T dS^T (keys 16 ks + ...)
      u32x4_t pw[2];
#pragma unroll
      for (int r = 0; r < 16; r += 2) {
        const float p0 = fast_exp2(fmaf(s[r], a.sl, nlse2));
        const float p1 = fast_exp2(fmaf(s[r + 1], a.sl, nlse2));
        pw[r >> 3][(r & 7) >> 1] = pk_bf16(p0 * (dp[r] - dl), p1 * (dp[r + 1] - dl));
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * kb2 + kk;
        const bf16x8_t bop = __builtin_bit_cast(bf16x8_t, pw[kk]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4_t lo = lds_read_tr(kl, toff[0][db] + 16 * ROW_BYTES * ks);
          const bf16x4_t hi = lds_read_tr(kl, toff[1][db] + 16 * ROW_BYTES * ks);
          const bf16x8_t aop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          dqacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(aop, bop, dqacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  };

  if (n_total > 0) {
    load_tile(rsrc_k, lds_k[0], 0);
    load_tile(rsrc_v, lds_v[0], 0);
    __syncthreads();
  }
  for (int tt = 0; tt < n_total; tt += 2) {
    iter(std::integral_constant<int, 0>(), tt);
    if (tt + 1 < n_total) iter(std::integral_constant<int, 1>(), tt + 1);
  }
  if (!q_valid) return;
  bf16_t* op = dq + (static_cast<int64_t>(b) * a.L + qrow) * a.hq * D + static_cast<int64_t>(h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * db + 8 * qq + 4 * half;
      uint2 w;
      w.x = pk_bf16(dqacc[db][4 * qq + 0] * a.scale, dqacc[db][4 * qq + 1] * a.scale);
      w.y = pk_bf16(dqacc[db][4 * qq + 2] * a.scale, dqacc[db][4 * qq + 3] * a.scale);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
}

// ---------------------------------------------------------------------------
// dk, dv: keys fixed per workgroup, query tiles streamed.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void bwd_dkdv_body(const BwdArgs& a, int blk, const bf16_t* __restrict__ q,
                                              const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx,
                                              const bf16_t* __restrict__ dout, const float* __restrict__ lse,
                                              const float* __restrict__ delta, bf16_t* __restrict__ dk,
                                              bf16_t* __restrict__ dv, float* __restrict__ part, char* lds) {
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int half = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nbh = a.batch * a.hkv;
  const int bid = blk;
  const bool sum_keys = bid < a.n_sum_wg;
  int b, kvh, key0, u = 0, nkeys;
  // query runs: text positions [qt0, qt1) in 64-row tiles, then (text keys
  // only) summaries [cs0, cs1]
  int qt0, qt1, cs0 = 0, cs1 = -1;
  if (sum_keys) {
    const int slot = bid % nbh;
    int idx = bid / nbh;
    b = slot / a.hkv;
    kvh = slot % a.hkv;
    int jt = 0;
    for (u = 0; u < a.nu; ++u) {
      const int cnt = seg_tiles(a, u);
      if (idx < cnt) {
        jt = idx;
        break;
      }
      idx -= cnt;
    }
    key0 = jt * KW;
    nkeys = min(KW, a.M - key0);
    const int qa = (key0 + a.C + 1) * a.k;  // first text query that sees key0
    qt0 = max(qa, u * a.qseg) & ~(BN - 1);
    qt1 = min(a.n, (u + 1) * a.qseg);
  } else {
    const int t = bid - a.n_sum_wg;
    const int slot = t % nbh;
    b = slot / a.hkv;
    kvh = slot % a.hkv;
    key0 = (t / nbh) * KW;
    nkeys = min(KW, a.n - key0);
    const int xl = key0 + nkeys - 1;
    const int hi = a.mode == KSA_MODE_SWA ? xl + a.W - 1 : (div_k(a, xl) + a.C + 1) * a.k - 1;
    qt0 = key0;
    qt1 = min(a.n, hi + 1);
    cs0 = div_k(a, key0);
    cs1 = min(a.M - 1, div_k(a, xl));
  }
  // uniform over the workgroup: kept in scalar registers
  b = __builtin_amdgcn_readfirstlane(b);
  kvh = __builtin_amdgcn_readfirstlane(kvh);
  key0 = __builtin_amdgcn_readfirstlane(key0);
  u = __builtin_amdgcn_readfirstlane(u);
  nkeys = __builtin_amdgcn_readfirstlane(nkeys);
  qt0 = __builtin_amdgcn_readfirstlane(qt0);
  qt1 = __builtin_amdgcn_readfirstlane(qt1);
  cs0 = __builtin_amdgcn_readfirstlane(cs0);
  cs1 = __builtin_amdgcn_readfirstlane(cs1);
  const int ntq = (qt1 - qt0 + BN - 1) / BN;
  const int nts = cs1 >= cs0 ? (cs1 - cs0 + BN) / BN : 0;
  const int per_head = ntq + nts;
  const int n_total = per_head * a.g;

  // This wave's 32 keys; the lane's key is column lane % 32.
  const int kw0 = key0 + 32 * wave;
  const int key = kw0 + (lane & 31);
  const bool key_valid = key < key0 + nkeys;
  const int krow = sum_keys ? summary_row(key_valid ? key : key0, a.k) : trow(a, key_valid ? key : key0);
  bf16x8_t kop[8], vop[8];
  {
    const int64_t o = (static_cast<int64_t>(b) * a.L + krow) * a.hkv * D + static_cast<int64_t>(kvh) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      kop[ks] = *reinterpret_cast<const bf16x8_t*>(kx + o + 16 * ks);
      vop[ks] = *reinterpret_cast<const bf16x8_t*>(vx + o + 16 * ks);
    }
  }
  // Queries that see the lane's key, as an index range [lo, hi] of the text
  // queries or of the summary queries (sq):
  //   text key x, chunk c:  text x .. (c+C+1)k - 1 (or x + W - 1), summary c
  //   summary key j:        text (j+C+1)k .. n - 1
  // Formed per masked tile from an opaque copy of the lane: kept across the
  // loop, these per-lane bounds are spilled.
  auto key_bounds = [&](bool sq, int* lo, int* hi) {
    int ln = lane;
    asm volatile("" : "+v"(ln));
    const int kl = kw0 + (ln & 31);
    const bool kv = kl < key0 + nkeys;
    const int kc = div_k(a, kv ? kl : key0);
    if (sum_keys) {
      *lo = (kl + a.C + 1) * a.k;
      *hi = kv ? qt1 - 1 : -1;
    } else if (sq) {
      *lo = kc;
      *hi = kv && kc <= cs1 ? kc : -1;
    } else {
      *lo = kl;
      *hi = !kv ? -1 : min(qt1 - 1, a.mode == KSA_MODE_SWA ? kl + a.W - 1 : (kc + a.C + 1) * a.k - 1);
    }
  };
  // wave-uniform: the smallest key's upper bound, the largest key
  const int kwl = min(kw0 + 31, key0 + nkeys - 1);
  const int whi_min = sum_keys ? 0 : a.mode == KSA_MODE_SWA ? kw0 + a.W - 1 : (div_k(a, kw0) + a.C + 1) * a.k - 1;

  // Q / dO tiles: 64 rows of one query head, rows gathered by the Eq. 1 map.
  const int qhs = a.hq * D;  // elements per augmented row
  const int QRB = qhs * 2;
  char* const lds_q[2] = {lds, lds + TILE_BYTES};
  char* const lds_g[2] = {lds + 2 * TILE_BYTES, lds + 3 * TILE_BYTES};
  float(*const lds_st)[2][BN] = reinterpret_cast<float(*)[2][BN]>(lds + 4 * TILE_BYTES);  // [buffer][lse, delta][row]
  const int64_t qbase = static_cast<int64_t>(b) * a.L * qhs;
  // iteration it -> (head, kind, first query index of the tile)
  auto tile_of = [&](int it, int* h, bool* sq, int* i0) {
    const int hh = it / per_head;
    const int r = it - hh * per_head;
    *h = kvh * a.g + hh;
    *sq = r >= ntq;
    *i0 = *sq ? cs0 + (r - ntq) * BN : qt0 + r * BN;
  };
  auto row_of = [&](bool sq, int idx) { return sq ? summary_row(idx, a.k) : trow(a, idx); };
  auto load_tile = [&](char* qb, char* gb, int it, float* st_buf) {
    // the thread's row and chunk are formed here, each time: kept across the
    // loop they are spilled, and a spill reload waits for every tile copy in
    // flight, the next tile's included
    int t_ = tid;
    asm volatile("" : "+v"(t_));
    const int lrow = t_ >> 4;
    const int lchunk16 = 16 * ((t_ & 15) ^ lds_swz(lrow));
    int h, i0;
    bool sq;
    tile_of(it, &h, &sq, &i0);
    const int last = sq ? cs1 : qt1 - 1;
    const int hoff = h * D;
    const __amdgpu_buffer_rsrc_t rq = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(q + qbase + hoff), static_cast<short>(0), (a.L * qhs - hoff) * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rg = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(dout + qbase + hoff), static_cast<short>(0), (a.L * qhs - hoff) * 2, 0x00020000);
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const int idx = min(i0 + lrow + 16 * uu, last);
      const int vo = static_cast<int>(__umul24(static_cast<uint32_t>(row_of(sq, idx)), QRB)) + lchunk16;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rq, (__attribute__((address_space(3))) void*)(qb + (64 * wave + 256 * uu) * 16), 16, vo, 0, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rg, (__attribute__((address_space(3))) void*)(gb + (64 * wave + 256 * uu) * 16), 16, vo, 0, 0, 0);
    }
    // statistics of the 64 rows straight into LDS, like the tiles: wave 0
    // the natural-log normaliser, wave 1 delta (no register holds them
    // across the loop, and the tile's barrier covers them)
    if (wave < 2) {
      const int64_t head_row0 = (static_cast<int64_t>(b) * a.hq + h) * a.L;
      const int vo = row_of(sq, min(i0 + (t_ & (BN - 1)), last)) * 4;
      if (wave == 0) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(lse + head_row0), static_cast<short>(0), a.L * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(st_buf), 4, vo, 0,
                                                 0, 0);
      } else {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(delta + head_row0), static_cast<short>(0), a.L * 4, 0x00020000);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (__attribute__((address_space(3))) void*)(st_buf + BN), 4, vo,
                                                 0, 0, 0);
      }
    }
  };

  // LDS offsets: row operands (row lane % 32 (+32), chunk 2 ks + half);
  // transposing reads (query rows 16 ks + 8 rd + 4 (G / 2) + rr).
  int qoff0, toff[2][4];
  {
    const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
    qoff0 = lds_off(lane & 31, half);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + 16 * (G & 1) + 4 * c4;
      const int row0 = 4 * (G >> 1) + rr;
      toff[0][db] = lds_off(row0, d >> 3) + 2 * (d & 7);
      toff[1][db] = lds_off(row0 + 8, d >> 3) + 2 * (d & 7);
    }
  }

  f32x16_t dkacc[4], dvacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) dkacc[db][r] = dvacc[db][r] = 0.f;

  auto iter = [&](auto cur_c, int it) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    if (it + 1 < n_total) load_tile(lds_q[cur ^ 1], lds_g[cur ^ 1], it + 1, &lds_st[cur ^ 1][0][0]);
    int h, i0;
    bool sq;
    tile_of(it, &h, &sq, &i0);
    (void)h;
    const char* ql = lds_q[cur];
    const char* gl = lds_g[cur];
    // this lane's rows of the statistics: the lane part comes from an opaque
    // copy, so the reads take one address register and immediate offsets
    // (left visible, their addresses are formed ahead and spilled)
    int hb = 4 * half;
    asm volatile("" : "+v"(hb));
    const float* st = &lds_st[cur][0][0] + hb;
    // full: every row of the tile is a query of the run and sees every key
    // of the wave (the first row the largest key, the last row the smallest)
    bool full;
    if (sq)
      full = false;
    else if (sum_keys)
      full = i0 + BN - 1 < qt1 && kwl <= div_k(a, i0) - a.C - 1;
    else
      full = i0 + BN - 1 < qt1 && i0 >= kwl && i0 + BN - 1 <= whi_min;
    const int base = i0 + 4 * half;
    int lo = 0, hi = -1;
    if (!full) {
      key_bounds(sq, &lo, &hi);
      lo -= base;
      hi -= base;
    }
    // two halves of 32 query rows, one after the other (keeps the live
    // registers within two waves per SIMD)
#pragma unroll
    for (int blk = 0; blk < 2; ++blk) {
      // S first, turned into P (kept in fp32 only until packed to bf16),
      // then dP: the two score blocks are never live together
      f32x16_t s;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (qoff0 ^ (ks << 5)) + 32 * ROW_BYTES * blk;
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(ql + off), kop[ks], s, 0, 0,
                                                    0);
      }
      // visibility of (query row 32 blk + 8 (r / 4) + 4 half + r % 4, lane's key)
      if (!full) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * blk + 8 * (r >> 2) + (r & 3);
          s[r] = (off >= lo && off <= hi) ? s[r] : kNegInf;
        }
      }
      float p[16];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t l4 = *reinterpret_cast<const f32x4_t*>(st + 32 * blk + 8 * r4);
#pragma unroll
        for (int e = 0; e < 4; ++e) p[4 * r4 + e] = fast_exp2(s[4 * r4 + e] * a.sl - l4[e] * kLog2e);
      }
      f32x16_t dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) dp[r] = 0.f;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const int off = (qoff0 ^ (ks << 5)) + 32 * ROW_BYTES * blk;
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(*reinterpret_cast<const bf16x8_t*>(gl + off), vop[ks], dp, 0, 0,
                                                     0);
      }
      u32x4_t pw[2], dw[2];
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4_t d4 = *reinterpret_cast<const f32x4_t*>(st + BN + 32 * blk + 8 * r4);
        float ds[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) ds[e] = p[4 * r4 + e] * (dp[4 * r4 + e] - d4[e]);
        // query k-slots of step 2 blk + r4 / 2: rows 16 ks + 4 half + {0..3}, +8
        const int kk = r4 >> 1;
        const int w0 = 2 * (r4 & 1);
        pw[kk][w0] = pk_bf16(p[4 * r4 + 0], p[4 * r4 + 1]);
        pw[kk][w0 + 1] = pk_bf16(p[4 * r4 + 2], p[4 * r4 + 3]);
        dw[kk][w0] = pk_bf16(ds[0], ds[1]);
        dw[kk][w0 + 1] = pk_bf16(ds[2], ds[3]);
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        const int ks = 2 * blk + kk;
        const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw[kk]);
        const bf16x8_t dop = __builtin_bit_cast(bf16x8_t, dw[kk]);
#pragma unroll
        for (int db = 0; db < 4; ++db) {
          const bf16x4_t glo = lds_read_tr(gl, toff[0][db] + 16 * ROW_BYTES * ks);
          const bf16x4_t ghi = lds_read_tr(gl, toff[1][db] + 16 * ROW_BYTES * ks);
          dvacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_shufflevector(glo, ghi, 0, 1, 2, 3, 4, 5, 6, 7), pop, dvacc[db], 0, 0, 0);
          const bf16x4_t qlo = lds_read_tr(ql, toff[0][db] + 16 * ROW_BYTES * ks);
          const bf16x4_t qhi = lds_read_tr(ql, toff[1][db] + 16 * ROW_BYTES * ks);
          dkacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              __builtin_shufflevector(qlo, qhi, 0, 1, 2, 3, 4, 5, 6, 7), dop, dkacc[db], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  };

  if (n_total > 0) {
    load_tile(lds_q[0], lds_g[0], 0, &lds_st[0][0][0]);
    __syncthreads();
  }
  for (int it = 0; it < n_total; it += 2) {
    iter(std::integral_constant<int, 0>(), it);
    if (it + 1 < n_total) iter(std::integral_constant<int, 1>(), it + 1);
  }
  if (!key_valid) return;
  // dV^T / dK^T: lane's key column, d = 32 db + 8 qq + 4 half + e
  if (sum_keys) {
    float* pp = part + (static_cast<int64_t>(b) * a.hkv + kvh) * a.part_stride_bh +
                (static_cast<int64_t>(u) * a.nt_sum * KW + key) * 256;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * half;
        f32x4_t wk, wv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wk[e] = dkacc[db][4 * qq + e] * a.scale;
          wv[e] = dvacc[db][4 * qq + e];
        }
        *reinterpret_cast<f32x4_t*>(pp + d) = wk;
        *reinterpret_cast<f32x4_t*>(pp + 128 + d) = wv;
      }
  } else {
    const int64_t o = (static_cast<int64_t>(b) * a.L + krow) * a.hkv * D + static_cast<int64_t>(kvh) * D;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int qq = 0; qq < 4; ++qq) {
        const int d = 32 * db + 8 * qq + 4 * half;
        uint2 wk, wv;
        wk.x = pk_bf16(dkacc[db][4 * qq + 0] * a.scale, dkacc[db][4 * qq + 1] * a.scale);
        wk.y = pk_bf16(dkacc[db][4 * qq + 2] * a.scale, dkacc[db][4 * qq + 3] * a.scale);
        wv.x = pk_bf16(dvacc[db][4 * qq + 0], dvacc[db][4 * qq + 1]);
        wv.y = pk_bf16(dvacc[db][4 * qq + 2], dvacc[db][4 * qq + 3]);
        *reinterpret_cast<uint2*>(dk + o + d) = wk;
        *reinterpret_cast<uint2*>(dv + o + d) = wv;
      }
  }
}

// ---------------------------------------------------------------------------
// One launch for both: the dkdv workgroups (the long summary-key ones first)
// take the first block indices and the dq workgroups follow, so dq work fills
// the machine while the last dkdv workgroups finish.  The two share one LDS
// buffer (each uses four 16 KB tiles; dkdv adds its row statistics).
// ---------------------------------------------------------------------------
constexpr int BWD_LDS_BYTES = 4 * TILE_BYTES + 2 * 2 * BN * static_cast<int>(sizeof(float));

template <int HPW>
__global__ void __launch_bounds__(256, 2) bwd_dkdv_dq_kernel(
    BwdArgs a, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx,
    const bf16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    bf16_t* __restrict__ dq, bf16_t* __restrict__ dk, bf16_t* __restrict__ dv, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) char lds[BWD_LDS_BYTES];
  const int bid = blockIdx.x;
  if (bid < a.n_kv_blocks)
    bwd_dkdv_body(a, bid, q, kx, vx, dout, lse, delta, dk, dv, part, lds);
  else
    bwd_dq_body<HPW>(a, bid - a.n_kv_blocks, q, kx, vx, dout, lse, delta, dq, lds);
}

// ---------------------------------------------------------------------------
// Summary keys: partials of the segments plus the summary's own query.
// One wave per (sequence, kv head, summary); lanes 0..31 own dk dims
// 4 l .. 4 l + 3, lanes 32..63 own dv dims 4 (l - 32) ...
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) bwd_sum_keys_kernel(BwdArgs a, const bf16_t* __restrict__ q,
                                                           const bf16_t* __restrict__ kx,
                                                           const bf16_t* __restrict__ vx,
                                                           const bf16_t* __restrict__ dout,
                                                           const float* __restrict__ lse,
                                                           const float* __restrict__ delta,
                                                           const float* __restrict__ part,
                                                           bf16_t* __restrict__ dk, bf16_t* __restrict__ dv) {
  const int lane = threadIdx.x & 63;
  const int64_t item = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (item >= static_cast<int64_t>(a.batch) * a.hkv * a.M) return;
  const int j = static_cast<int>(item % a.M);
  const int kvh = static_cast<int>((item / a.M) % a.hkv);
  const int b = static_cast<int>(item / (static_cast<int64_t>(a.M) * a.hkv));
  const bool is_v = lane >= 32;
  const int d0 = 4 * (lane & 31);
  f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
  if (a.mode == KSA_MODE_KSA) {
    const int qa = ((j / KW) * KW + a.C + 1) * a.k;  // first query of the tile's workgroups
    if (qa < a.n) {
      const float* pp = part + (static_cast<int64_t>(b) * a.hkv + kvh) * a.part_stride_bh +
                        static_cast<int64_t>(j) * 256 + (is_v ? 128 : 0) + d0;
      for (int u = qa / a.qseg; u < a.nu; ++u) {
        const f32x4_t w = *reinterpret_cast<const f32x4_t*>(pp + static_cast<int64_t>(u) * a.nt_sum * KW * 256);
        acc += w;
      }
    }
  }
  // the summary query s_j sees its own key
  const int srow = summary_row(j, a.k);
  const int64_t kvo = (static_cast<int64_t>(b) * a.L + srow) * a.hkv * D + static_cast<int64_t>(kvh) * D + d0;
  const uint2 kw = *reinterpret_cast<const uint2*>(kx + kvo);
  const uint2 vw = *reinterpret_cast<const uint2*>(vx + kvo);
  for (int hh = 0; hh < a.g; ++hh) {
    const int h = kvh * a.g + hh;
    const int64_t qo = (static_cast<int64_t>(b) * a.L + srow) * a.hq * D + static_cast<int64_t>(h) * D + d0;
    const uint2 qw = *reinterpret_cast<const uint2*>(q + qo);
    const uint2 gw = *reinterpret_cast<const uint2*>(dout + qo);
    // lanes 0..31: q . k; lanes 32..63: dout . v (each over all 128 dims)
    const uint2 xa = is_v ? gw : qw, xb = is_v ? vw : kw;
    float part_dot = bf_lo(xa.x) * bf_lo(xb.x) + bf_hi(xa.x) * bf_hi(xb.x) + bf_lo(xa.y) * bf_lo(xb.y) +
                     bf_hi(xa.y) * bf_hi(xb.y);
    part_dot = with_row_pair_sum(sum16(part_dot));
    // v_permlane32_swap of a value with itself yields the lower half's copy
    // in the first result and the upper half's in the second, in every lane
    const auto both = __builtin_amdgcn_permlane32_swap(__float_as_uint(part_dot), __float_as_uint(part_dot), false, false);
    const float s = __uint_as_float(both[0]);
    const float dpv = __uint_as_float(both[1]);
    const int64_t so = (static_cast<int64_t>(b) * a.hq + h) * a.L + srow;
    const float p = fast_exp2(s * a.sl - lse[so] * kLog2e);
    const float ds = p * (dpv - delta[so]);
    const float f = is_v ? p : ds * a.scale;
    const uint2 src = is_v ? gw : qw;
    acc[0] += f * bf_lo(src.x);
    acc[1] += f * bf_hi(src.x);
    acc[2] += f * bf_lo(src.y);
    acc[3] += f * bf_hi(src.y);
  }
  uint2 w;
  w.x = pk_bf16(acc[0], acc[1]);
  w.y = pk_bf16(acc[2], acc[3]);
  *reinterpret_cast<uint2*>((is_v ? dv : dk) + kvo) = w;
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
namespace {

BwdArgs make_args(const PrefillArgs& p) {
  BwdArgs a{};
  a.batch = p.batch;
  a.n = static_cast<int32_t>(p.n_text);
  a.L = static_cast<int32_t>(p.L);
  a.k = p.k;
  a.C = p.C;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.g = p.hq / p.hkv;
  a.M = static_cast<int32_t>(p.n_text / p.k);
  a.mode = p.mode;
  a.W = static_cast<int32_t>(p.window_tokens);
  fast_div(static_cast<uint32_t>(a.k), &a.divk_m, &a.divk_l);
  a.sl = p.scale * kLog2e;
  a.scale = p.scale;
  a.nt_sum = (a.M + KW - 1) / KW;
  // segments of at least 2048 queries, at most 16 per sequence
  const int64_t seg = ((p.n_text + 15) / 16 + BN - 1) / BN * BN;
  a.qseg = static_cast<int32_t>(seg > 2048 ? seg : 2048);
  a.nu = static_cast<int32_t>((p.n_text + a.qseg - 1) / a.qseg);
  a.part_stride_bh = static_cast<int64_t>(a.nu) * a.nt_sum * KW * 256;
  return a;
}

// Host twin of seg_tiles.
int32_t seg_tiles_host(const BwdArgs& a, int32_t u) {
  const int32_t lim = std::min(a.n, (u + 1) * a.qseg) - 1;
  const int32_t top = lim / a.k - a.C - 1;
  if (top < 0) return 0;
  return std::min(a.nt_sum, top / KW + 1);
}

}  // namespace

bool prefill_bwd_mfma_supported(const PrefillArgs& a, int32_t dtype) {
  const int g = a.hq / a.hkv;
  // 32-bit byte offsets inside the kernels
  const bool fits = a.L < (int64_t(1) << 24) && a.L * a.hkv * D * 2 < (int64_t(1) << 31) &&
                    a.L * static_cast<int64_t>(a.hq) * D * 2 < (int64_t(1) << 31) &&
                    static_cast<int64_t>(a.batch) * a.hkv * g * ((a.n_text + 31) / 32) < (int64_t(1) << 31);
  return dtype == KSA_DTYPE_BF16 && a.dqk == D && a.dv == D && !a.v_is_k_prefix && fits &&
         (g == 1 || g == 2 || g % 4 == 0);
}

size_t prefill_bwd_mfma_partial_bytes(const PrefillArgs& p) {
  const BwdArgs a = make_args(p);
  if (p.mode != KSA_MODE_KSA) return 0;
  return static_cast<size_t>(a.batch) * a.hkv * a.part_stride_bh * sizeof(float);
}

template <int HPW>
static hipError_t launch_main(BwdArgs a, const void* q, const void* k, const void* v, const void* dout,
                              const float* lse, const float* delta, float* part, void* dq, void* dk, void* dv,
                              hipStream_t s) {
  constexpr int PT = 32 * (4 / HPW);
  // dq: summary query waves, then text tiles
  a.n_hg = a.g / HPW;
  a.n_tiles = (a.n + PT - 1) / PT;
  const int64_t n_slots = static_cast<int64_t>(a.batch) * a.hkv * a.n_hg;
  const int64_t sum_items = static_cast<int64_t>(a.batch) * a.hkv * a.M;
  a.n_sum_blocks = static_cast<int32_t>((sum_items + 3) / 4);
  const int64_t dq_blocks = n_slots * a.n_tiles + a.n_sum_blocks;
  // dkdv: summary-key workgroups per query segment, then text keys
  const int64_t nbh = static_cast<int64_t>(a.batch) * a.hkv;
  int64_t per_head = 0;
  if (a.mode == KSA_MODE_KSA)
    for (int u = 0; u < a.nu; ++u) per_head += seg_tiles_host(a, u);
  a.n_sum_wg = static_cast<int32_t>(per_head * nbh);
  const int64_t text_wg = nbh * ((a.n + KW - 1) / KW);
  a.n_kv_blocks = static_cast<int32_t>(a.n_sum_wg + text_wg);
  const int64_t blocks = a.n_kv_blocks + dq_blocks;
  if (blocks == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_dkdv_dq_kernel<HPW>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, a,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                     static_cast<const bf16_t*>(dout), lse, delta, static_cast<bf16_t*>(dq),
                     static_cast<bf16_t*>(dk), static_cast<bf16_t*>(dv), part);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t items = nbh * a.M;
  if (items == 0) return hipSuccess;
  hipLaunchKernelGGL(bwd_sum_keys_kernel, dim3(static_cast<uint32_t>((items + 3) / 4)), dim3(256), 0, s, a,
                     static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                     static_cast<const bf16_t*>(dout), lse, delta, part, static_cast<bf16_t*>(dk),
                     static_cast<bf16_t*>(dv));
  return hipGetLastError();
}

hipError_t launch_prefill_bwd_mfma(const PrefillArgs& p, const void* q, const void* k, const void* v,
                                   const void* dout, const float* lse, const float* delta, float* part,
                                   void* dq, void* dk, void* dv, hipStream_t s) {
  const BwdArgs a = make_args(p);
  if (a.g == 1) return launch_main<1>(a, q, k, v, dout, lse, delta, part, dq, dk, dv, s);
  if (a.g == 2) return launch_main<2>(a, q, k, v, dout, lse, delta, part, dq, dk, dv, s);
  return launch_main<4>(a, q, k, v, dout, lse, delta, part, dq, dk, dv, s);
}

}  // namespace ksa
