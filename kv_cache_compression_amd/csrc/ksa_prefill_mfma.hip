// Block-sparse KSA prefill for bf16, Dqk = Dv = 128, on gfx950 MFMA.
//
// "Kwai Summary Attention Technical Report", Sec. 2.3: the prefill kernel
// splits Q/K/V into fixed-size blocks and loads only block pairs that hold
// visible entries; the O(L^2) mask is never built.  The visible set of text
// token t_i (chunk c = floor(i/k)) is, by Eq. (3), the summaries
// s_0 .. s_{c-C-1} and the text t_{(c-C)k} .. t_i.  For a block of
// consecutive text queries the visible keys are therefore two runs, each
// contiguous in its own index space: a summary run [0, c_last - C) and a
// text run [(c_first - C) k, i_last].  The kernel walks those runs in 64-key
// tiles; only tiles on a run's edge need an element mask, computed from
// integer compares on chunk indices.  A summary query s_j reads only its own
// chunk's k text tokens and itself (Sec. 2.2.1), i.e. the k+1 consecutive
// augmented rows j(k+1) .. j(k+1)+k; those rows are handled by the first
// workgroups of the same launch (a wave per four summaries and kv head
// when k <= 8, else per summary).
//
// Text workgroups (4 wavefronts, 256 threads):
//   - a workgroup owns one kv head and HPW of its query heads over PT
//     consecutive text positions (HPW * PT = 128 query rows); every wave owns
//     32 query rows of one head, so each K/V tile staged in LDS feeds 4 waves;
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q in
//     registers): each lane owns one query row, so the softmax statistics
//     stay in-lane apart from one swap with the lane 32 away;
//   - O^T += V^T P^T on the same MFMA: P goes from the score registers into
//     the B operand; V^T comes from the row-major V tile through
//     ds_read_b64_tr_b16 (4x16 bf16 transposes within each 16 lanes);
//   - software pipeline over tiles: while the MFMAs of S for tile t+1 run,
//     the VALU turns the scores of tile t into P; while the MFMAs of P V for
//     tile t run, the VALU finishes P, masks tile t+1 and takes its maximum;
//   - the running maximum is only moved (and O rescaled) when a tile's
//     maximum exceeds it by more than 2^8, which keeps every exponent <= 8;
//     that decision is taken one tile ahead, so no branch splits the
//     MFMA/VALU interleave;
//   - K/V tiles go straight from global memory into double-buffered LDS
//     (buffer_load ... lds, swizzle applied on the global side), one tile
//     ahead, through buffer resources with 32-bit row offsets: one barrier
//     per tile, no staging registers;
//   - workgroups run longest-first (later queries see more summaries) and,
//     when the head count allows, all workgroups of one (sequence, kv head)
//     sit on one XCD so that its K/V stay in that XCD's L2.
#include <cmath>
#include <type_traits>

#include "ksa_internal.h"
#include "ksa_mfma_common.h"

namespace ksa {

namespace {

using namespace mfma;

constexpr int BN = 64;            // keys per tile
constexpr int TILE_BYTES = BN * ROW_BYTES;
constexpr float kLazyRescale = 8.f;  // log2 units
// Byte range of the query-row buffer resource: above every in-range offset
// (fewer than 64 augmented rows of Hq heads after the wave's first row).
constexpr int kQRange = 1 << 30;

struct MfmaArgs {
  int32_t batch, n, L, k, C, hq, hkv, g, M;
  int32_t n_tiles, n_hg, xcd_map, n_text_blocks, n_sum_blocks;
  uint32_t divk_m, divk_l;  // floor(t / k) = (umulhi(t, m) + t) >> l for t < 2^31
  float sl;                 // softmax scale * log2(e)
  int32_t mode;             // KSA_MODE_*: summaries and text window of text queries
  int32_t W;                // token window of KSA_MODE_SWA
  // Query rotary embedding applied on load (the QROT kernels): frequency f
  // turns by theta^(-2f/128) radians per position; rope_fq[f] is that rate
  // in revolutions as a 64-bit binary fraction (rate * 2^64, rounded).
  uint64_t rope_fq[64];
};

// sin and cos of position pos at rate fq (a 64-bit fraction of a
// revolution per position).  pos * fq modulo 2^64 is the angle's fraction
// of a turn, exact in integers; its top 32 bits, read as a signed number,
// are the angle in [-1/2, 1/2) revolutions to 2^-32, which v_sin_f32 /
// v_cos_f32 take directly (their argument is in revolutions).  The rate's
// rounding adds at most pos * 2^-65 revolutions.
__device__ __forceinline__ void rope_sincos(uint32_t pos, uint64_t fq, float* sn, float* cs) {
  const uint32_t lo = static_cast<uint32_t>(fq), hi = static_cast<uint32_t>(fq >> 32);
  const uint32_t top = __umulhi(lo, pos) + hi * pos;
  const float r = static_cast<float>(static_cast<int32_t>(top)) * 0x1p-32f;
  *sn = __builtin_amdgcn_sinf(r);
  *cs = __builtin_amdgcn_cosf(r);
}

// Sec. 2.2.1 half-split rotation of one (x, partner) pair of bf16x2 words:
// lower-half dims get x cos - y sin, upper-half dims x cos + y sin, in fp32,
// rounded to bf16 as a separate rotation pass would store them.
__device__ __forceinline__ uint32_t rope_pair(uint32_t x, uint32_t y, bool upper, float sn0, float cs0, float sn1,
                                              float cs1) {
  const float s0 = upper ? sn0 : -sn0, s1 = upper ? sn1 : -sn1;
  return pk_bf16(bf_lo(x) * cs0 + bf_lo(y) * s0, bf_hi(x) * cs1 + bf_hi(y) * s1);
}

__device__ __forceinline__ int32_t div_k(const MfmaArgs& a, int32_t t) {
  return fast_div_apply(t, a.divk_m, a.divk_l);
}
__device__ __forceinline__ int32_t trow(const MfmaArgs& a, int32_t t) { return t + div_k(a, t); }

// Summary query rows: one wave per (sequence, kv head, summary j) attends
// the group's query heads to the k + 1 rows j(k+1) .. j(k+1)+k.  Lane
// (hh, c) = (lane / 16, lane % 16) holds dims 8c .. 8c+7 of head hh of a
// group of four; the key/value rows of a pass are all loaded before any is
// used, so a pass costs one memory round trip.  SUM_R = 16 key rows per
// pass; rows past the chunk are masked.  This path serves k > 8; for
// k <= 8, summary_rows_wave_multi below.
template <int SUM_R, bool QROT>
__device__ void summary_rows_wave(const MfmaArgs& a, int64_t item, const bf16_t* __restrict__ q,
                                  const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx,
                                  bf16_t* __restrict__ out, float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int hh = lane >> 4;
  const int j = static_cast<int>(item % a.M);
  const int kvh = static_cast<int>((item / a.M) % a.hkv);
  const int b = static_cast<int>(item / (static_cast<int64_t>(a.M) * a.hkv));
  const int r0 = j * (a.k + 1);
  const int nrows = a.k + 1;
  const int srow_a = r0 + a.k;  // the summary's own augmented row
  const int64_t kvs = static_cast<int64_t>(a.hkv) * D;
  const bf16_t* kb = kx + static_cast<int64_t>(b) * a.L * kvs + kvh * D + 8 * c;
  const bf16_t* vb = vx + static_cast<int64_t>(b) * a.L * kvs + kvh * D + 8 * c;
  for (int hg = 0; hg < a.g; hg += 4) {
    const int hloc = hg + hh;
    const bool hval = hloc < a.g;
    const int h = kvh * a.g + (hval ? hloc : 0);
    u32x4_t qw = *reinterpret_cast<const u32x4_t*>(
        q + (static_cast<int64_t>(b) * a.L + srow_a) * a.hq * D + static_cast<int64_t>(h) * D + 8 * c);
    if constexpr (QROT) {
      // position of s_j: its chunk's last text token; dims 8c .. 8c+7 pair
      // with dims 8c +- 64, which lane c ^ 8 of the same 16 holds.  The
      // wave needs the 64 angles f = 0..63 at one position: lane l forms
      // angle l and each lane gathers its eight (f = 8 (c % 8) + e) with
      // ds_bpermute.
      float sn_l, cs_l;
      rope_sincos(static_cast<uint32_t>((j + 1) * a.k - 1), a.rope_fq[lane], &sn_l, &cs_l);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t y = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(qw[w]), 0x128, 0xF, 0xF, false));  // row_ror:8
        const int f0 = 4 * (8 * (c & 7) + 2 * w);  // byte address of lane f
        const float sn0 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0, __float_as_int(sn_l)));
        const float cs0 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0, __float_as_int(cs_l)));
        const float sn1 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0 + 4, __float_as_int(sn_l)));
        const float cs1 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0 + 4, __float_as_int(cs_l)));
        qw[w] = rope_pair(qw[w], y, c >= 8, sn0, cs0, sn1, cs1);
      }
    }
    float m = kNegInf, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nrows; s0 += SUM_R) {
      u32x4_t kw[SUM_R], vw[SUM_R];
#pragma unroll
      for (int r = 0; r < SUM_R; ++r) {
        const int row = r0 + min(s0 + r, nrows - 1);
        kw[r] = *reinterpret_cast<const u32x4_t*>(kb + row * kvs);
        vw[r] = *reinterpret_cast<const u32x4_t*>(vb + row * kvs);
      }
      float sc[SUM_R];
      float mx = m;
#pragma unroll
      for (int r = 0; r < SUM_R; ++r) {
        float part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.x),
                                                     as_bf16x2(kw[r].x), 0.f, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.y),
                                               as_bf16x2(kw[r].y), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.z),
                                               as_bf16x2(kw[r].z), part, false);
        part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.w),
                                               as_bf16x2(kw[r].w), part, false);
        part = sum16(part);
        sc[r] = s0 + r < nrows ? part * a.sl : kNegInf;
        mx = fmaxf(mx, sc[r]);
      }
      const float al = m == kNegInf ? 0.f : fast_exp2(m - mx);
      l *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= al;
#pragma unroll
      for (int r = 0; r < SUM_R; ++r) {
        const float p = fast_exp2(sc[r] - mx);
        l += p;
        const u32x4_t w = vw[r];
        o[0] += p * bf_lo(w.x); o[1] += p * bf_hi(w.x);
        o[2] += p * bf_lo(w.y); o[3] += p * bf_hi(w.y);
        o[4] += p * bf_lo(w.z); o[5] += p * bf_hi(w.z);
        o[6] += p * bf_lo(w.w); o[7] += p * bf_hi(w.w);
      }
      m = mx;
    }
    if (hval) {
      const float inv = 1.f / l;
      u32x4_t ow;
      ow.x = pk_bf16(o[0] * inv, o[1] * inv);
      ow.y = pk_bf16(o[2] * inv, o[3] * inv);
      ow.z = pk_bf16(o[4] * inv, o[5] * inv);
      ow.w = pk_bf16(o[6] * inv, o[7] * inv);
      *reinterpret_cast<u32x4_t*>(out + (static_cast<int64_t>(b) * a.L + srow_a) * a.hq * D +
                                  static_cast<int64_t>(h) * D + 8 * c) = ow;
      if (lse && c == 0)
        lse[(static_cast<int64_t>(b) * a.hq + h) * a.L + srow_a] = (m + log2f(l)) * kLn2;
    }
  }
}

// Summary query rows for k <= 8, several per wave: a wave attends
// kSumPerWave consecutive (summary, head group) units, the next unit's key,
// value and query rows loaded while the current one is computed, so a wave
// pays one memory round trip for all of them.  The summary workgroups run
// two per CU (the launch's LDS allocation), first in the launch; with one
// summary per wave the 8192 of them filled about the first 65 us of the
// 32K prefill, with four about 50 us (per-workgroup timestamps).  Unit u
// is summary j of (sequence, kv head) item u / n_hgrp and head group
// 4 (u % n_hgrp); lane (hh, c) holds dims 8c .. 8c+7 of head hh of the
// group; the k + 1 rows j(k+1) .. j(k+1)+k are read as 9 rows, rows past
// the chunk repeating its last row and masked.  The arithmetic is that of
// summary_rows_wave's single pass.
constexpr int kSumPerWave = 4;

struct SumUnitRows {
  u32x4_t qw, kw[9], vw[9];
};

template <bool QROT>
__device__ void summary_rows_wave_multi(const MfmaArgs& a, int64_t u0, int64_t n_units,
                                        const bf16_t* __restrict__ q, const bf16_t* __restrict__ kx,
                                        const bf16_t* __restrict__ vx, bf16_t* __restrict__ out,
                                        float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int hh = lane >> 4;
  const int n_hgrp = (a.g + 3) >> 2;
  const int64_t kvs = static_cast<int64_t>(a.hkv) * D;
  // this lane's rotation rate (frequency lane), read before any row load:
  // a wait for a later-issued load would also wait for every row load
  // issued before it
  uint64_t fq_lane = 0;
  if constexpr (QROT) fq_lane = a.rope_fq[lane];
  __builtin_amdgcn_sched_barrier(0);
  struct Unit {
    int b, kvh, j, hg;
  };
  // Units past the last are read and computed as the last one (the same
  // values stored again): the loop below has no branch, so every wait for a
  // unit's rows counts exactly the row loads issued after them.
  const uint32_t u_last = static_cast<uint32_t>(n_units - 1);
  auto unit_of = [&](int64_t u) {
    const uint32_t uc = static_cast<uint32_t>(u) < u_last ? static_cast<uint32_t>(u) : u_last;
    Unit t;
    const uint32_t item = uc / static_cast<uint32_t>(n_hgrp);
    t.hg = 4 * static_cast<int>(uc - item * n_hgrp);
    const uint32_t bk = item / static_cast<uint32_t>(a.M);
    t.j = static_cast<int>(item - bk * a.M);
    t.b = static_cast<int>(bk / static_cast<uint32_t>(a.hkv));
    t.kvh = static_cast<int>(bk - t.b * a.hkv);
    return t;
  };
  auto head_of = [&](const Unit& t) {
    const int hloc = t.hg + hh;
    return t.kvh * a.g + (hloc < a.g ? hloc : 0);
  };
  auto load = [&](const Unit& t, SumUnitRows& r) __attribute__((always_inline)) {
    const int r0 = t.j * (a.k + 1);
    const int srow_a = r0 + a.k;
    r.qw = *reinterpret_cast<const u32x4_t*>(q + (static_cast<int64_t>(t.b) * a.L + srow_a) * a.hq * D +
                                             static_cast<int64_t>(head_of(t)) * D + 8 * c);
    const bf16_t* kb = kx + static_cast<int64_t>(t.b) * a.L * kvs + t.kvh * D + 8 * c;
    const bf16_t* vb = vx + static_cast<int64_t>(t.b) * a.L * kvs + t.kvh * D + 8 * c;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const int row = r0 + min(i, a.k);
      r.kw[i] = *reinterpret_cast<const u32x4_t*>(kb + row * kvs);
      r.vw[i] = *reinterpret_cast<const u32x4_t*>(vb + row * kvs);
    }
  };
  auto compute = [&](const Unit& t, SumUnitRows& r) __attribute__((always_inline)) {
    const int srow_a = t.j * (a.k + 1) + a.k;
    const int h = head_of(t);
    u32x4_t qw = r.qw;
    if constexpr (QROT) {
      // position of s_j: its chunk's last text token; dims 8c .. 8c+7 pair
      // with dims 8c +- 64, which lane c ^ 8 of the same 16 holds; lane l
      // forms angle l and each lane gathers its eight with ds_bpermute
      float sn_l, cs_l;
      rope_sincos(static_cast<uint32_t>((t.j + 1) * a.k - 1), fq_lane, &sn_l, &cs_l);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const uint32_t y = static_cast<uint32_t>(
            __builtin_amdgcn_update_dpp(0, static_cast<int>(qw[w]), 0x128, 0xF, 0xF, false));  // row_ror:8
        const int f0 = 4 * (8 * (c & 7) + 2 * w);  // byte address of lane f
        const float sn0 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0, __float_as_int(sn_l)));
        const float cs0 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0, __float_as_int(cs_l)));
        const float sn1 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0 + 4, __float_as_int(sn_l)));
        const float cs1 = __int_as_float(__builtin_amdgcn_ds_bpermute(f0 + 4, __float_as_int(cs_l)));
        qw[w] = rope_pair(qw[w], y, c >= 8, sn0, cs0, sn1, cs1);
      }
    }
    float sc[9];
    float mx = kNegInf;
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      float part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.x), as_bf16x2(r.kw[i].x), 0.f, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.y), as_bf16x2(r.kw[i].y), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.z), as_bf16x2(r.kw[i].z), part, false);
      part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw.w), as_bf16x2(r.kw[i].w), part, false);
      part = sum16(part);
      sc[i] = i <= a.k ? part * a.sl : kNegInf;
      mx = fmaxf(mx, sc[i]);
    }
    float l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int i = 0; i < 9; ++i) {
      const float p = fast_exp2(sc[i] - mx);
      l += p;
      const u32x4_t w = r.vw[i];
      o[0] += p * bf_lo(w.x); o[1] += p * bf_hi(w.x);
      o[2] += p * bf_lo(w.y); o[3] += p * bf_hi(w.y);
      o[4] += p * bf_lo(w.z); o[5] += p * bf_hi(w.z);
      o[6] += p * bf_lo(w.w); o[7] += p * bf_hi(w.w);
    }
    if (t.hg + hh < a.g) {
      const float inv = 1.f / l;
      u32x4_t ow;
      ow.x = pk_bf16(o[0] * inv, o[1] * inv);
      ow.y = pk_bf16(o[2] * inv, o[3] * inv);
      ow.z = pk_bf16(o[4] * inv, o[5] * inv);
      ow.w = pk_bf16(o[6] * inv, o[7] * inv);
      *reinterpret_cast<u32x4_t*>(out + (static_cast<int64_t>(t.b) * a.L + srow_a) * a.hq * D +
                                  static_cast<int64_t>(h) * D + 8 * c) = ow;
      if (lse && c == 0)
        lse[(static_cast<int64_t>(t.b) * a.hq + h) * a.L + srow_a] = (mx + log2f(l)) * kLn2;
    }
  };
  // two register sets in turn, in straight-line code: unit i + 1 loads
  // while unit i is computed; the scheduling barriers keep the compiler
  // from hoisting later units' loads (which would need a third set)
  if (u0 >= n_units) return;
  Unit ut[2];
  SumUnitRows rs[2];
  ut[0] = unit_of(u0);
  load(ut[0], rs[0]);
#pragma unroll
  for (int i = 0; i < kSumPerWave; ++i) {
    if (i + 1 < kSumPerWave) {
      ut[(i + 1) & 1] = unit_of(u0 + i + 1);
      load(ut[(i + 1) & 1], rs[(i + 1) & 1]);
    }
    __builtin_amdgcn_sched_barrier(0);
    compute(ut[i & 1], rs[i & 1]);
    __builtin_amdgcn_sched_barrier(0);
  }
}

}  // namespace

template <int HPW, bool QROT>
__global__ void __launch_bounds__(256, 2) prefill_mfma_d128_kernel(
    MfmaArgs a, const bf16_t* __restrict__ q, const bf16_t* __restrict__ kx,
    const bf16_t* __restrict__ vx, bf16_t* __restrict__ out, float* __restrict__ lse) {
  constexpr int PT = 32 * (4 / HPW);  // text positions per workgroup

  // Every argument the set-up reads, named at once: the compiler reads a
  // kernel argument where it is first used, and through the branches of the
  // set-up below that was a chain of scalar-load round trips; an empty asm
  // that takes them all in scalar registers makes it one round of loads.
  asm volatile("" ::"s"(a.batch), "s"(a.n), "s"(a.L), "s"(a.k), "s"(a.C), "s"(a.hq), "s"(a.hkv), "s"(a.g),
               "s"(a.M), "s"(a.n_tiles), "s"(a.n_hg), "s"(a.xcd_map), "s"(a.n_sum_blocks), "s"(a.divk_m),
               "s"(a.divk_l), "s"(a.sl), "s"(a.mode), "s"(a.W));
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (static_cast<int>(blockIdx.x) < a.n_sum_blocks) {
    const int64_t wid = static_cast<int64_t>(blockIdx.x) * 4 + wave;
    const int64_t n_items = static_cast<int64_t>(a.batch) * a.hkv * a.M;
    if (a.k <= 8) {
      summary_rows_wave_multi<QROT>(a, wid * kSumPerWave, n_items * ((a.g + 3) >> 2), q, kx, vx, out, lse);
    } else if (wid < n_items) {
      summary_rows_wave<16, QROT>(a, wid, q, kx, vx, out, lse);
    }
    return;
  }

  const int n_slots = a.batch * a.hkv * a.n_hg;
  const int bid = blockIdx.x - a.n_sum_blocks;
  int hslot, t_rev;
  if (a.xcd_map) {  // blocks are dispatched round-robin over the 8 XCDs
    const int x = bid & 7, s = bid >> 3;
    hslot = (s / a.n_tiles) * 8 + x;
    t_rev = s % a.n_tiles;
  } else {
    hslot = bid % n_slots;
    t_rev = bid / n_slots;
  }
  const int tile = a.n_tiles - 1 - t_rev;  // longest first
  const int hg = hslot % a.n_hg;
  const int kvh = (hslot / a.n_hg) % a.hkv;
  const int b = hslot / (a.n_hg * a.hkv);
  const int h = kvh * a.g + hg * HPW + (wave % HPW);

  // Key runs of the workgroup.
  const int p0 = tile * PT;
  const int p_last = (p0 + PT < a.n ? p0 + PT : a.n) - 1;
  const int c_first = div_k(a, p0), c_last = div_k(a, p_last);
  // summaries s_0 .. s_{sn-1} and text t0 .. p_last; the summary-free
  // baselines have no summary run, SWA a token window instead of a chunk one
  const int sn = a.mode == KSA_MODE_KSA && c_last - a.C > 0 ? c_last - a.C : 0;
  const int t0 = a.mode == KSA_MODE_SWA ? (p0 - a.W + 1 > 0 ? p0 - a.W + 1 : 0)
                                        : (c_first - a.C > 0 ? (c_first - a.C) * a.k : 0);
  const int ns = (sn + BN - 1) / BN;
  const int n_total = ns + (p_last - t0 + BN) / BN;

  // This wave's 32 queries and this lane's query.
  const int iw0 = p0 + 32 * (wave / HPW);
  const int iw1 = iw0 + 31 < a.n ? iw0 + 31 : a.n - 1;
  const bool wave_active = iw0 < a.n;
  const int qi = iw0 + (lane & 31);
  const bool q_valid = qi < a.n;
  const int ci = div_k(a, q_valid ? qi : 0);
  const int smax = q_valid ? ci - a.C - 1 : -1;                       // summaries j <= smax
  // first visible text key of this lane's query and of the wave's last query
  auto text_lo = [&](int i, int c) { return a.mode == KSA_MODE_SWA ? (i - a.W + 1 > 0 ? i - a.W + 1 : 0)
                                                                    : (c - a.C > 0 ? (c - a.C) * a.k : 0); };
  const int tlo = q_valid ? text_lo(qi, ci) : 0x7fffffff;
  const int thi = qi;
  const int cw0 = div_k(a, wave_active ? iw0 : 0), cw1 = div_k(a, wave_active ? iw1 : 0);
  const int tlo_w1 = text_lo(wave_active ? iw1 : 0, cw1);

  // Q^T as the B operand: column = query (lane % 32), k-slots
  // d = 16 ks + 8 (lane / 32) + j.  The rows are read through a buffer
  // resource based at the wave's first query row: a lane past the sequence
  // end gets an offset beyond the resource's range and reads zeros, so no
  // branch (and no wait for these loads) comes before the tile loads below.
  const int half = lane >> 5;
  bf16x8_t qop[8];
  {
    const int qrow0 = trow(a, wave_active ? iw0 : 0);
    const __amdgpu_buffer_rsrc_t rsrc_q = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(q + (static_cast<int64_t>(b) * a.L + qrow0) * a.hq * D + static_cast<int64_t>(h) * D),
        static_cast<short>(0), kQRange, 0x00020000);
    const int qoff = q_valid ? (trow(a, qi) - qrow0) * a.hq * ROW_BYTES + 16 * half : kQRange;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qop[ks] = __builtin_bit_cast(bf16x8_t, __builtin_amdgcn_raw_buffer_load_b128(rsrc_q, qoff + 32 * ks, 0, 0));
  }

  // Tile loads: thread owns 16-byte chunk (tid % 16) of rows tid/16 + 16 u
  // of a tile.  Tile indices are clamped to the last tile, so the loop body
  // loads without branching on the tile count.
  const int ld_chunk = tid & 15;
  const int ld_row = tid >> 4;
  const int kvs = a.hkv * D;  // elements per augmented row
  const int RB = kvs * 2;     // bytes per augmented row
  const int64_t kv_base = static_cast<int64_t>(b) * a.L * kvs + kvh * D;
  const int kv_bytes = (a.L * kvs - kvh * D) * 2;
  const __amdgpu_buffer_rsrc_t rsrc_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(kx + kv_base), static_cast<short>(0), kv_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rsrc_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(vx + kv_base), static_cast<short>(0), kv_bytes, 0x00020000);
  // direct-to-LDS loads place lane chunks linearly (row tid/16 + 16 u,
  // physical chunk tid % 16); the thread loads the logical chunk that the
  // swizzle maps there
  const int chunk16 = 16 * (ld_chunk ^ lds_swz(ld_row));
  const int sum_step = (a.k + 1) * RB;  // bytes between consecutive summary rows
  const int s_c0 = ld_row * sum_step + a.k * RB + chunk16;
  __shared__ __attribute__((aligned(16))) char lds_k0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILE_BYTES];
  char* const lds_k[2] = {lds_k0, lds_k1};
  char* const lds_v[2] = {lds_v0, lds_v1};

  // byte offsets of this thread's 4 rows of tile tt.  Rows past a run's end
  // are read (masked later) or, past the sequence, return zeros through the
  // buffer range check.  When k divides 64 a text tile starts 64 + 64/k rows
  // after the previous one.
  int t_base[4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
    t_base[u] = static_cast<int>(__umul24(static_cast<uint32_t>(trow(a, t0 + ld_row + 16 * u)), RB)) + chunk16;
  const int t_step = (BN + BN / a.k) * RB;
  const bool k_div = (BN % a.k) == 0;
  auto tile_offsets = [&](int tt, int* vo) {
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
  };
  auto load_tile = [&](const __amdgpu_buffer_rsrc_t& rs, char* buf, int tt) {
    int vo[4];
    tile_offsets(tt, vo);
#pragma unroll
    for (int u = 0; u < 4; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + (64 * wave + 256 * u) * 16), 16, vo[u], 0, 0, 0);
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float l_run = 0.f;      // this lane's half of the row sum

  // Per-lane LDS byte offsets, fixed for the whole loop.  K operand: row
  // lane % 32 (+32), chunk 2 ks + half.  Transposing V reads: in 16-lane
  // group G, lane (4 rr + c4) points at key row 16 ks + 8 rd + 4 (G / 2) + rr
  // and d = 32 db + 16 (G % 2) + 4 c4, and receives V[4 keys][d = 32 db + lane % 32].
  // chunk 2 ks + half of a row sits at lds_off(row, half) ^ (ks << 5)
  int koff0, voff[2][4];
  {
    const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
    koff0 = lds_off(lane & 31, half);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int d = 32 * db + 16 * (G & 1) + 4 * c4;
      const int row0 = 4 * (G >> 1) + rr;
      voff[0][db] = lds_off(row0, d >> 3) + 2 * (d & 7);
      voff[1][db] = lds_off(row0 + 8, d >> 3) + 2 * (d & 7);
    }
  }
  const uint32_t one2 = 0x3f803f80u;  // two bf16 ones

  // S^T = K Q^T for one tile: two independent 32-key MFMA chains.
  auto s_tile = [&](const char* kl, f32x16_t* sacc) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(kl + (koff0 ^ (ks << 5)) + 32 * ROW_BYTES * kb2);
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], sacc[kb2], 0, 0, 0);
      }
  };

  // Mask of tile tt (edge tiles only): visible iff lo <= key <= hi, with
  // key of (kb2, r) = key0 + 32 kb2 + 8 (r / 4) + 4 half + r % 4.
  auto mask_tile = [&](int tt, f32x16_t* sacc) {
    const bool is_sum = tt < ns;
    const int key0 = is_sum ? tt * BN : t0 + (tt - ns) * BN;
    bool full;
    if (is_sum)
      full = key0 + BN - 1 <= cw0 - a.C - 1;
    else
      full = key0 >= tlo_w1 && key0 + BN - 1 <= iw0;
    if (!full) {
      const int lo = is_sum ? -1 : tlo;
      const int hi = is_sum ? smax : thi;
      const int kbase = key0 + 4 * half;
      // key offsets 32 kb2 + 8 (r / 4) + r % 4 against per-lane bounds
      const int lo_r = lo - kbase, hi_r = hi - kbase;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int off = 32 * kb2 + 8 * (r >> 2) + (r & 3);
          sacc[kb2][r] = (off >= lo_r && off <= hi_r) ? sacc[kb2][r] : kNegInf;
        }
    }
  };
  // Row maximum of a score tile (log2 units, both lane halves).
  auto tile_max = [&](const f32x16_t* sacc) {
    float t = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) t = fmaxf(t, sacc[kb2][r]);
    return with_upper_half_max(t) * a.sl;
  };

  // P (bf16) of one 32-key half of a score tile and its row-sum share.
  auto p_of = [&](const f32x16_t* sc, int kb2, float nm, u32x4_t* pw) __attribute__((always_inline)) {
#pragma unroll
    for (int r = 0; r < 16; r += 2) {
      const float p0f = fast_exp2(fmaf(sc[kb2][r], a.sl, nm));
      const float p1f = fast_exp2(fmaf(sc[kb2][r + 1], a.sl, nm));
      const uint32_t w = pk_bf16(p0f, p1f);
      pw[2 * kb2 + (r >> 3)][(r & 7) >> 1] = w;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                              __builtin_bit_cast(bf16x2_t, one2), l_run, false);
    }
  };
  // O^T += V^T P^T for 16 keys (k-slot ks of a tile).
  auto pv_of = [&](const char* vl, const u32x4_t* pw, int ks) __attribute__((always_inline)) {
    const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw[ks]);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const bf16x4_t lo = lds_read_tr(vl, voff[0][db] + 16 * ROW_BYTES * ks);
      const bf16x4_t hi = lds_read_tr(vl, voff[1][db] + 16 * ROW_BYTES * ks);
      const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[db], 0, 0, 0);
    }
  };

  // Software pipeline.  Iteration tt: (A) the MFMAs of S for tile tt + 1
  // run while the VALU turns the scores of tile tt into P; (B) the MFMAs of
  // O += P V_tt run while the VALU masks tile tt + 1 and takes its maximum,
  // which decides the (rare) rescale applied at the top of the next
  // iteration.  LDS holds K_{tt+1} and V_tt; K_{tt+2} and V_{tt+1} are
  // loaded into registers at the top and stored at the bottom into the
  // buffers of K_tt and V_{tt-1}: one barrier per tile.
  float m_cur = kNegInf;  // maximum used for P of the current tile
  float m_nxt = kNegInf;  // maximum for the next tile
  bool grow = false;      // the next tile moves the maximum (wave-uniform)
  auto iter = [&](auto cur_c, int tt, f32x16_t* s_cur, f32x16_t* s_nxt) {
    constexpr int cur = decltype(cur_c)::value;
    const int last = n_total - 1;
    // rescale decided by the previous iteration
    const float alpha = m_cur == kNegInf ? 0.f : fast_exp2(m_cur - m_nxt);
    if (grow) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    l_run *= alpha;
    m_cur = m_nxt;
    load_tile(rsrc_v, lds_v[cur ^ 1], tt + 1 < last ? tt + 1 : last);
    load_tile(rsrc_k, lds_k[cur], tt + 2 < last ? tt + 2 : last);

    // ---- phase A: S of tile tt + 1 on MFMA, P of tile tt on VALU ----
    s_tile(lds_k[cur ^ 1], s_nxt);
    const float nm = m_cur == kNegInf ? 0.f : -m_cur;
    u32x4_t pw[4];
    // P of the first 32-key half here, the second half in phase B
    auto p_half = [&](int kb2) { p_of(s_cur, kb2, nm, pw); };
    p_half(0);
    asm volatile("" : "+v"(pw[0]));
    asm volatile("" : "+v"(pw[1]));
    asm volatile("" : "+v"(l_run));
    mask_tile(tt + 1, s_nxt);

    // ---- phase B: O^T += V^T P^T on MFMA, maximum of tile tt + 1 on VALU ----
    const char* vl = lds_v[cur];
    p_half(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pv_of(vl, pw, ks);
    const float tmax = tile_max(s_nxt);
    grow = __any(tmax > m_cur + kLazyRescale);
    m_nxt = grow ? fmaxf(m_cur, tmax) : m_cur;
    __syncthreads();
  };

  f32x16_t sa[2], sb[2];
  // Query rotation: text t_qi sits at position qi; dims f = 16 ks + 8 half
  // + j (ks < 4) and f + 64 are both in this lane.  (sin, cos) of the
  // angle of (position, f): with four heads per block all waves hold the
  // same 32 positions, so each thread forms 8 of the 32 x 64 pairs into
  // the second V buffer (not yet in use: the barrier before the loop orders
  // these reads before its first load) and every lane reads its 32;
  // otherwise each lane forms its own.  The table is written before the
  // first tile loads are issued (LDS accesses after a direct-to-LDS load
  // wait for it), so it is ready when the query rows arrive.
  [[maybe_unused]] float2* const tab = reinterpret_cast<float2*>(lds_v1);  // [f][position in the block's 32]
  if constexpr (QROT && HPW == 4) {
    static_assert(64 * 32 * sizeof(float2) <= TILE_BYTES, "the table fits one tile buffer");
    // thread (tp, fg) forms frequencies 8 fg .. 8 fg + 7, fg = 2 wave +
    // half, from wave-uniform (scalar) reads of the rates
    const int tp = tid & 31, fg = tid >> 5;
    const uint32_t pos = static_cast<uint32_t>(iw0 + tp);
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint64_t f_lo = a.rope_fq[16 * wave + j], f_hi = a.rope_fq[16 * wave + 8 + j];
      float sn, cs;
      rope_sincos(pos, half ? f_hi : f_lo, &sn, &cs);
      tab[(8 * fg + j) * 32 + tp] = make_float2(sn, cs);
    }
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): this thread's table writes are done
    __builtin_amdgcn_s_barrier();
  }
  if (n_total > 0) {
    load_tile(rsrc_k, lds_k[0], 0);
    load_tile(rsrc_v, lds_v[0], 0);
    load_tile(rsrc_k, lds_k[1], n_total > 1 ? 1 : 0);
  }
  if constexpr (QROT) {
    const uint32_t pos = static_cast<uint32_t>(qi);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      u32x4_t lo = __builtin_bit_cast(u32x4_t, qop[ks]), hi = __builtin_bit_cast(u32x4_t, qop[ks + 4]);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const int f = 16 * ks + 8 * half + 2 * w;
        float sn0, cs0, sn1, cs1;
        if constexpr (HPW == 4) {
          const float2 e0 = tab[f * 32 + (lane & 31)], e1 = tab[(f + 1) * 32 + (lane & 31)];
          sn0 = e0.x, cs0 = e0.y, sn1 = e1.x, cs1 = e1.y;
        } else {
          const int fu = 16 * ks + 2 * w;  // f without the lane half, wave-uniform
          rope_sincos(pos, half ? a.rope_fq[fu + 8] : a.rope_fq[fu], &sn0, &cs0);
          rope_sincos(pos, half ? a.rope_fq[fu + 9] : a.rope_fq[fu + 1], &sn1, &cs1);
        }
        const uint32_t x = lo[w], y = hi[w];
        lo[w] = rope_pair(x, y, false, sn0, cs0, sn1, cs1);
        hi[w] = rope_pair(y, x, true, sn0, cs0, sn1, cs1);
      }
      qop[ks] = __builtin_bit_cast(bf16x8_t, lo);
      qop[ks + 4] = __builtin_bit_cast(bf16x8_t, hi);
    }
  }

  if (n_total > 0) {
    __syncthreads();
    s_tile(lds_k[0], sa);
    mask_tile(0, sa);
    const float tmax = tile_max(sa);
    grow = true;
    m_nxt = tmax;
    __syncthreads();
  }
  // The loop runs every tile but the last, each iteration also forming the
  // scores of the next tile; the last tile only needs its P and P V (its
  // upper 32 keys are skipped when no query of the wave sees them, as on
  // the diagonal tile that ends every text run).
  const int n_loop = n_total - 1;
  for (int tt = 0; tt < n_loop; tt += 2) {
    iter(std::integral_constant<int, 0>(), tt, sa, sb);
    if (tt + 1 < n_loop) iter(std::integral_constant<int, 1>(), tt + 1, sb, sa);
  }
  if (n_total > 0) {
    const int tl = n_total - 1;
    const f32x16_t* s_last = (tl & 1) ? sb : sa;
    const char* vl = (tl & 1) ? lds_v[1] : lds_v[0];
    const float alpha = m_cur == kNegInf ? 0.f : fast_exp2(m_cur - m_nxt);
    if (grow) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    l_run *= alpha;
    m_cur = m_nxt;
    const float nm = m_cur == kNegInf ? 0.f : -m_cur;
    u32x4_t pw[4];
    p_of(s_last, 0, nm, pw);
    pv_of(vl, pw, 0);
    pv_of(vl, pw, 1);
    const int key0 = tl < ns ? tl * BN : t0 + (tl - ns) * BN;
    const bool hi_live = tl < ns ? key0 + 32 <= cw1 - a.C - 1 : key0 + 32 <= iw1;
    if (hi_live) {
      p_of(s_last, 1, nm, pw);
      pv_of(vl, pw, 2);
      pv_of(vl, pw, 3);
    }
  }
  const float m_ref = m_cur;

  if (!wave_active) return;
  const float l_tot = with_upper_half_sum(l_run);
  if (!q_valid) return;
  const float inv = 1.f / l_tot;
  const int orow = trow(a, qi);
  bf16_t* op = out + (static_cast<int64_t>(b) * a.L + orow) * a.hq * D + static_cast<int64_t>(h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * db + 8 * qq + 4 * half;
      uint2 w;
      w.x = pk_bf16(oacc[db][4 * qq + 0] * inv, oacc[db][4 * qq + 1] * inv);
      w.y = pk_bf16(oacc[db][4 * qq + 2] * inv, oacc[db][4 * qq + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
  if (lse && half == 0)
    lse[(static_cast<int64_t>(b) * a.hq + h) * a.L + orow] = (m_ref + log2f(l_tot)) * kLn2;
}

bool prefill_mfma_supported(const PrefillArgs& a, int32_t dtype) {
  const int g = a.hq / a.hkv;
  // 32-bit index arithmetic inside the kernel
  const bool fits = a.L < (int64_t(1) << 24) && a.L * a.hkv * D * 2 < (int64_t(1) << 31) &&
                    a.L * static_cast<int64_t>(a.hq > a.hkv ? a.hq : a.hkv) * D < (int64_t(1) << 31) &&
                    static_cast<int64_t>(a.batch) * a.hkv * g * ((a.n_text + 31) / 32) < (int64_t(1) << 31);
  return dtype == KSA_DTYPE_BF16 && a.dqk == D && a.dv == D && !a.v_is_k_prefix && fits &&
         (g == 1 || g == 2 || g % 4 == 0);
}

template <int HPW>
static hipError_t launch_hpw(const PrefillArgs& p, const void* q, const void* k, const void* v,
                             void* out, float* lse, hipStream_t s) {
  constexpr int PT = 32 * (4 / HPW);
  MfmaArgs a;
  a.batch = p.batch;
  a.n = static_cast<int32_t>(p.n_text);
  a.L = static_cast<int32_t>(p.L);
  a.k = p.k;
  a.C = p.C;
  a.hq = p.hq;
  a.hkv = p.hkv;
  a.g = p.hq / p.hkv;
  a.M = static_cast<int32_t>(p.n_text / p.k);
  a.n_hg = a.g / HPW;
  a.n_tiles = static_cast<int32_t>((p.n_text + PT - 1) / PT);
  const int64_t n_slots = static_cast<int64_t>(a.batch) * a.hkv * a.n_hg;
  a.n_text_blocks = static_cast<int32_t>(n_slots * a.n_tiles);
  a.xcd_map = (n_slots % 8) == 0 ? 1 : 0;
  fast_div(static_cast<uint32_t>(a.k), &a.divk_m, &a.divk_l);
  a.sl = p.scale * kLog2e;
  a.mode = p.mode;
  a.W = static_cast<int32_t>(p.window_tokens);
  const int64_t sum_items = static_cast<int64_t>(a.batch) * a.hkv * a.M;
  // waves of summary rows: kSumPerWave (summary, head group) units each
  // when k <= 8, else one summary with all head groups
  const int64_t sum_waves =
      p.k <= 8 ? (sum_items * ((a.g + 3) / 4) + kSumPerWave - 1) / kSumPerWave : sum_items;
  a.n_sum_blocks = static_cast<int32_t>(((sum_waves + 3) / 4 + 7) / 8 * 8);  // keeps text blocks XCD-aligned
  const bool qrot = p.rope_theta > 0.0;
  for (int f = 0; f < 64; ++f) {
    // theta^(-2f/128) / (2 pi) revolutions per position, below 1/6, as a
    // 64-bit binary fraction: split so that each part is exact in a double
    constexpr long double kTwoPi = 6.283185307179586476925286766559L;
    const long double rate = qrot ? std::pow(static_cast<long double>(p.rope_theta), -2.0L * f / D) / kTwoPi : 0.0L;
    const long double scaled_hi = std::floor(std::ldexp(rate, 32));
    const long double rest = std::ldexp(rate, 32) - scaled_hi;  // in [0, 1)
    a.rope_fq[f] = (static_cast<uint64_t>(scaled_hi) << 32) + static_cast<uint64_t>(std::llround(std::ldexp(rest, 32)));
  }
  const int64_t blocks = a.n_text_blocks + a.n_sum_blocks;
  if (blocks == 0) return hipSuccess;
  if (qrot)
    hipLaunchKernelGGL((prefill_mfma_d128_kernel<HPW, true>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s,
                       a, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<bf16_t*>(out), lse);
  else
    hipLaunchKernelGGL((prefill_mfma_d128_kernel<HPW, false>), dim3(static_cast<uint32_t>(blocks)), dim3(256), 0,
                       s, a, static_cast<const bf16_t*>(q), static_cast<const bf16_t*>(k),
                       static_cast<const bf16_t*>(v), static_cast<bf16_t*>(out), lse);
  return hipGetLastError();
}

hipError_t launch_prefill_mfma_d128(const PrefillArgs& a, const void* q, const void* k,
                                    const void* v, void* out, float* lse, hipStream_t s) {
  const int g = a.hq / a.hkv;
  if (g == 1) return launch_hpw<1>(a, q, k, v, out, lse, s);
  if (g == 2) return launch_hpw<2>(a, q, k, v, out, lse, s);
  return launch_hpw<4>(a, q, k, v, out, lse, s);
}

}  // namespace ksa
