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
// tile is partial), loaded straight into LDS with per-lane row addresses
// from the Eq. (1) map (summary j at row j(k+1)+k, text x at x + x/k).
// Wave w owns heads 16w .. 16w+15 over the full key and value width:
// S^T = K Q^T on 16x16x32 bf16 MFMA (two 16-key blocks), and O^T += V^T P^T
// with V^T read through ds_read_b64_tr_b16 from the same tile in the key
// order in which the lane holds its probabilities, so no score leaves the
// wave.  The exponentials of a row use one reference per head (the first
// tile's maximum), so the 128 output accumulators are never rescaled; a row
// whose later tiles exceed that reference by more than 2^8 is computed again
// with its own maximum (found by the first pass).  Rows are taken longest
// first (text rows from the end of the sequence), summary rows last.
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
// LDS rows are padded to 1184 bytes (74 chunks of 16): 296 dwords, 40 mod
// the 64 banks, so the 8 rows a half wave reads in a transposing V^T read
// (8 dwords each) fall on 8 disjoint groups of 8 banks; rows 8 .. 15 of
// every 16 store their 16-byte chunks pairwise swapped (chunk c at c ^ 1),
// so the 16 rows of a K operand read (4 dwords each) cover all 64 banks too.
// (With 1168-byte rows, 36 mod 64, both reads met two-way conflicts.)
constexpr int RB = GRB + 32;            // 1184
constexpr int RCH = RB / 16;            // 74
constexpr int TILE_LDS = 37 * 64 * 16;  // 37888 bytes = 32 x 1184
static_assert(TILE_LDS == 32 * RB, "a tile fills its buffer exactly");
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
  const int g4 = lane >> 4;    // lane group: keys 4 g4 .. (and 16 + 4 g4 ..)
  const int l16 = lane & 15;   // head within the wave's 16
  const int head = 16 * wave + l16;
  const int64_t qo = (static_cast<int64_t>(b) * a.L + row) * HQ + head;

  // Q^T as the B operand of S^T = K Q^T on 16x16x32 MFMA: column = head
  // (lane % 16), k-slots d = 32 kd + 8 (lane / 16) + j over all 576 columns.
  bf16x8_t qop[18];
  {
    const bf16_t* qp = q + qo * DQK + 8 * g4;
#pragma unroll
    for (int kd = 0; kd < 18; ++kd) qop[kd] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * kd);
  }

  // Tile loads: LDS chunk s = 64 (8 i + wave) + lane of a tile (i < 5,
  // 8 i + wave < 37) is tile row s / 74, stored chunk s % 74, which holds
  // the row's chunk (s % 74) ^ ((row / 8) % 2); chunks 72 and 73 are LDS
  // padding and read 32 bytes past the row.
  const int nld = wave < 5 ? 5 : 4;
  auto trw = [&](int i) { return ((8 * i + wave) * 64 + lane) / RCH; };
  auto tch = [&](int i) {
    const int s_ = (8 * i + wave) * 64 + lane;
    const int r_ = s_ / RCH;
    return 16 * ((s_ - r_ * RCH) ^ ((r_ >> 3) & 1));
  };
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<bf16_t*>(kx + static_cast<int64_t>(b) * a.L * DQK), static_cast<short>(0), a.L * GRB, 0x00020000);
  auto prefetch = [&](int t, char* buf) __attribute__((always_inline)) {
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

  // O^T over the 512 value columns in 32 blocks of 16: lane holds head
  // lane % 16, d = 16 db + 4 (lane / 16) + r.
  f32x4_t oacc[32];
  float l_run = 0.f;
  // One exponent reference per head for the whole row, so the output
  // accumulators are never rescaled: the first pass takes the maximum of the
  // first tile; if a later tile exceeds it by more than 2^8, the row is
  // computed again with the row's maximum, which the first pass found.
  float m_ref = kNegInf, m_all = kNegInf;
  bool over = false;
  __shared__ int restart;
  if (tid == 0) restart = 0;
  const uint32_t one2 = 0x3f803f80u;
  // K operand (A of 16x16x32): key row lane % 16 (+16), d = 32 kd + 8 (lane / 16) + j
  // (chunk 4 kd + g4, stored at 4 kd + (g4 ^ 1) in rows 8 .. 15 of 16)
  const int krow_off = l16 * RB + 16 * (g4 ^ ((l16 >> 3) & 1));
  // V^T operand (A): in 16-lane group g4, lane (4 rr + c4) points at key row
  // 4 g4 + rr (+16 for the upper k-slots) and d = 16 db + 4 c4; the
  // transposing read gives lane i V[4 keys][d = 16 db + i % 16].  The k-slot
  // order {4 g4 .. 4 g4 + 3, 16 + 4 g4 .. 16 + 4 g4 + 3} is the order in which
  // the lane holds its probabilities, so P needs no exchange.
  const int rr = l16 >> 2, c4 = l16 & 3;
  const int vrow_off = (4 * g4 + rr) * RB + 16 * ((c4 >> 1) ^ ((g4 >> 1) & 1)) + 8 * (c4 & 1);

  auto tile_step = [&](auto cur_c, int t, bool first_pass) __attribute__((always_inline)) {
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
    // tile t + 2 goes into the buffer of tile t - 1 (released by the barrier)
    if (t + 2 < ntile) prefetch(t + 2, lds[(cur + 2) % NBUF]);
    const char* kl = lds[cur];
    // ---- S^T = K Q^T: two 16-key blocks x 16 heads, two chains each ----
    f32x4_t s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int kd = 0; kd < 18; ++kd) {
      const bf16x8_t k0 = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 64 * kd);
      const bf16x8_t k1 = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 16 * RB + 64 * kd);
      s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qop[kd], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qop[kd], s1, 0, 0, 0);
    }
    float sv[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
    // keys of the tile: 16 (e / 4) + 4 g4 + e % 4 < valid
    const int valid = t < ns ? sn - t * TK : x_last - (t0 + (t - ns) * TK) + 1;
    if (valid < TK) {
#pragma unroll
      for (int e = 0; e < 8; ++e) sv[e] = (16 * (e >> 2) + 4 * g4 + (e & 3)) < valid ? sv[e] : kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int e = 0; e < 8; ++e) tmax = fmaxf(tmax, sv[e]);
    tmax = with_upper_half_max(with_row_pair_max(tmax)) * a.sl;
    if (first_pass) {
      if (t == 0) m_ref = tmax;
      m_all = fmaxf(m_all, tmax);
      over = over || tmax > m_ref + kLazy;
    }
    const float nm = -m_ref;
    u32x4_t pw;
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const uint32_t w = pk_bf16(fast_exp2(fmaf(sv[e], a.sl, nm)), fast_exp2(fmaf(sv[e + 1], a.sl, nm)));
      pw[e >> 1] = w;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, one2),
                                              l_run, false);
    }
    const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw);
    // ---- O^T += V^T P^T over 32 blocks of 16 value columns ----
#pragma unroll
    for (int db = 0; db < 32; ++db) {
      const int off = vrow_off + 32 * db;
      const bf16x4_t lo = lds_read_tr(kl, off);
      const bf16x4_t hi = lds_read_tr(kl, off + 16 * RB);
      const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[db] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, oacc[db], 0, 0, 0);
    }
  };
  for (int pass = 0; pass < 2; ++pass) {
#pragma unroll
    for (int db = 0; db < 32; ++db)
#pragma unroll
      for (int r = 0; r < 4; ++r) oacc[db][r] = 0.f;
    l_run = 0.f;
    const bool first_pass = pass == 0;
    if (!first_pass) m_ref = m_all;
    if (ntile > 0) prefetch(0, lds[0]);
    if (ntile > 1) prefetch(1, lds[1]);
    for (int t = 0; t < ntile; t += 3) {
      tile_step(std::integral_constant<int, 0>(), t, first_pass);
      if (t + 1 < ntile) tile_step(std::integral_constant<int, 1>(), t + 1, first_pass);
      if (t + 2 < ntile) tile_step(std::integral_constant<int, 2>(), t + 2, first_pass);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS write in flight
    if (!first_pass) break;
    // one decision for the workgroup (the tiles are shared); the barrier also
    // releases the tile buffers for a second pass
    if (__any(over) && lane == 0) restart = 1;
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    wg_barrier();
    if (!restart) break;
  }

  const float l_tot = with_upper_half_sum(with_row_pair_sum(l_run));
  const float inv = 1.f / l_tot;
  bf16_t* op = out + qo * DV + 4 * g4;
#pragma unroll
  for (int db = 0; db < 32; ++db) {
    u32x2_t w;
    w.x = pk_bf16(oacc[db][0] * inv, oacc[db][1] * inv);
    w.y = pk_bf16(oacc[db][2] * inv, oacc[db][3] * inv);
    *reinterpret_cast<u32x2_t*>(op + 16 * db) = w;
  }
  if (lse && g4 == 0)
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
