// Block-sparse KSA prefill for bf16, Dqk = Dv = 128, on gfx950 MFMA.
//
// "Kwai Summary Attention Technical Report", Sec. 2.3: the prefill kernel
// splits Q/K/V into fixed-size blocks and loads only block pairs that hold
// visible entries; the O(L^2) mask is never built.  The visible set of text
// token t_i (chunk c = floor(i/k)) is, by Eq. (3), the summaries
// s_0 .. s_{c-C-1} and the text t_{(c-C)k} .. t_i.  So for a block of
// consecutive text queries the visible keys are two runs, each contiguous in
// its own index space: a summary run [0, c_last - C) and a text run
// [(c_first - C) k, i_last].  This kernel walks those two runs in 64-key
// tiles; only tiles on a run's edge need an element mask, computed from
// integer compares on chunk indices.  Summary-query rows (k+1 keys each) are
// handled by the generic kernel.
//
// Work decomposition (one workgroup = 4 wavefronts):
//   - a workgroup owns one kv head and HPW of its query heads over PT
//     consecutive text positions (HPW * PT = 128 query rows); every wave owns
//     32 query rows of one head, so the K/V tile staged in LDS feeds 4 waves;
//   - S^T = K Q^T on v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q
//     held in registers), so each lane ends up owning one query row and the
//     softmax row statistics stay in-lane (one lane swap per tile);
//   - O^T += V^T P^T on the same MFMA: P goes straight from the score
//     registers into the B operand; V^T comes from the row-major V tile via
//     ds_read_b64_tr_b16 (transposing 4x16 bf16 blocks per 16 lanes);
//   - K/V tiles are prefetched into registers one tile ahead;
//   - workgroups are ordered longest-first (later queries see more
//     summaries) and, when the head count allows, all workgroups of one
//     (sequence, kv head) run on one XCD so its K/V stay in that XCD's L2.
#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

namespace {

constexpr int D = 128;
constexpr int BN = 64;            // keys per tile
constexpr int ROW_BYTES = D * 2;  // 256 B per key row
constexpr int TILE_BYTES = BN * ROW_BYTES;

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// 16-byte chunk c (0..15) of LDS row `row` is stored at chunk c ^ swz(row):
// 8 consecutive rows hit 8 different even chunks, and the next 8 the odd
// ones, so the MFMA operand reads of 32 rows x 16 B and the transposing
// reads of 4 rows x 32 B are spread over all banks.
__device__ __forceinline__ int lds_off(int row, int chunk) {
  const int swz = ((row & 7) << 1) | ((row >> 3) & 1);
  return row * ROW_BYTES + ((chunk ^ swz) << 4);
}

typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

__device__ __forceinline__ bf16x4_t lds_read_tr(const char* lds_base, int byte_off) {
  const lds_bf16x4_t* p = (const lds_bf16x4_t*)((__attribute__((address_space(3))) char*)(lds_base) + byte_off);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(const_cast<lds_bf16x4_t*>(p));
}

struct TileRuns {
  int64_t sn;   // summaries visible to the block: s_0 .. s_{sn-1}
  int64_t t0;   // first text key
  int64_t t1;   // last text key (inclusive)
  int ns, nt;   // summary tiles, text tiles
};

__device__ __forceinline__ TileRuns block_runs(int64_t p_first, int64_t p_last, int32_t k,
                                               int32_t C) {
  TileRuns r;
  const int64_t c_first = p_first / k;
  const int64_t c_last = p_last / k;
  r.sn = c_last - C > 0 ? c_last - C : 0;
  r.t0 = c_first - C > 0 ? (c_first - C) * k : 0;
  r.t1 = p_last;
  r.ns = static_cast<int>((r.sn + BN - 1) / BN);
  r.nt = static_cast<int>((r.t1 - r.t0 + 1 + BN - 1) / BN);
  return r;
}

}  // namespace

template <int HPW>
__global__ void __launch_bounds__(256, 2) prefill_mfma_d128_kernel(
    PrefillArgs a, int n_tiles, int n_hg, int xcd_map, const bf16_t* __restrict__ q,
    const bf16_t* __restrict__ kx, const bf16_t* __restrict__ vx, bf16_t* __restrict__ out,
    float* __restrict__ lse) {
  constexpr int PT = 32 * (4 / HPW);  // text positions per workgroup
  __shared__ __attribute__((aligned(16))) char k_lds[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char v_lds[TILE_BYTES];

  const int g = a.hq / a.hkv;
  const int64_t n_slots = static_cast<int64_t>(a.batch) * a.hkv * n_hg;
  const int64_t bid = blockIdx.x;
  int64_t hslot, t_rev;
  if (xcd_map) {  // blocks are dispatched round-robin over the 8 XCDs
    const int64_t x = bid & 7, s = bid >> 3;
    hslot = (s / n_tiles) * 8 + x;
    t_rev = s % n_tiles;
  } else {
    hslot = bid % n_slots;
    t_rev = bid / n_slots;
  }
  const int tile = n_tiles - 1 - static_cast<int>(t_rev);  // longest first
  const int hg = static_cast<int>(hslot % n_hg);
  const int kvh = static_cast<int>((hslot / n_hg) % a.hkv);
  const int b = static_cast<int>(hslot / (static_cast<int64_t>(n_hg) * a.hkv));

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = kvh * g + hg * HPW + (wave % HPW);
  const int64_t p0 = static_cast<int64_t>(tile) * PT;
  const int64_t p_last = (p0 + PT < a.n_text ? p0 + PT : a.n_text) - 1;
  const TileRuns runs = block_runs(p0, p_last, a.k, a.C);

  // This wave's 32 queries and this lane's query.
  const int64_t iw0 = p0 + 32 * (wave / HPW);
  const int64_t iw1 = (iw0 + 31 < a.n_text ? iw0 + 31 : a.n_text - 1);
  const bool wave_active = iw0 < a.n_text;
  const int64_t qi = iw0 + (lane & 31);
  const bool q_valid = qi < a.n_text;
  const int64_t ci = qi / a.k;
  const int64_t smax = q_valid ? ci - a.C - 1 : -1;  // visible summaries: j <= smax
  const int64_t tlo = q_valid ? (ci - a.C > 0 ? (ci - a.C) * a.k : 0) : INT64_MAX;
  const int64_t thi = qi;
  const int64_t cw0 = iw0 / a.k, cw1 = iw1 / a.k;
  const int64_t tlo_w1 = cw1 - a.C > 0 ? (cw1 - a.C) * a.k : 0;
  const int64_t tlo_w0 = cw0 - a.C > 0 ? (cw0 - a.C) * a.k : 0;

  // Q^T as the B operand: column = query (lane % 32), k-slots
  // d = 16 ks + 8 (lane / 32) + j.
  const int half = lane >> 5;
  bf16x8_t qop[8];
  {
    const int64_t qrow = text_row(q_valid ? qi : 0, a.k);
    const bf16_t* qp = q + ((static_cast<int64_t>(b) * a.L + qrow) * a.hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qop[ks] = q_valid ? *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks) : bf16x8_t{};
    }
  }

  // Global -> register prefetch of one K and one V tile: thread owns chunk
  // (tid % 16) of rows tid/16 + 16 u.
  const int ld_chunk = tid & 15;
  const int ld_row = tid >> 4;
  const int64_t kv_row_stride = static_cast<int64_t>(a.hkv) * D;  // elements per augmented row
  const bf16_t* kb = kx + static_cast<int64_t>(b) * a.L * kv_row_stride + kvh * D + 8 * ld_chunk;
  const bf16_t* vb = vx + static_cast<int64_t>(b) * a.L * kv_row_stride + kvh * D + 8 * ld_chunk;
  u32x4_t kreg[4], vreg[4];
  const int n_total = runs.ns + runs.nt;

  // Augmented row of key r of tile tt, clamped inside its run.
  auto tile_key_row = [&](int tt, int r) -> int64_t {
    if (tt < runs.ns) {
      int64_t j = static_cast<int64_t>(tt) * BN + r;
      if (j >= runs.sn) j = runs.sn - 1;
      return summary_row(j, a.k);
    }
    int64_t t = runs.t0 + static_cast<int64_t>(tt - runs.ns) * BN + r;
    if (t > runs.t1) t = runs.t1;
    return text_row(t, a.k);
  };
#define KSA_PREFETCH(tt)                                                        \
  do {                                                                          \
    _Pragma("unroll") for (int u = 0; u < 4; ++u) {                             \
      const int64_t ar = tile_key_row((tt), ld_row + 16 * u);                   \
      kreg[u] = *reinterpret_cast<const u32x4_t*>(kb + ar * kv_row_stride);    \
      vreg[u] = *reinterpret_cast<const u32x4_t*>(vb + ar * kv_row_stride);    \
    }                                                                           \
  } while (0)

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = kNegInf;
  float l_run = 0.f;
  const float sl = a.scale * kLog2e;

  if (n_total > 0) KSA_PREFETCH(0);
  for (int tt = 0; tt < n_total; ++tt) {
    __syncthreads();  // everyone is done with the previous tile
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int r = ld_row + 16 * u;
      *reinterpret_cast<u32x4_t*>(k_lds + lds_off(r, ld_chunk)) = kreg[u];
      *reinterpret_cast<u32x4_t*>(v_lds + lds_off(r, ld_chunk)) = vreg[u];
    }
    __syncthreads();
    if (tt + 1 < n_total) KSA_PREFETCH(tt + 1);

    // Does this tile hold anything for this wave, and does it need a mask?
    const bool is_sum = tt < runs.ns;
    const int64_t key0 = is_sum ? static_cast<int64_t>(tt) * BN
                                : runs.t0 + static_cast<int64_t>(tt - runs.ns) * BN;
    bool empty, full;
    if (is_sum) {
      empty = key0 > cw1 - a.C - 1;
      full = key0 + BN - 1 <= cw0 - a.C - 1;
    } else {
      empty = key0 > iw1 || key0 + BN - 1 < tlo_w0;
      full = key0 >= tlo_w1 && key0 + BN - 1 <= iw0;
    }
    if (!wave_active || empty) continue;

    // ---- S^T = K Q^T: two 32-key blocks ----
    f32x16_t sacc[2];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb2][r] = 0.f;
      const int krow = 32 * kb2 + (lane & 31);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8_t kop =
            *reinterpret_cast<const bf16x8_t*>(k_lds + lds_off(krow, 2 * ks + half));
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], sacc[kb2], 0, 0, 0);
      }
    }

    // ---- online softmax; lane = query, registers = keys ----
    // key of (kb2, r) = 32 kb2 + 8 (r / 4) + 4 half + r % 4
    float tmax = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s = sacc[kb2][r] * sl;
        if (!full) {
          const int64_t key = key0 + 32 * kb2 + 8 * (r >> 2) + 4 * half + (r & 3);
          const bool vis = is_sum ? key <= smax : (key >= tlo && key <= thi);
          s = vis ? s : kNegInf;
        }
        sacc[kb2][r] = s;
        tmax = fmaxf(tmax, s);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(m_run, tmax);
    const float m_use = m_new == kNegInf ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    m_run = m_new;
    float psum = 0.f;
    bf16x8_t pop[4];
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(sacc[kb2][r] - m_use);
        psum += p;
        pop[2 * kb2 + (r >> 3)][r & 7] = static_cast<__bf16>(p);
      }
    l_run = l_run * alpha + psum;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

    // ---- O^T += V^T P^T ----
    // Transposing read: in 16-lane group G, lane (4 rr + c4) points at key
    // row 16 ks + 8 rd + 4 (G / 2) + rr, d = 32 db + 16 (G % 2) + 4 c4; lane
    // then receives V[4 keys][d = 32 db + lane % 32].
    const int G = lane >> 4;
    const int l16 = lane & 15;
    const int rr = l16 >> 2, c4 = l16 & 3;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int d = 32 * db + 16 * (G & 1) + 4 * c4;
        const int row0 = 16 * ks + 4 * (G >> 1) + rr;
        const bf16x4_t lo = lds_read_tr(v_lds, lds_off(row0, d >> 3) + 2 * (d & 7));
        const bf16x4_t hi = lds_read_tr(v_lds, lds_off(row0 + 8, d >> 3) + 2 * (d & 7));
        const bf16x8_t vop = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop[ks], oacc[db], 0, 0, 0);
      }
    }
  }

#undef KSA_PREFETCH
  if (!wave_active) return;
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  if (!q_valid) return;
  const float inv = 1.f / l_tot;
  const int64_t orow = text_row(qi, a.k);
  bf16_t* op = out + ((static_cast<int64_t>(b) * a.L + orow) * a.hq + h) * D;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * db + 8 * qq + 4 * half;
      uint2 w;
      w.x = pack_bf16x2(oacc[db][4 * qq + 0] * inv, oacc[db][4 * qq + 1] * inv);
      w.y = pack_bf16x2(oacc[db][4 * qq + 2] * inv, oacc[db][4 * qq + 3] * inv);
      *reinterpret_cast<uint2*>(op + d) = w;
    }
  if (lse && half == 0)
    lse[(static_cast<int64_t>(b) * a.hq + h) * a.L + orow] = (m_run + log2f(l_tot)) * kLn2;
}

bool prefill_mfma_supported(const PrefillArgs& a, int32_t dtype) {
  const int g = a.hq / a.hkv;
  return dtype == KSA_DTYPE_BF16 && a.dqk == D && a.dv == D && !a.v_is_k_prefix &&
         (g == 1 || g == 2 || g % 4 == 0);
}

template <int HPW>
static hipError_t launch_hpw(const PrefillArgs& a, const void* q, const void* k, const void* v,
                             void* out, float* lse, hipStream_t s) {
  constexpr int PT = 32 * (4 / HPW);
  const int g = a.hq / a.hkv;
  const int n_hg = g / HPW;
  const int n_tiles = static_cast<int>((a.n_text + PT - 1) / PT);
  const int64_t n_slots = static_cast<int64_t>(a.batch) * a.hkv * n_hg;
  const int64_t blocks = n_slots * n_tiles;
  if (blocks == 0) return hipSuccess;
  const int xcd_map = (n_slots % 8) == 0 ? 1 : 0;
  hipLaunchKernelGGL(prefill_mfma_d128_kernel<HPW>, dim3(static_cast<uint32_t>(blocks)), dim3(256),
                     0, s, a, n_tiles, n_hg, xcd_map, static_cast<const bf16_t*>(q),
                     static_cast<const bf16_t*>(k), static_cast<const bf16_t*>(v),
                     static_cast<bf16_t*>(out), lse);
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
