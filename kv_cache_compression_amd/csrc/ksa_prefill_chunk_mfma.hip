// Chunked (and variable-length, batched) KSA prefill against the cache for
// bf16, Dqk = Dv = 128, on gfx950 MFMA.
//
// A sequence with m committed chunks and r current-chunk tokens in its
// cache ("Kwai Summary Attention Technical Report", Sec. 2.3.1, Fig. 4)
// continues at augmented row a0 = m (k+1) + r of Eq. (1); its segment is
// the next R rows, packed with the other sequences' segments.  Every
// segment row gets exactly the output of the one-shot prefill (Eq. 3 and
// the summary rule).  The keys of a block of text queries are, as in the
// one-shot kernel, a summary run and a text run, each contiguous in its own
// index space; here each run is cut where the cache ends and the segment
// begins, giving up to four runs walked in 64-key tiles:
//   summaries j < m        cache summary buffer, slot 1 + k + C k + j;
//   summaries j >= m       segment rows;
//   text before the segment  the current chunk (token o at slot k - o) or
//                          ring chunk slot c mod C (token o at k - 1 - o);
//   text in the segment    segment rows.
// A tile never mixes sources, so each tile has one buffer resource and the
// loads stay direct-to-LDS; a run's last tile masks keys past the run's
// end.  The compute pipeline is the one-shot kernel's: S^T = K Q^T and
// O^T += V^T P^T on v_mfma_f32_32x32x16_bf16, lazy rescale, one barrier
// per tile; workgroups run longest-first and, when the slot count allows,
// all tiles of one (sequence, kv head) sit on one XCD so that the cache's
// summaries stay in that XCD's L2.  Summary query rows of the segments, one
// wave per (sequence, kv head, summary), take the last workgroups of the
// same launch: the shortest work fills the tail.
#include <type_traits>

#include "ksa_internal.h"
#include "ksa_mfma_common.h"

namespace ksa {

namespace {

using namespace mfma;

constexpr int BN = 64;
constexpr int TILE_BYTES = BN * ROW_BYTES;
constexpr float kLazyRescale = 8.f;  // log2 units
constexpr int SLOT_BYTES = ROW_BYTES; // one (slot, kv head) row of the cache

struct CkArgs {
  int32_t batch, k, C, hq, hkv, g, n_hg, n_tiles;
  uint32_t divk_m, divk_l, divc_m, divc_l;
  float sl;
  int32_t slots, sum0;  // cache slots per (sequence, kv head); first summary slot
  int32_t max_rows, max_sum_seg, n_sum_blocks, n_text_blocks, xcd_map;
  int64_t total_rows;
};

__device__ __forceinline__ int32_t div_k(const CkArgs& a, int32_t t) { return fast_div_apply(t, a.divk_m, a.divk_l); }
__device__ __forceinline__ int32_t trow(const CkArgs& a, int32_t t) { return t + div_k(a, t); }

// Cache slot of history text x (chunk cx <= m).
__device__ __forceinline__ int32_t text_slot(const CkArgs& a, int32_t x, int32_t m) {
  const int32_t cx = div_k(a, x);
  const int32_t ox = x - cx * a.k;
  if (cx == m) return a.k - ox;
  const int32_t ring = a.C > 0 ? cx - a.C * fast_div_apply(cx, a.divc_m, a.divc_l) : 0;
  return 1 + a.k + ring * a.k + (a.k - 1 - ox);
}

// Summary query s_j of a segment: its chunk's k text keys and itself.  Lane
// (hh, c) holds dims 8c .. 8c+7 of head hh of a group of four.  The key and
// value rows of a pass (SUM_R rows: 9, one pass, when k <= 8, else 16) are
// all loaded before any is used, so a pass costs one memory round trip;
// rows past the chunk are loaded (clamped) and masked.
template <int SUM_R>
__device__ void chunk_summary_wave(const CkArgs& a, int64_t item, const ChunkPtrs& p) {
  const int lane = threadIdx.x & 63;
  const int c = lane & 15;
  const int hh = lane >> 4;
  const int jl = static_cast<int>(item % a.max_sum_seg);
  const int kvh = static_cast<int>((item / a.max_sum_seg) % a.hkv);
  const int b = static_cast<int>(item / (static_cast<int64_t>(a.max_sum_seg) * a.hkv));
  const int m = p.state[4 * b], r = p.state[4 * b + 1];
  const int64_t off = p.seg_rows[b];
  const int64_t R = p.seg_rows[b + 1] - off;
  // state out of range or segment outside 0..max_rows: skipped, and flagged
  // once per sequence
  if (m < 0 || m > a.slots - a.sum0 || r < 0 || r > a.k || R < 0 || R > a.max_rows) {
    if (jl == 0 && kvh == 0 && lane == 0) p.state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SEGMENT;
    return;
  }
  const int a0 = m * (a.k + 1) + r;
  const int a1 = a0 + static_cast<int>(R);
  const int j = m + jl;
  if (j >= a1 / (a.k + 1)) return;
  const int t_seg = a0 - a0 / (a.k + 1);
  const int srow = j * (a.k + 1) + a.k;
  const int nrows = a.k + 1;
  const bf16_t* ckb = static_cast<const bf16_t*>(p.ck) + (static_cast<int64_t>(b) * a.hkv + kvh) * a.slots * D + 8 * c;
  const bf16_t* cvb = static_cast<const bf16_t*>(p.cv) + (static_cast<int64_t>(b) * a.hkv + kvh) * a.slots * D + 8 * c;
  const int64_t kvs = static_cast<int64_t>(a.hkv) * D;
  const bf16_t* skb = static_cast<const bf16_t*>(p.k) + (off - a0) * kvs + kvh * D + 8 * c;
  const bf16_t* svb = static_cast<const bf16_t*>(p.v) + (off - a0) * kvs + kvh * D + 8 * c;
  const bf16_t* qb = static_cast<const bf16_t*>(p.q);
  // key e of the chunk: text j k + e (the cache's current chunk, slot k - e,
  // while it precedes the segment; else a segment row), e = k: s_j itself
  auto kv_offset = [&](int e, bool* in_cache) -> int64_t {
    if (e == a.k) {
      *in_cache = false;
      return static_cast<int64_t>(srow) * kvs;
    }
    const int x = j * a.k + e;
    *in_cache = x < t_seg;
    return *in_cache ? static_cast<int64_t>(a.k - e) * D : static_cast<int64_t>(x + j) * kvs;
  };
  for (int hg = 0; hg < a.g; hg += 4) {
    const int hloc = hg + hh;
    const bool hval = hloc < a.g;
    const int h = kvh * a.g + (hval ? hloc : 0);
    const int64_t qrow = off + srow - a0;
    const u32x4_t qw = *reinterpret_cast<const u32x4_t*>(qb + (qrow * a.hq + h) * D + 8 * c);
    float m_run = kNegInf, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < nrows; s0 += SUM_R) {
      u32x4_t kw[SUM_R], vw[SUM_R];
#pragma unroll
      for (int rr = 0; rr < SUM_R; ++rr) {
        bool in_cache;
        const int64_t o_ = kv_offset(min(s0 + rr, nrows - 1), &in_cache);
        kw[rr] = *reinterpret_cast<const u32x4_t*>((in_cache ? ckb : skb) + o_);
        vw[rr] = *reinterpret_cast<const u32x4_t*>((in_cache ? cvb : svb) + o_);
      }
      float sc[SUM_R];
      float mx = m_run;
#pragma unroll
      for (int rr = 0; rr < SUM_R; ++rr) {
        float part = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w)
          part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qw[w]), as_bf16x2(kw[rr][w]), part, false);
        part = sum16(part);
        sc[rr] = s0 + rr < nrows ? part * a.sl : kNegInf;
        mx = fmaxf(mx, sc[rr]);
      }
      const float al = m_run == kNegInf ? 0.f : fast_exp2(m_run - mx);
      l *= al;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[e] *= al;
#pragma unroll
      for (int rr = 0; rr < SUM_R; ++rr) {
        const float pr = fast_exp2(sc[rr] - mx);
        l += pr;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          o[2 * w] += pr * bf_lo(vw[rr][w]);
          o[2 * w + 1] += pr * bf_hi(vw[rr][w]);
        }
      }
      m_run = mx;
    }
    if (hval) {
      const float inv = 1.f / l;
      u32x4_t ow;
#pragma unroll
      for (int w = 0; w < 4; ++w) ow[w] = pk_bf16(o[2 * w] * inv, o[2 * w + 1] * inv);
      *reinterpret_cast<u32x4_t*>(static_cast<bf16_t*>(p.out) + (qrow * a.hq + h) * D + 8 * c) = ow;
      if (p.lse && c == 0) p.lse[static_cast<int64_t>(h) * a.total_rows + qrow] = (m_run + log2f(l)) * kLn2;
    }
  }
}

}  // namespace

template <int HPW>
__global__ void __launch_bounds__(256, 2) prefill_chunk_d128_kernel(CkArgs a, ChunkPtrs p) {
  constexpr int PT = 32 * (4 / HPW);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int n_slots = a.batch * a.hkv * a.n_hg;
  const int bid = blockIdx.x;
  if (bid >= a.n_text_blocks) {  // summary query rows: the shortest work, last
    const int64_t item = static_cast<int64_t>(bid - a.n_text_blocks) * 4 + wave;
    if (item < static_cast<int64_t>(a.batch) * a.hkv * a.max_sum_seg) {
      if (a.k <= 8)
        chunk_summary_wave<9>(a, item, p);
      else
        chunk_summary_wave<16>(a, item, p);
    }
    return;
  }
  int hslot, t_rev;
  if (a.xcd_map) {  // blocks go round-robin to the 8 XCDs: one slot's tiles share an L2
    const int x = bid & 7, s8 = bid >> 3;
    hslot = (s8 / a.n_tiles) * 8 + x;
    t_rev = s8 % a.n_tiles;
  } else {
    hslot = bid % n_slots;
    t_rev = bid / n_slots;
  }
  const int tile = a.n_tiles - 1 - t_rev;  // later positions (more keys) first
  const int hg = hslot % a.n_hg;
  const int kvh = (hslot / a.n_hg) % a.hkv;
  const int b = hslot / (a.n_hg * a.hkv);
  const int h = kvh * a.g + hg * HPW + (wave % HPW);

  const int m = __builtin_amdgcn_readfirstlane(p.state[4 * b]);
  const int r = __builtin_amdgcn_readfirstlane(p.state[4 * b + 1]);
  if (m < 0 || m > a.slots - a.sum0 || r < 0 || r > a.k) return;  // state out of range: skipped
  const int64_t off = p.seg_rows[b];
  const int64_t R64 = p.seg_rows[b + 1] - off;
  if (R64 < 0 || R64 > a.max_rows) return;  // outside the launch's reach: skipped (flagged by the summary waves)
  const int R = static_cast<int>(R64);
  const int a0 = m * (a.k + 1) + r, a1 = a0 + R;
  const int t_seg = a0 - a0 / (a.k + 1), t_end = a1 - a1 / (a.k + 1);  // segment text [t_seg, t_end)
  const int p0 = (t_seg / PT) * PT + tile * PT;
  if (p0 >= t_end) return;
  const int qlo = p0 > t_seg ? p0 : t_seg;
  const int p_last = (p0 + PT < t_end ? p0 + PT : t_end) - 1;
  const int c_first = div_k(a, qlo), c_last = div_k(a, p_last);
  const int sn = c_last - a.C > 0 ? c_last - a.C : 0;
  const int t0 = c_first - a.C > 0 ? (c_first - a.C) * a.k : 0;
  // runs: [0, e0) cache summaries, [m, sn) segment summaries,
  //       [t0, e2) cache text, [s3, p_last] segment text
  const int e0 = sn < m ? sn : m;
  const int len1 = sn - m > 0 ? sn - m : 0;
  const int e2 = p_last + 1 < t_seg ? p_last + 1 : t_seg;
  const int len2 = e2 - t0 > 0 ? e2 - t0 : 0;
  const int s3 = t0 > t_seg ? t0 : t_seg;
  const int n0 = (e0 + BN - 1) / BN, n1 = (len1 + BN - 1) / BN, n2 = (len2 + BN - 1) / BN;
  const int n01 = n0 + n1, n012 = n01 + n2;
  const int n_total = n012 + (p_last - s3 + BN) / BN;

  const int iw0 = p0 + 32 * (wave / HPW);
  const int iw0v = iw0 > t_seg ? iw0 : t_seg;  // first valid query of the wave
  const int iw1 = iw0 + 31 < p_last ? iw0 + 31 : p_last;
  const bool wave_active = iw0v <= iw1;
  const int qi = iw0 + (lane & 31);
  const bool q_valid = qi >= t_seg && qi <= p_last;
  const int ci = div_k(a, q_valid ? qi : t_seg);
  const int smax = q_valid ? ci - a.C - 1 : -1;
  const int tlo = q_valid ? (ci - a.C > 0 ? (ci - a.C) * a.k : 0) : 0x7fffffff;
  const int cw0 = div_k(a, wave_active ? iw0v : t_seg), cw1 = div_k(a, wave_active ? iw1 : t_seg);
  const int tlo_w1 = cw1 - a.C > 0 ? (cw1 - a.C) * a.k : 0;

  const int half = lane >> 5;
  const int64_t qrow = off + (q_valid ? trow(a, qi) : t_seg + div_k(a, t_seg)) - a0;
  bf16x8_t qop[8];
  {
    const bf16_t* qp = static_cast<const bf16_t*>(p.q) + (qrow * a.hq + h) * D + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qop[ks] = q_valid ? *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks) : bf16x8_t{};
  }

  const int ld_chunk = tid & 15;
  const int ld_row = tid >> 4;
  const int RB = a.hkv * D * 2;  // bytes per segment row
  const int chunk16 = 16 * (ld_chunk ^ lds_swz(ld_row));
  const int64_t cbase = (static_cast<int64_t>(b) * a.hkv + kvh) * a.slots * D;
  const int cbytes = a.slots * SLOT_BYTES;
  const int64_t sbase = off * a.hkv * D + kvh * D;
  const int sbytes = R * RB - kvh * D * 2;
  const __amdgpu_buffer_rsrc_t rc_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const bf16_t*>(p.ck) + cbase)), static_cast<short>(0), cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rc_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const bf16_t*>(p.cv) + cbase)), static_cast<short>(0), cbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_k = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const bf16_t*>(p.k) + sbase)), static_cast<short>(0), sbytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rs_v = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<void*>(static_cast<const void*>(static_cast<const bf16_t*>(p.v) + sbase)), static_cast<short>(0), sbytes, 0x00020000);
  __shared__ __attribute__((aligned(16))) char lds_k0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_k1[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v0[TILE_BYTES];
  __shared__ __attribute__((aligned(16))) char lds_v1[TILE_BYTES];
  char* const lds_k[2] = {lds_k0, lds_k1};
  char* const lds_v[2] = {lds_v0, lds_v1};
  // tile tt -> run (0..3), first key, run end (exclusive); computed once per
  // tile and carried through the pipeline
  struct TileDesc {
    int run, key0, kend;
  };
  // tile tt of run r starts at key tt BN + shift_r and ends its run at
  // kend_r: sums of steps taken at the run boundaries, no branches
  const int dsh1 = m - n0 * BN, dsh2 = t0 - n01 * BN - dsh1, dsh3 = s3 - n012 * BN - dsh1 - dsh2;
  const int dke1 = sn - e0, dke2 = e2 - sn, dke3 = p_last + 1 - e2;
  auto tile_run = [&](int tt) {
    TileDesc d;
    const int r1 = -static_cast<int>(tt >= n0), r2 = -static_cast<int>(tt >= n01), r3 = -static_cast<int>(tt >= n012);
    // wave-uniform by construction; said so, or hipcc may treat the run's
    // buffer resource as per-lane and loop over its values
    d.run = __builtin_amdgcn_readfirstlane(-(r1 + r2 + r3));
    d.key0 = __builtin_amdgcn_readfirstlane(tt * BN + (r1 & dsh1) + (r2 & dsh2) + (r3 & dsh3));
    d.kend = __builtin_amdgcn_readfirstlane(e0 + (r1 & dke1) + (r2 & dke2) + (r3 & dke3));
    return d;
  };
  // Where a tile's 64 rows live: the source (cache or segment), a uniform
  // byte offset and one per-lane offset per 16-row group.  Rows past the
  // run's end repeat its last row, so V stays finite under the masked P = 0.
  // Formed once per tile for its K load and kept for its V load a step later.
  struct TileAddr {
    int vo[4];
    int so;
    int cache;  // 1: the cache, 0: the segment
  };
  auto tile_addr = [&](const TileDesc& d) {
    TileAddr t;
    const int lim = d.kend - 1 - d.key0;  // the run's last row within the tile
    t.cache = (d.run & 1) ^ 1;
    if (d.run < 2) {
      // summaries: slot sum0 + j in the cache, row j (k+1) + k - a0 in the
      // segment, both affine in j
      const int stride = d.run == 0 ? SLOT_BYTES : (a.k + 1) * RB;
      t.so = d.run == 0 ? (a.sum0 + d.key0) * SLOT_BYTES : (d.key0 * (a.k + 1) + a.k - a0) * RB;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        t.vo[u] = static_cast<int>(__umul24(static_cast<uint32_t>(min(ld_row + 16 * u, lim)), stride)) + chunk16;
    } else if (d.run == 3) {
      // segment text x = key0 + xl at row x + x / k - a0, where
      // x / k = key0 / k + (key0 mod k + xl) / k
      const int q0 = div_k(a, d.key0), r0 = d.key0 - q0 * a.k;
      t.so = (d.key0 + q0 - a0) * RB;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int xl = min(ld_row + 16 * u, lim);
        t.vo[u] = static_cast<int>(__umul24(static_cast<uint32_t>(xl + div_k(a, r0 + xl)), RB)) + chunk16;
      }
    } else {
      t.so = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        t.vo[u] = text_slot(a, d.key0 + min(ld_row + 16 * u, lim), m) * SLOT_BYTES + chunk16;
    }
    t.so = __builtin_amdgcn_readfirstlane(t.so);  // the load's scalar offset
    return t;
  };
  // a tile of K (is_v false) or V into buf, straight to LDS
  auto load_tile = [&](bool is_v, char* buf, const TileAddr& t) {
    const __amdgpu_buffer_rsrc_t rs = t.cache != 0 ? (is_v ? rc_v : rc_k) : (is_v ? rs_v : rs_k);
    const int so = t.so;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      // offsets go to the builtin as plain ints: handed a struct member
      // directly, hipcc's host pass emits no launch stub for the kernel
      const int vo = t.vo[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(
          rs, (__attribute__((address_space(3))) void*)(buf + (64 * wave + 256 * u) * 16), 16, vo, so, 0, 0);
    }
  };

  f32x16_t oacc[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int rr = 0; rr < 16; ++rr) oacc[db][rr] = 0.f;
  float l_run = 0.f;

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
  const uint32_t one2 = 0x3f803f80u;

  auto s_tile = [&](const char* kl, f32x16_t* sacc) {
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) sacc[kb2][rr] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2) {
        const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(kl + (koff0 ^ (ks << 5)) + 32 * ROW_BYTES * kb2);
        sacc[kb2] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], sacc[kb2], 0, 0, 0);
      }
  };
  // visible iff lo <= key <= hi and key < the run's end
  auto mask_tile = [&](const TileDesc& d, f32x16_t* sacc) {
    const int run = d.run, key0 = d.key0, kend = d.kend;
    const bool is_sum = run < 2;
    bool full;
    if (is_sum)
      full = key0 + BN - 1 <= min(cw0 - a.C - 1, kend - 1);
    else
      full = key0 >= tlo_w1 && key0 + BN - 1 <= min(iw0v, kend - 1);
    if (!full) {
      const int lo = is_sum ? -1 : tlo;
      const int hi = min(is_sum ? smax : qi, kend - 1);
      const int kbase = key0 + 4 * half;
#pragma unroll
      for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int key = kbase + 32 * kb2 + 8 * (rr >> 2) + (rr & 3);
          sacc[kb2][rr] = (key >= lo && key <= hi) ? sacc[kb2][rr] : kNegInf;
        }
    }
  };
  auto tile_max = [&](const f32x16_t* sacc) {
    float t = kNegInf;
#pragma unroll
    for (int kb2 = 0; kb2 < 2; ++kb2)
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) t = fmaxf(t, sacc[kb2][rr]);
    return with_upper_half_max(t) * a.sl;
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

  float m_cur = kNegInf, m_nxt = kNegInf;
  bool grow = false;
  TileDesc d1;  // tile tt + 1 (clamped to the last), carried between iterations
  TileAddr t1;  // its rows
  auto iter = [&](auto cur_c, int tt, f32x16_t* s_cur, f32x16_t* s_nxt) __attribute__((always_inline)) {
    constexpr int cur = decltype(cur_c)::value;
    const int last = n_total - 1;
    const float alpha = m_cur == kNegInf ? 0.f : fast_exp2(m_cur - m_nxt);
    if (grow) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= alpha;
    }
    l_run *= alpha;
    m_cur = m_nxt;
    // LDS holds K_{tt+1} and V_tt; V_{tt+1} and K_{tt+2} replace V_{tt-1}, K_tt
    const TileDesc d2 = tile_run(tt + 2 < last ? tt + 2 : last);
    load_tile(true, lds_v[cur ^ 1], t1);
    const TileAddr t2 = tile_addr(d2);
    load_tile(false, lds_k[cur], t2);
    s_tile(lds_k[cur ^ 1], s_nxt);
    const float nm = m_cur == kNegInf ? 0.f : -m_cur;
    u32x4_t pw[4];
    auto p_half = [&](int kb2) __attribute__((always_inline)) {
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const float p0f = fast_exp2(fmaf(s_cur[kb2][rr], a.sl, nm));
        const float p1f = fast_exp2(fmaf(s_cur[kb2][rr + 1], a.sl, nm));
        const uint32_t w = pk_bf16(p0f, p1f);
        pw[2 * kb2 + (rr >> 3)][(rr & 7) >> 1] = w;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, one2),
                                                l_run, false);
      }
    };
    p_half(0);
    mask_tile(d1, s_nxt);
    const char* vl = lds_v[cur];
    p_half(1);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) pv_of(vl, pw, ks);
    const float tmax = tile_max(s_nxt);
    grow = __any(tmax > m_cur + kLazyRescale);
    m_nxt = grow ? fmaxf(m_cur, tmax) : m_cur;
    d1 = d2;
    t1 = t2;
    __syncthreads();
  };

  f32x16_t sa[2], sb[2];
  // n_total >= 1: the segment's own text run holds at least the query
  {
    const TileDesc d0 = tile_run(0);
    d1 = tile_run(n_total > 1 ? 1 : 0);
    const TileAddr t0a = tile_addr(d0);
    t1 = tile_addr(d1);
    load_tile(false, lds_k[0], t0a);
    load_tile(true, lds_v[0], t0a);
    load_tile(false, lds_k[1], t1);
    __syncthreads();
    s_tile(lds_k[0], sa);
    mask_tile(d0, sa);
  }
  m_nxt = tile_max(sa);
  grow = true;
  __syncthreads();
  // Every tile but the last goes through the pipeline (which also forms the
  // next tile's scores); the last tile, always in the segment's own text run,
  // only needs its P and P V, and its upper 32 keys only when a query of the
  // wave reaches them.
  const int n_loop = n_total - 1;
  for (int tt = 0; tt < n_loop; tt += 2) {
    iter(std::integral_constant<int, 0>(), tt, sa, sb);
    if (tt + 1 < n_loop) iter(std::integral_constant<int, 1>(), tt + 1, sb, sa);
  }
  {
    const int tl = n_total - 1;
    const f32x16_t* s_last = (tl & 1) ? sb : sa;
    const char* vl = (tl & 1) ? lds_v[1] : lds_v[0];
    const float alpha = m_cur == kNegInf ? 0.f : fast_exp2(m_cur - m_nxt);
    if (grow) {
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) oacc[db][rr] *= alpha;
    }
    l_run *= alpha;
    m_cur = m_nxt;
    const float nm = m_cur == kNegInf ? 0.f : -m_cur;
    u32x4_t pw[4];
    auto p_half = [&](int kb2) __attribute__((always_inline)) {
#pragma unroll
      for (int rr = 0; rr < 16; rr += 2) {
        const float p0f = fast_exp2(fmaf(s_last[kb2][rr], a.sl, nm));
        const float p1f = fast_exp2(fmaf(s_last[kb2][rr + 1], a.sl, nm));
        const uint32_t w = pk_bf16(p0f, p1f);
        pw[2 * kb2 + (rr >> 3)][(rr & 7) >> 1] = w;
        l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w), __builtin_bit_cast(bf16x2_t, one2),
                                                l_run, false);
      }
    };
    p_half(0);
    pv_of(vl, pw, 0);
    pv_of(vl, pw, 1);
    const TileDesc dl = tile_run(tl);
    const bool hi_live = dl.run >= 2 ? dl.key0 + 32 <= iw1 : dl.key0 + 32 <= cw1 - a.C - 1;
    if (hi_live) {
      p_half(1);
      pv_of(vl, pw, 2);
      pv_of(vl, pw, 3);
    }
  }
  const float m_ref = m_cur;
  if (!wave_active) return;
  const float l_tot = with_upper_half_sum(l_run);
  if (!q_valid) return;
  const float inv = 1.f / l_tot;
  bf16_t* op = static_cast<bf16_t*>(p.out) + (qrow * a.hq + h) * D;
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
  if (p.lse && half == 0) p.lse[static_cast<int64_t>(h) * a.total_rows + qrow] = (m_ref + log2f(l_tot)) * kLn2;
}

bool prefill_chunk_mfma_supported(const ChunkArgs& a, int32_t dtype) {
  const int g = a.hq / a.hkv;
  const int64_t max_len = a.max_rows + a.slots;  // bounds every index the kernel forms
  return dtype == KSA_DTYPE_BF16 && a.dqk == D && a.dv == D && !a.v_is_k_prefix &&
         (g == 1 || g == 2 || g % 4 == 0) && a.slots * SLOT_BYTES < (int64_t(1) << 31) &&
         a.total_rows * a.hkv * D * 2 < (int64_t(1) << 31) && a.total_rows * a.hq * D < (int64_t(1) << 31) &&
         max_len < (int64_t(1) << 24) && (a.k + 1) * static_cast<int64_t>(a.hkv) * D * 2 < (int64_t(1) << 24);
}

template <int HPW>
static hipError_t launch_hpw(const ChunkArgs& c, const ChunkPtrs& p, hipStream_t s) {
  constexpr int PT = 32 * (4 / HPW);
  CkArgs a;
  a.batch = c.batch;
  a.k = c.k;
  a.C = c.C;
  a.hq = c.hq;
  a.hkv = c.hkv;
  a.g = c.hq / c.hkv;
  a.n_hg = a.g / HPW;
  // text tokens of a segment <= its rows; one more tile for the alignment
  a.n_tiles = static_cast<int32_t>((c.max_rows + PT - 1) / PT + 1);
  fast_div(static_cast<uint32_t>(a.k), &a.divk_m, &a.divk_l);
  fast_div(static_cast<uint32_t>(a.C > 0 ? a.C : 1), &a.divc_m, &a.divc_l);
  a.sl = c.scale * kLog2e;
  a.slots = static_cast<int32_t>(c.slots);
  a.sum0 = 1 + a.k + a.C * a.k;
  a.max_rows = static_cast<int32_t>(c.max_rows);
  a.max_sum_seg = static_cast<int32_t>(c.max_rows / (c.k + 1) + 1);
  a.total_rows = c.total_rows;
  const int64_t sum_items = static_cast<int64_t>(a.batch) * a.hkv * a.max_sum_seg;
  a.n_sum_blocks = static_cast<int32_t>((sum_items + 3) / 4);
  const int64_t n_slots = static_cast<int64_t>(a.batch) * a.hkv * a.n_hg;
  a.n_text_blocks = static_cast<int32_t>(n_slots * a.n_tiles);
  a.xcd_map = (n_slots % 8) == 0 ? 1 : 0;
  const int64_t blocks = static_cast<int64_t>(a.n_text_blocks) + a.n_sum_blocks;
  hipLaunchKernelGGL(prefill_chunk_d128_kernel<HPW>, dim3(static_cast<uint32_t>(blocks)), dim3(256), 0, s, a, p);
  return hipGetLastError();
}

hipError_t launch_prefill_chunk_mfma(const ChunkArgs& a, const ChunkPtrs& p, hipStream_t s) {
  const int g = a.hq / a.hkv;
  if (g == 1) return launch_hpw<1>(a, p, s);
  if (g == 2) return launch_hpw<2>(a, p, s);
  return launch_hpw<4>(a, p, s);
}

}  // namespace ksa
