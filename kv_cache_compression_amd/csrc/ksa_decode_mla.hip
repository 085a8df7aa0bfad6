// KSA decode over an absorbed-MLA cache: 128 query heads share one latent
// key/value head; keys are 576 wide (512 latent + 64 rotary) and values are
// the first 512 key columns.
//
// "Kwai Summary Attention Technical Report", Sec. 3.2, Eq. (6) and Table 1:
// the summary compression composes with MLA, so the cache holds
// n/k + w*k + (current chunk) latent rows, read per decode step as one
// contiguous slice (Sec. 2.3.1, Fig. 4).
//
// Work decomposition: the slices of all sequences are cut into row ranges of
// about (total rows / CU count) rows; one workgroup of 8 wavefronts handles a
// range for all 128 heads, so every cache row leaves HBM once.  Every
// workgroup derives the cut itself from the cache states (a few lanes of
// arithmetic per sequence), so the decode is two launches: split and merge.
//   - 32-key tiles go straight from global memory into LDS (buffer_load ...
//     lds), two tiles ahead, triple-buffered; rows are padded to 1168 bytes
//     so that both the MFMA operand reads (32 rows x 16 B) and the
//     transposing reads (4 rows x 32 B) are free of bank conflicts; a lane
//     past the range reads zeros, so the last, partial tile needs no
//     clamping;
//   - waves 2p and 2p+1 own heads 32p .. 32p+31.  Wave 2p+h computes the
//     part of S^T = K Q^T over key columns 288h .. 288h+287 on 32x32x16 bf16
//     MFMA; the two parts are summed through LDS, both waves run the same
//     softmax, and wave 2p+h accumulates value columns 256h .. 256h+255 of
//     O^T += V^T P^T, V^T read through ds_read_b64_tr_b16 from the same
//     tile.  Splitting the key width as well as the value width keeps the
//     MFMA work undivided while each wave holds half of Q and of O, and
//     halves the LDS operand traffic of one wave per 16 heads;
//   - each range writes (max, sum, unnormalised output in bf16) per head;
//     the merge kernel combines the ranges of a sequence by their maxima and
//     flags sequences whose slice cannot be read.
#include <type_traits>

#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

namespace {

constexpr int DQK = 576, DV = 512;
constexpr int HQ = 128;
constexpr int TK = 32;                    // keys per tile
constexpr int RB = DQK * 2 + 16;          // padded LDS row: 1168 bytes (73 chunks)
constexpr int RCH = RB / 16;              // 73
constexpr int TILE_CH = 37 * 64;          // 16-byte chunks per tile buffer: 2368 >= 32 x 73
constexpr int TILE_LDS = TILE_CH * 16;    // 37888 bytes
constexpr int NBUF = 3;                   // tiles in LDS: the current one and two in flight
constexpr float kLazy = 8.f;
constexpr int KPF = 4;                    // K operand reads issued this many MFMAs ahead
constexpr int VPF = 4;                    // V^T operand reads issued this many MFMAs ahead

typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;

__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// Workgroup barrier without a memory fence; callers wait for exactly the
// counters they need first.
__device__ __forceinline__ void wg_barrier() {
  __asm__ volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

__device__ __forceinline__ bf16x4_t lds_read_tr(const char* base, int byte_off) {
  auto p = (lds_bf16x4_t*)((__attribute__((address_space(3))) char*)(base) + byte_off);
  return __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p);
}

struct MlaArgs {
  int32_t batch, k, C, max_summaries, n_cu, max_items;
  int64_t slots;
  float sl;  // scale * log2(e)
};

struct MlaSlice {
  int32_t start, len;
  bool ok;
};

// The slice of one sequence (Sec. 2.3.1): text queries read the current
// chunk, the ring and the summaries that left the window; summary queries
// read the scratch slot and the current chunk.  A slice that cannot be read
// (a summary query without a committed chunk, a state out of range) has
// length 0.
__device__ __forceinline__ MlaSlice mla_slice(const MlaArgs& a, const int32_t* state, int kind) {
  const int m = state[0], r = state[1];
  MlaSlice s;
  if (kind == 0) {
    s.ok = r >= 0 && r <= a.k && m >= 0 && m <= a.max_summaries;
    s.start = 1 + a.k - r;
    s.len = s.ok ? r + (m < a.C ? m : a.C) * a.k + (m > a.C ? m - a.C : 0) : 0;
  } else {
    s.ok = r == 0 && m >= 1 && m <= a.max_summaries;  // the summary was just committed
    s.start = 0;
    s.len = s.ok ? a.k + 1 : 0;
  }
  return s;
}

__device__ __forceinline__ int seq_len(const MlaArgs& a, const int32_t* state, const int32_t* kind, int b) {
  return (b < a.batch && kind[b] >= 0) ? mla_slice(a, state + 4 * b, kind[b]).len : 0;
}

// Rows per range: about total / (CU count - batch), at least 64, a whole
// number of tiles; with it the ranges of all sequences number at most the CU
// count.  Every lane of the calling wave gets the same value.
__device__ int mla_per(const MlaArgs& a, const int32_t* state, const int32_t* kind) {
  const int lane = threadIdx.x & 63;
  int64_t total = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    int64_t v = seq_len(a, state, kind, b0 + lane);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    total += v;
  }
  const int64_t slots = a.n_cu - a.batch > a.n_cu / 2 ? a.n_cu - a.batch : a.n_cu / 2;
  int64_t per = (total + slots - 1) / slots;
  if (per < 64) per = 64;
  return static_cast<int>((per + TK - 1) / TK * TK);
}

// Inclusive prefix sum over the 64 lanes of a wave.
__device__ __forceinline__ int wave_scan(int v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o);
    if (lane >= o) v += u;
  }
  return v;
}

// Work item `item` of the cut: ranges are numbered sequence by sequence;
// b = -1 when the item is past the last range.
struct MlaItem {
  int32_t b, sp, start, len, per;
};

__device__ MlaItem mla_item(const MlaArgs& a, const int32_t* state, const int32_t* kind, int item) {
  const int lane = threadIdx.x & 63;
  const int per = mla_per(a, state, kind);
  MlaItem it = {-1, 0, 0, 0, per};
  int first = 0;  // ranges of the sequences before this 64-sequence chunk
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    const int len = seq_len(a, state, kind, b);
    const int nsp = (len + per - 1) / per;
    const int incl = wave_scan(nsp);
    const bool mine = item >= first + incl - nsp && item < first + incl;
    const uint64_t hit = __ballot(mine);
    if (hit) {
      const int src = __builtin_ctzll(hit);
      it.b = __shfl(b, src);
      it.sp = item - first - (__shfl(incl, src) - __shfl(nsp, src));
      it.len = __shfl(len, src);
      it.start = (b < a.batch && kind[b] >= 0) ? mla_slice(a, state + 4 * b, kind[b]).start : 0;
      it.start = __shfl(it.start, src);
      return it;
    }
    first += __shfl(incl, 63);
  }
  return it;
}

// The cut per sequence for the merge: {first range, number of ranges},
// written by one wave of the first workgroup of the split launch.
__device__ void mla_write_cut(const MlaArgs& a, const int32_t* state, const int32_t* kind, int2* hdr) {
  const int lane = threadIdx.x & 63;
  const int per = mla_per(a, state, kind);
  int first = 0;
  for (int b0 = 0; b0 < a.batch; b0 += 64) {
    const int b = b0 + lane;
    const int nsp = (seq_len(a, state, kind, b) + per - 1) / per;
    const int incl = wave_scan(nsp);
    if (b < a.batch) hdr[b] = make_int2(first + incl - nsp, nsp);
    first += __shfl(incl, 63);
  }
}

}  // namespace

// At most CU count + batch work items (the cut above), whatever the device.
static constexpr int kMlaCuCap = 1024;

// Record of one (work item, head): {m (log2 units), l} as two floats, then
// 512 bf16 of the unnormalised output.  One bf16 rounding of the partial
// output before the merge costs the result about what its own bf16 output
// rounding does, and fp32 records would double the records' HBM traffic.
constexpr int kMlaRec = 8 + DV * 2;

// Workspace: the records of at most max_items = CUs + batch work items,
// then the per-sequence cut.
__host__ __device__ inline size_t mla_cut_offset(int max_items) {
  return static_cast<size_t>(max_items) * HQ * kMlaRec;
}

// CU count of the current device, capped at kMlaCuCap (the cut's slots).
static int mla_cu_count() {
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  return ncu > 0 ? (ncu < kMlaCuCap ? ncu : kMlaCuCap) : 256;
}

__global__ void __launch_bounds__(512, 1) decode_mla_split_kernel(
    MlaArgs a, const bf16_t* __restrict__ ck, const int32_t* __restrict__ state,
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kind, char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds0[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds1[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds2[TILE_LDS];
  // partial S^T exchange between the two waves of a pair: 16 values + 4
  // padding per lane
  __shared__ __attribute__((aligned(16))) float xs[8][64][20];
  char* const lds[NBUF] = {lds0, lds1, lds2};
  if (blockIdx.x == 0 && threadIdx.x < 64)
    mla_write_cut(a, state, kind, reinterpret_cast<int2*>(ws + mla_cut_offset(a.max_items)));
  const MlaItem it = mla_item(a, state, kind, blockIdx.x);
  // wave-uniform: keep them in scalar registers
  const int b = __builtin_amdgcn_readfirstlane(it.b);
  if (b < 0) return;  // uniform over the block
  const int per = __builtin_amdgcn_readfirstlane(it.per);
  const int len = __builtin_amdgcn_readfirstlane(it.len);
  const int start = __builtin_amdgcn_readfirstlane(it.start);
  const int r0 = __builtin_amdgcn_readfirstlane(it.sp) * per;
  const int r1 = r0 + per < len ? r0 + per : len;
  const int ntile = (r1 - r0 + TK - 1) / TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int pair = wave >> 1;  // heads 32 pair .. 32 pair + 31
  const int hf = wave & 1;     // key columns 288 hf .., value columns 256 hf ..
  const int half = lane >> 5;
  const int head = 32 * pair + (lane & 31);
  const bf16_t* kseq = ck + (static_cast<int64_t>(b) * a.slots + start + r0) * DQK;

  // Q^T (this wave's key-column half) as the B operand of S^T = K Q^T on
  // 32x32x16 MFMA: column = head (lane % 32), k-slots d = 288 hf + 16 ks + 8 half + j.
  bf16x8_t qop[18];
  {
    const bf16_t* qp = q + (static_cast<int64_t>(b) * HQ + head) * DQK + 288 * hf + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
  }

  // Tile copy straight into LDS through a buffer resource that starts at the
  // tile's first row and ends with this range's last row (the hardware range
  // check covers the per-lane offset only, so the tile base goes into the
  // resource).  Chunk s = 64 (8 i + wave) + lane of a tile (i < 5,
  // 8 i + wave < 37) is row s / 73, 16-byte chunk s % 73; chunk 72 is row
  // padding in LDS and just reads the next row's first chunk.
  const int nld = wave < 5 ? 5 : 4;
  int voff[5];
#pragma unroll
  for (int i = 0; i < 5; ++i) {
    const int s_ = (8 * i + wave) * 64 + lane;
    const int row = s_ / RCH;
    voff[i] = row * (DQK * 2) + 16 * (s_ - row * RCH);
  }
  auto prefetch = [&](int t, char* buf) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<bf16_t*>(kseq + static_cast<int64_t>(t) * TK * DQK), static_cast<short>(0),
        (r1 - r0 - t * TK) * (DQK * 2), 0x00020000);
#pragma unroll
    for (int i = 0; i < 5; ++i)
      if (i < nld)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(
            rsrc, (__attribute__((address_space(3))) void*)(buf + (8 * i + wave) * 1024), 16, voff[i], 0, 0, 0);
  };

  // O^T over this wave's 256 value columns in 8 blocks of 32: lane holds
  // head lane % 32, d = 256 hf + 32 db + 8 (r / 4) + 4 half + r % 4.
  f32x16_t oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_ref = kNegInf, l_run = 0.f;
  const uint32_t one2 = 0x3f803f80u;

  // K operand: row = key lane % 32, bytes 576 hf + 32 ks + 16 half.
  const int krow_off = (lane & 31) * RB + 16 * half + 576 * hf;
  // V^T operand: in 16-lane group G, lane (4 rr + c4) reads key row
  // 4 (G / 2) + rr (+ 8 for the second half of the k-slots) and d =
  // 256 hf + 32 db + 16 (G % 2) + 4 c4; the transposing read gives lane i
  // V[4 keys][d = 256 hf + 32 db + i % 32].
  const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
  const int vrow_off = (4 * (G >> 1) + rr) * RB + 2 * (16 * (G & 1) + 4 * c4) + 512 * hf;

  if (ntile > 0) prefetch(0, lds[0]);
  if (ntile > 1) prefetch(1, lds[1]);
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
    // operand reads run KPF MFMAs ahead of their use (measured: 4 deep and
    // the max-ilp scheduler take the decode from 115.6 to 108.5 us)
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
    // at the top of this iteration); issued after the exchange reads so that
    // they do not wait for it
    if (t + 2 < ntile) prefetch(t + 2, lds[(cur + 2) % NBUF]);
    // ---- softmax: lane = head, registers = keys 8 (r/4) + 4 half + r%4 ----
    const int valid = (r1 - r0) - t * TK;
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
    const float nm = m_ref == kNegInf ? 0.f : -m_ref;
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
      // V^T operand reads run VPF MFMAs ahead of their use
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
  for (int t = 0; t < ntile; t += 3) {
    tile_step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntile) tile_step(std::integral_constant<int, 1>(), t + 1);
    if (t + 2 < ntile) tile_step(std::integral_constant<int, 2>(), t + 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS write in flight at exit

  // ---- this range's partial (both waves of a pair hold the same m and l) ----
  const float l_tot = with_upper_half_sum(l_run);
  char* rec = ws + (static_cast<int64_t>(blockIdx.x) * HQ + head) * kMlaRec;
  if (half == 0 && hf == 0) {
    reinterpret_cast<float*>(rec)[0] = m_ref;
    reinterpret_cast<float*>(rec)[1] = l_tot;
  }
  bf16_t* ro = reinterpret_cast<bf16_t*>(rec + 8) + 256 * hf;
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq) {
      const int d = 32 * db + 8 * qq + 4 * half;
      u32x2_t w;
      w.x = pk_bf16(oacc[db][4 * qq + 0], oacc[db][4 * qq + 1]);
      w.y = pk_bf16(oacc[db][4 * qq + 2], oacc[db][4 * qq + 3]);
      *reinterpret_cast<u32x2_t*>(ro + d) = w;
    }
}

// One wave per (head, sequence), four heads per block: combine the ranges of
// the sequence by their maxima; the head-0 wave also flags a slice that
// cannot be read.  Every lane owns eight output columns and reads, sixteen
// ranges at a time, each range's (maximum, sum) and its eight columns in one
// round of loads; the 1024 blocks of the 32 x 128 case fit the chip at once.
__global__ void __launch_bounds__(256) decode_mla_merge_kernel(MlaArgs a, int32_t* __restrict__ state,
                                                               const int32_t* __restrict__ kind,
                                                               const char* __restrict__ ws,
                                                               bf16_t* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int lane = threadIdx.x & 63;
  const int head = 4 * blockIdx.x + __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int b = blockIdx.y;
  // both loads in one round trip: the cut is written for every sequence
  const int kb = kind[b];
  const int2 cut = reinterpret_cast<const int2*>(ws + mla_cut_offset(a.max_items))[b];
  if (kb < 0) return;
  if (head == 0 && lane == 0 && !mla_slice(a, state + 4 * b, kb).ok)
    state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SUMMARY_READ;
  const int nsp = cut.y;
  const char* rec0 = ws + (static_cast<int64_t>(cut.x) * HQ + head) * kMlaRec;
  const int64_t stride = static_cast<int64_t>(HQ) * kMlaRec;
  const int d = 8 * lane;  // 64 lanes x 8 columns = 512
  float mx = kNegInf, l = 0.f, o[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  constexpr int G = 16;
  for (int s0 = 0; s0 < nsp; s0 += G) {
    float2 ml[G];
    u32x2_t v[G][2];  // records are 8-byte aligned
#pragma unroll
    for (int u = 0; u < G; ++u) {
      if (s0 + u < nsp) {
        const char* r = rec0 + (s0 + u) * stride;
        ml[u] = *reinterpret_cast<const float2*>(r);
        v[u][0] = *reinterpret_cast<const u32x2_t*>(r + 8 + 2 * d);
        v[u][1] = *reinterpret_cast<const u32x2_t*>(r + 16 + 2 * d);
      } else {
        ml[u] = make_float2(kNegInf, 0.f);
        v[u][0] = v[u][1] = (u32x2_t){0u, 0u};
      }
    }
    float gm = mx;
#pragma unroll
    for (int u = 0; u < G; ++u) gm = fmaxf(gm, ml[u].x);
    const float mu = gm == kNegInf ? 0.f : gm;
    const float sc = mx == kNegInf ? 0.f : fast_exp2(mx - mu);
    l *= sc;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= sc;
#pragma unroll
    for (int u = 0; u < G; ++u) {
      const float w = ml[u].x == kNegInf ? 0.f : fast_exp2(ml[u].x - mu);
      l += w * ml[u].y;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t x = v[u][e >> 1][e & 1];
        o[2 * e] += w * __uint_as_float(x << 16);
        o[2 * e + 1] += w * __uint_as_float(x & 0xffff0000u);
      }
    }
    mx = gm;
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  u32x4_t ow;
#pragma unroll
  for (int e = 0; e < 4; ++e) ow[e] = pk_bf16(o[2 * e] * inv, o[2 * e + 1] * inv);
  *reinterpret_cast<u32x4_t*>(out + (static_cast<int64_t>(b) * HQ + head) * DV + d) = ow;
  if (lse && lane == 0)
    lse[static_cast<int64_t>(b) * HQ + head] = l > 0.f ? (mx + log2f(l)) * kLn2 : kNegInf;
}

bool decode_mla_supported(const DecodeArgs& a, int32_t dtype) {
  return dtype == KSA_DTYPE_BF16 && a.v_is_k_prefix && a.dqk == DQK && a.dv == DV && a.hq == HQ &&
         a.hkv == 1 && a.slots < (int64_t(1) << 31) / DQK;
}

// Any device (up to kMlaCuCap CUs).
size_t decode_mla_workspace_bytes(const DecodeArgs& a) {
  return mla_cut_offset(kMlaCuCap + a.batch) + static_cast<size_t>(a.batch) * sizeof(int2);
}

// What a launch on the current device uses.
size_t decode_mla_workspace_bytes_used(const DecodeArgs& a) {
  return mla_cut_offset(mla_cu_count() + a.batch) + static_cast<size_t>(a.batch) * sizeof(int2);
}

hipError_t launch_decode_mla(const DecodeArgs& d, const void* ck, int32_t* state, const void* q,
                             const int32_t* kind, void* out, float* lse, void* ws, hipStream_t s) {
  MlaArgs a;
  a.batch = d.batch;
  a.k = d.k;
  a.C = d.C;
  a.max_summaries = d.max_summaries;
  a.slots = d.slots;
  a.sl = d.scale * kLog2e;
  a.n_cu = mla_cu_count();
  a.max_items = a.n_cu + d.batch;
  if (d.batch > 0) {
    hipLaunchKernelGGL(decode_mla_split_kernel, dim3(a.max_items), dim3(512), 0, s, a,
                       static_cast<const bf16_t*>(ck), state, static_cast<const bf16_t*>(q), kind,
                       static_cast<char*>(ws));
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(decode_mla_merge_kernel, dim3(HQ / 4, d.batch), dim3(256), 0, s, a, state, kind,
                       static_cast<const char*>(ws), static_cast<bf16_t*>(out), lse);
  }
  return hipGetLastError();
}

}  // namespace ksa
