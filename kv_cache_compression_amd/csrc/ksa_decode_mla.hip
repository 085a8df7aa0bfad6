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
// range for all 128 heads, so every cache row leaves HBM once.
//   - 32-key tiles go straight from global memory into LDS (buffer_load ...
//     lds), two tiles ahead, triple-buffered; rows are padded to 1168 bytes
//     so that the MFMA operand reads (16 rows x 16 B) and the transposing
//     reads (4 rows x 32 B) are free of bank conflicts; a lane past the
//     range reads zeros, so the last, partial tile needs no clamping;
//   - wave w owns heads 16w .. 16w+15 over the full key width: S^T = K Q^T
//     on 16x16x32 bf16 MFMA (Q^T of its heads in registers), softmax in
//     registers (lane = head, 8 keys per lane), and O^T += V^T P^T on the
//     same MFMA with V^T read through ds_read_b64_tr_b16 from the same
//     tile; P stays in the registers the scores were in, with the keys of a
//     tile ordered to match (each lane group holds keys 4g..4g+3 and
//     16+4g..16+4g+3);
//   - each range writes (max, sum, unnormalised output in bf16) per head;
//     a second kernel merges the ranges of a sequence by their maxima.
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
  int32_t batch, k, C, max_summaries, smax, n_cu;
  int64_t slots;
  float sl;  // scale * log2(e)
};

struct MlaSlice {
  int32_t start, len;
};

__device__ __forceinline__ MlaSlice mla_slice(const MlaArgs& a, const int32_t* state, int kind) {
  const int m = state[0], r = state[1];
  MlaSlice s;
  if (kind == 0) {
    const bool ok = r >= 0 && r <= a.k && m >= 0 && m <= a.max_summaries;
    s.start = 1 + a.k - r;
    s.len = ok ? r + (m < a.C ? m : a.C) * a.k + (m > a.C ? m - a.C : 0) : 0;
  } else if (kind == 1) {
    const bool ok = r == 0 && m >= 1 && m <= a.max_summaries;
    s.start = 0;
    s.len = ok ? a.k + 1 : 0;
  } else {
    s.start = 0;
    s.len = 0;
  }
  return s;
}

// Per-sequence plan, computed once per call by mla_plan_kernel:
// {slice start, slice length, rows per range, number of ranges}, followed
// by a work list of (sequence, range) pairs, one per split workgroup.
struct MlaPlan {
  int32_t start, len, per, nsp, first, pad0, pad1, pad2;  // first: index of its first work item
};

constexpr int kMlaCuCap = 1024;  // CU counts above this are clamped

}  // namespace

// Record of one (sequence, range, head): {m (log2 units), l} as two floats,
// then 512 bf16 of the unnormalised output.  The workspace starts with the
// per-sequence plans (256-byte aligned), then the records.
constexpr int kMlaRec = 8 + DV * 2;

// Work-list capacity: with ranges of ceil(total / n_cu) rows there are at
// most n_cu + batch of them.
__host__ __device__ __forceinline__ int mla_max_items(int batch) { return kMlaCuCap + batch; }

__host__ __device__ __forceinline__ size_t mla_plan_bytes(int batch) {
  return (static_cast<size_t>(batch) * sizeof(MlaPlan) + sizeof(int32_t) * 2 * mla_max_items(batch) + 255) /
         256 * 256;
}

// Cut every slice into ranges of about (total rows / CU count) rows, at least
// 64, and list the (sequence, range) work items.  One workgroup, one thread
// per sequence (batch <= 1024).
__global__ void __launch_bounds__(1024) mla_plan_kernel(MlaArgs a, const int32_t* __restrict__ state,
                                                        const int32_t* __restrict__ kind,
                                                        MlaPlan* __restrict__ plan) {
  __shared__ int64_t part[1024 / 64];
  const int b = threadIdx.x;
  MlaSlice sl = {0, 0};
  if (b < a.batch && kind[b] >= 0) sl = mla_slice(a, state + 4 * b, kind[b]);
  int64_t v = sl.len;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  if ((b & 63) == 0) part[b >> 6] = v;
  __syncthreads();
  int64_t total = 0;
  for (int w = 0; w < (static_cast<int>(blockDim.x) + 63) / 64; ++w) total += part[w];
  // ranges of total / (n_cu - batch) rows give at most n_cu ranges, so the
  // two head groups fill exactly two rounds of workgroups
  const int64_t slots = a.n_cu - a.batch > a.n_cu / 2 ? a.n_cu - a.batch : a.n_cu / 2;
  int64_t target = (total + slots - 1) / slots;
  if (target < 64) target = 64;
  target = (target + TK - 1) / TK * TK;
  __shared__ int32_t nsp_s[1024];
  MlaPlan pl;
  pl.start = sl.start;
  pl.len = sl.len;
  pl.per = static_cast<int32_t>(target);
  pl.nsp = static_cast<int32_t>((sl.len + target - 1) / target);
  nsp_s[b] = b < a.batch ? pl.nsp : 0;
  __syncthreads();
  // work list: item i -> (sequence, range); unused items get sequence -1
  int32_t* items = reinterpret_cast<int32_t*>(plan + a.batch);
  if (b < a.batch) {
    int first = 0;
    for (int i = 0; i < b; ++i) first += nsp_s[i];
    pl.first = first;
    plan[b] = pl;
    for (int r = 0; r < pl.nsp; ++r) {
      items[2 * (first + r)] = b;
      items[2 * (first + r) + 1] = r;
    }
  }
  int used = 0;
  for (int i = 0; i < a.batch; ++i) used += nsp_s[i];
  for (int i = used + b; i < mla_max_items(a.batch); i += blockDim.x) items[2 * i] = -1;
}

__global__ void __launch_bounds__(512, 1) decode_mla_split_kernel(
    MlaArgs a, const bf16_t* __restrict__ ck, const int32_t* __restrict__ state,
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kind, char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds0[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds1[TILE_LDS];
  __shared__ __attribute__((aligned(16))) char lds2[TILE_LDS];
  char* const lds[NBUF] = {lds0, lds1, lds2};
  const int item = blockIdx.x;
  const int32_t* items = reinterpret_cast<const int32_t*>(reinterpret_cast<const MlaPlan*>(ws) + a.batch);
  const int b = items[2 * item];
  if (b < 0) return;  // uniform over the block
  const int sp = items[2 * item + 1];
  const MlaPlan pl = reinterpret_cast<const MlaPlan*>(ws)[b];
  const MlaSlice sl = {pl.start, pl.len};
  const int per = pl.per, nsp = pl.nsp;
  if (sp >= nsp) return;  // uniform over the block
  const int r0 = sp * per;
  const int r1 = r0 + per < sl.len ? r0 + per : sl.len;
  const int ntile = (r1 - r0 + TK - 1) / TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l16 = lane & 15;  // head within the wave (S, P, O layouts) / key or d row (operands)
  const int g4 = lane >> 4;   // 16-lane group
  const int head = 16 * wave + l16;
  const bf16_t* kseq = ck + (static_cast<int64_t>(b) * a.slots + sl.start + r0) * DQK;

  // Q^T as the B operand of S^T = K Q^T on 16x16x32 MFMA: column = head
  // (lane % 16), k-slots d = 32 ks + 8 (lane / 16) + j.
  bf16x8_t qop[18];
  {
    const bf16_t* qp = q + (static_cast<int64_t>(b) * HQ + head) * DQK + 8 * g4;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 32 * ks);
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

  // O^T (d x heads) in 32 blocks of 16 d: lane holds head lane % 16,
  // d = 16 blk + 4 (lane / 16) + r.
  f32x4_t oacc[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) oacc[i] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
  float m_ref = kNegInf, l_run = 0.f;

  // K operand (A of S^T): row = key 16 kb + lane % 16, bytes 64 ks + 16 (lane / 16).
  const int krow_off = l16 * RB + 16 * g4;
  // V^T operand (A of O^T += V^T P^T): the k-slots of lane group g are keys
  // 4g .. 4g+3 and 16+4g .. 16+4g+3 (the order in which the S^T layout holds
  // P); a transposing read over rows 4g + (lane % 16) / 4 and d = 16 blk +
  // 4 (lane % 4) gives lane i of the group V[4 keys][16 blk + i].
  const int vrow_off = (4 * g4 + (l16 >> 2)) * RB + 2 * (4 * (l16 & 3));

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
    if (t + 2 < ntile) prefetch(t + 2, lds[(cur + 2) % NBUF]);
    const char* kl = lds[cur];

    // ---- S^T = K Q^T: keys 0..15 and 16..31, two chains each ----
    f32x4_t s0a = {0.f, 0.f, 0.f, 0.f}, s0b = s0a, s1a = s0a, s1b = s0a;
#pragma unroll
    for (int ks = 0; ks < 18; ks += 2) {
      const bf16x8_t k0a = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 64 * ks);
      const bf16x8_t k1a = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 16 * RB + 64 * ks);
      const bf16x8_t k0b = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 64 * (ks + 1));
      const bf16x8_t k1b = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 16 * RB + 64 * (ks + 1));
      s0a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0a, qop[ks], s0a, 0, 0, 0);
      s1a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1a, qop[ks], s1a, 0, 0, 0);
      s0b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0b, qop[ks + 1], s0b, 0, 0, 0);
      s1b = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1b, qop[ks + 1], s1b, 0, 0, 0);
    }
    // lane: head lane % 16; sv[r] = key 4 g + r, sv[4 + r] = key 16 + 4 g + r
    float sv[8];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sv[r] = s0a[r] + s0b[r];
      sv[4 + r] = s1a[r] + s1b[r];
    }
    const int valid = (r1 - r0) - t * TK;
    if (valid < TK) {
#pragma unroll
      for (int j = 0; j < 8; ++j) sv[j] = (4 * g4 + (j & 3) + 16 * (j >> 2)) < valid ? sv[j] : kNegInf;
    }
    float tmax = kNegInf;
#pragma unroll
    for (int j = 0; j < 8; ++j) tmax = fmaxf(tmax, sv[j]);
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    tmax *= a.sl;
    if (__any(tmax > m_ref + kLazy)) {
      const float m_new = fmaxf(m_ref, tmax);
      const float alpha = m_ref == kNegInf ? 0.f : fast_exp2(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int i = 0; i < 32; ++i) oacc[i] *= alpha;
    }
    const float nm = m_ref == kNegInf ? 0.f : -m_ref;
    u32x4_t pw;
#pragma unroll
    for (int j = 0; j < 8; j += 2) {
      const uint32_t w = pk_bf16(fast_exp2(fmaf(sv[j], a.sl, nm)), fast_exp2(fmaf(sv[j + 1], a.sl, nm)));
      pw[j >> 1] = w;
      l_run = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                              __builtin_bit_cast(bf16x2_t, 0x3f803f80u), l_run, false);
    }
    const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw);
    // ---- O^T += V^T P^T over 32 blocks of 16 value columns ----
#pragma unroll
    for (int blk = 0; blk < 32; ++blk) {
      const bf16x4_t lo = lds_read_tr(kl, vrow_off + 32 * blk);
      const bf16x4_t hi = lds_read_tr(kl, vrow_off + 16 * RB + 32 * blk);
      const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      oacc[blk] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vop, pop, oacc[blk], 0, 0, 0);
    }
  };
  for (int t = 0; t < ntile; t += 3) {
    tile_step(std::integral_constant<int, 0>(), t);
    if (t + 1 < ntile) tile_step(std::integral_constant<int, 1>(), t + 1);
    if (t + 2 < ntile) tile_step(std::integral_constant<int, 2>(), t + 2);
  }
  __builtin_amdgcn_s_waitcnt(0x0070);  // no LDS write in flight at exit

  // ---- this range's partial: {m, l} and the unnormalised output (bf16) ----
  float l_tot = l_run + __shfl_xor(l_run, 16);
  l_tot += __shfl_xor(l_tot, 32);
  char* rec = ws + mla_plan_bytes(a.batch) + ((static_cast<int64_t>(item)) * HQ + head) * kMlaRec;
  if (g4 == 0) {
    reinterpret_cast<float*>(rec)[0] = m_ref;
    reinterpret_cast<float*>(rec)[1] = l_tot;
  }
  bf16_t* ro = reinterpret_cast<bf16_t*>(rec + 8);
#pragma unroll
  for (int blk = 0; blk < 32; ++blk) {
    u32x2_t w;
    w.x = pk_bf16(oacc[blk][0], oacc[blk][1]);
    w.y = pk_bf16(oacc[blk][2], oacc[blk][3]);
    *reinterpret_cast<u32x2_t*>(ro + 16 * blk + 4 * g4) = w;
  }
}

__global__ void __launch_bounds__(256) decode_mla_merge_kernel(MlaArgs a,
                                                               const int32_t* __restrict__ kind,
                                                               const char* __restrict__ ws,
                                                               bf16_t* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  if (kind[b] < 0) return;
  const MlaPlan pl = reinterpret_cast<const MlaPlan*>(ws)[b];
  const int nsp = pl.nsp;
  const char* rec0 = ws + mla_plan_bytes(a.batch) + (static_cast<int64_t>(pl.first) * HQ + head) * kMlaRec;
  const int64_t stride = static_cast<int64_t>(HQ) * kMlaRec;
  // weights of every range, computed once per block into LDS
  __shared__ float wgt[256];
  __shared__ float red[2];
  if (threadIdx.x < 64) {
    float mloc = kNegInf;
    for (int s = threadIdx.x; s < nsp; s += 64)
      mloc = fmaxf(mloc, reinterpret_cast<const float*>(rec0 + s * stride)[0]);
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mloc = fmaxf(mloc, __shfl_xor(mloc, o));
    const float mu = mloc == kNegInf ? 0.f : mloc;
    float lloc = 0.f;
    for (int s = threadIdx.x; s < nsp; s += 64) {
      const float* h = reinterpret_cast<const float*>(rec0 + s * stride);
      const float w = fast_exp2(h[0] - mu);
      if (s < 256) wgt[s] = w;
      lloc += w * h[1];
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) lloc += __shfl_xor(lloc, o);
    if (threadIdx.x == 0) {
      red[0] = mloc;
      red[1] = lloc;
    }
  }
  __syncthreads();
  const float mx = red[0], l = red[1];
  const float mu = mx == kNegInf ? 0.f : mx;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = 2 * threadIdx.x; d < DV; d += 2 * blockDim.x) {
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const char* r = rec0 + s * stride;
      const float w = s < 256 ? wgt[s] : fast_exp2(reinterpret_cast<const float*>(r)[0] - mu);
      const uint32_t v = *reinterpret_cast<const uint32_t*>(r + 8 + 2 * d);
      o0 += w * __uint_as_float(v << 16);
      o1 += w * __uint_as_float(v & 0xffff0000u);
    }
    *reinterpret_cast<uint32_t*>(out + (static_cast<int64_t>(b) * HQ + head) * DV + d) =
        pk_bf16(o0 * inv, o1 * inv);
  }
  if (lse && threadIdx.x == 0)
    lse[static_cast<int64_t>(b) * HQ + head] = l > 0.f ? (mx + log2f(l)) * kLn2 : kNegInf;
}

bool decode_mla_supported(const DecodeArgs& a, int32_t dtype) {
  return dtype == KSA_DTYPE_BF16 && a.v_is_k_prefix && a.dqk == DQK && a.dv == DV && a.hq == HQ &&
         a.hkv == 1 && a.batch <= 1024 && a.slots < (int64_t(1) << 31) / DQK;
}


size_t decode_mla_workspace_bytes(const DecodeArgs& a) {
  const size_t plan = mla_plan_bytes(a.batch);
  return plan + static_cast<size_t>(kMlaCuCap + a.batch) * HQ * kMlaRec;
}

hipError_t launch_decode_mla(const DecodeArgs& d, const void* ck, const int32_t* state, const void* q,
                             const int32_t* kind, void* out, float* lse, void* ws, hipStream_t s) {
  MlaArgs a;
  a.batch = d.batch;
  a.k = d.k;
  a.C = d.C;
  a.max_summaries = d.max_summaries;
  a.slots = d.slots;
  a.smax = 0;
  a.sl = d.scale * kLog2e;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    ncu = 256;
  a.n_cu = ncu > 0 ? (ncu < kMlaCuCap ? ncu : kMlaCuCap) : 256;
  hipLaunchKernelGGL(mla_plan_kernel, dim3(1), dim3(((d.batch + 63) / 64) * 64), 0, s, a, state, kind,
                     static_cast<MlaPlan*>(ws));
  hipError_t e0 = hipGetLastError();
  if (e0 != hipSuccess) return e0;
  hipLaunchKernelGGL(decode_mla_split_kernel, dim3(a.n_cu + d.batch), dim3(512), 0, s, a,
                     static_cast<const bf16_t*>(ck), state, static_cast<const bf16_t*>(q), kind,
                     static_cast<char*>(ws));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_merge_kernel, dim3(HQ, d.batch), dim3(256), 0, s, a, kind,
                     static_cast<const char*>(ws), static_cast<bf16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace ksa
