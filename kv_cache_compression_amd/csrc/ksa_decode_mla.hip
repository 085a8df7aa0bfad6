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
// about (total rows / CU count); one workgroup of 8 wavefronts handles one
// range for all 128 heads, so every cache row leaves HBM once.
//   - 32-key tiles are copied global -> LDS with global_load_lds_dwordx4
//     (no registers involved), three buffers deep; rows are padded to 1168
//     bytes so that both the MFMA operand reads (32 rows x 16 B) and the
//     transposing reads (4 rows x 32 B) are free of bank conflicts;
//   - waves 2j and 2j+1 own heads 32j .. 32j+31.  Each computes half of
//     S^T = K Q^T (key columns 0..287 or 288..575) on 32x32x16 bf16 MFMA,
//     the halves are summed through LDS, both run the same softmax, and
//     each accumulates half of O^T += V^T P^T (value columns 0..255 or
//     256..511), V^T read through ds_read_b64_tr_b16 from the same tile.
//     Splitting the key width as well as the value width keeps the MFMA
//     work undivided while each wave holds half of Q and half of O;
//   - each range writes (max, sum, unnormalised output in bf16) per head;
//     a second kernel merges the ranges of a sequence by their maxima.
#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

namespace {

constexpr int DQK = 576, DV = 512;
constexpr int HQ = 128;
constexpr int NW = 8;                     // waves per workgroup: 4 head blocks x 2 halves
constexpr int TK = 32;                    // keys per tile
constexpr int RB = DQK * 2 + 16;          // padded LDS row: 1168 bytes (73 chunks)
constexpr int RCH = RB / 16;              // 73
constexpr int LOADS_PER_WAVE = 5;         // 16-byte lanes: 5 x 64 x 8 = 2560 >= 32 x 73
constexpr int TILE_LDS = NW * LOADS_PER_WAVE * 64 * 16;  // 40960 bytes
constexpr int NBUF = 3;
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

// Rows per range for sequence b: about total/n_cu, at least 64, and at most
// smax ranges per sequence.  Both kernels derive the same split from the
// device-side cache state.
__device__ __forceinline__ void mla_split(const MlaArgs& a, const int32_t* state, const int32_t* kind,
                                          int b, MlaSlice* sl, int* per, int* nsp) {
  int64_t total = 0;
  for (int i = 0; i < a.batch; ++i) total += mla_slice(a, state + 4 * i, kind[i]).len;
  int64_t target = (total + a.n_cu - 1) / a.n_cu;
  if (target < 64) target = 64;
  target = (target + TK - 1) / TK * TK;
  *sl = mla_slice(a, state + 4 * b, kind[b]);
  int64_t p = target;
  if ((sl->len + p - 1) / p > a.smax) p = ((sl->len + a.smax - 1) / a.smax + TK - 1) / TK * TK;
  *per = static_cast<int>(p);
  *nsp = static_cast<int>((sl->len + p - 1) / p);
}

}  // namespace

// Record of one (sequence, range, head): {m (log2 units), l} as two floats,
// then 512 bf16 of the unnormalised output.
constexpr int kMlaRec = 8 + DV * 2;

__global__ void __launch_bounds__(512, 1) decode_mla_split_kernel(
    MlaArgs a, const bf16_t* __restrict__ ck, const int32_t* __restrict__ state,
    const bf16_t* __restrict__ q, const int32_t* __restrict__ kind, char* __restrict__ ws) {
  __shared__ __attribute__((aligned(16))) char lds[NBUF][TILE_LDS];
  __shared__ __attribute__((aligned(16))) float xs[NW][16][64];  // partial S^T exchange
  const int sp = blockIdx.x;
  const int b = blockIdx.y;
  if (kind[b] < 0) return;
  MlaSlice sl;
  int per, nsp;
  mla_split(a, state, kind, b, &sl, &per, &nsp);
  if (sp >= nsp) return;  // uniform over the block
  const int r0 = sp * per;
  const int r1 = r0 + per < sl.len ? r0 + per : sl.len;
  const int ntile = (r1 - r0 + TK - 1) / TK;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int hb = wave >> 1;  // head block: heads 32 hb .. 32 hb + 31
  const int hh = wave & 1;   // key columns 288 hh .., value columns 256 hh ..
  const int half = lane >> 5;
  const bf16_t* kseq = ck + (static_cast<int64_t>(b) * a.slots + sl.start + r0) * DQK;

  // Q^T (this wave's key-column half) as the B operand of S^T = K Q^T:
  // column = head 32 hb + lane % 32, k-slots d = 288 hh + 16 ks + 8 half + j.
  bf16x8_t qop[18];
  {
    const bf16_t* qp =
        q + (static_cast<int64_t>(b) * HQ + 32 * hb + (lane & 31)) * DQK + 288 * hh + 8 * half;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) qop[ks] = *reinterpret_cast<const bf16x8_t*>(qp + 16 * ks);
  }

  // Tile copy: lane chunk s = LOADS_PER_WAVE * 64 * wave + 64 i + lane of the
  // tile maps to row s / 73, chunk s % 73 (chunk 72 is padding and repeats
  // chunk 71; rows past the tile repeat its last row).
  auto issue_tile = [&](int t, int buf) {
    const int rows = (r1 - r0) - t * TK;  // rows left from this tile on (>= 1)
    const int last = (rows < TK ? rows : TK) - 1;
    const bf16_t* base = kseq + static_cast<int64_t>(t) * TK * DQK;
#pragma unroll
    for (int i = 0; i < LOADS_PER_WAVE; ++i) {
      const int s_ = (LOADS_PER_WAVE * wave + i) * 64 + lane;
      int row = s_ / RCH;
      int ch = s_ - row * RCH;
      row = row < last ? row : last;
      ch = ch < 72 ? ch : 71;
      char* dst = lds[buf] + (LOADS_PER_WAVE * wave + i) * 1024;
      __builtin_amdgcn_global_load_lds(
          (const void*)(base + row * DQK + 8 * ch),
          (__attribute__((address_space(3))) void*)((__attribute__((address_space(3))) char*)dst), 16, 0,
          0);
    }
  };

  f32x16_t oacc[8];
#pragma unroll
  for (int db = 0; db < 8; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_ref = kNegInf, l_run = 0.f;
  const uint32_t one2 = 0x3f803f80u;

  // per-lane LDS offsets
  const int krow_off = (lane & 31) * RB + 16 * half + 576 * hh;
  const int G = lane >> 4, l16 = lane & 15, rr = l16 >> 2, c4 = l16 & 3;
  const int vrow_off = (4 * (G >> 1) + rr) * RB + 2 * (16 * (G & 1) + 4 * c4) + 512 * hh;

  for (int t = 0; t < NBUF - 1 && t < ntile; ++t) issue_tile(t, t);
  for (int t = 0; t < ntile; ++t) {
    // tile t must be complete: later tiles' loads may stay in flight
    if (t + 1 < ntile)
      __builtin_amdgcn_s_waitcnt(0x0f70 | (LOADS_PER_WAVE & 15) | ((LOADS_PER_WAVE >> 4) << 14));
    else
      __builtin_amdgcn_s_waitcnt(0x0f70);
    __syncthreads();
    if (t + NBUF - 1 < ntile) issue_tile(t + NBUF - 1, (t + NBUF - 1) % NBUF);
    const char* kl = lds[t % NBUF];

    // ---- this wave's half of S^T = K Q^T ----
    f32x16_t s;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 18; ++ks) {
      const bf16x8_t kop = *reinterpret_cast<const bf16x8_t*>(kl + krow_off + 32 * ks);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop, qop[ks], s, 0, 0, 0);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) xs[wave][r][lane] = s[r];
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] += xs[wave ^ 1][r][lane];
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
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32)) * a.sl;
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
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const bf16x8_t pop = __builtin_bit_cast(bf16x8_t, pw[ks]);
#pragma unroll
      for (int db = 0; db < 8; ++db) {
        const int off = vrow_off + 16 * ks * RB + 64 * db;
        const bf16x4_t lo = lds_read_tr(kl, off);
        const bf16x4_t hi = lds_read_tr(kl, off + 8 * RB);
        const bf16x8_t vop = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop, pop, oacc[db], 0, 0, 0);
      }
    }
  }

  // ---- write this range's partial (both halves hold the same m and l) ----
  const float l_tot = l_run + __shfl_xor(l_run, 32);
  const int head = 32 * hb + (lane & 31);
  char* rec = ws + ((static_cast<int64_t>(b) * a.smax + sp) * HQ + head) * kMlaRec;
  if (half == 0 && hh == 0) {
    reinterpret_cast<float*>(rec)[0] = m_ref;
    reinterpret_cast<float*>(rec)[1] = l_tot;
  }
  bf16_t* ro = reinterpret_cast<bf16_t*>(rec + 8) + 256 * hh;
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

__global__ void __launch_bounds__(256) decode_mla_merge_kernel(MlaArgs a, const int32_t* __restrict__ state,
                                                               const int32_t* __restrict__ kind,
                                                               const char* __restrict__ ws,
                                                               bf16_t* __restrict__ out,
                                                               float* __restrict__ lse) {
  const int head = blockIdx.x;
  const int b = blockIdx.y;
  if (kind[b] < 0) return;
  MlaSlice sl;
  int per, nsp;
  mla_split(a, state, kind, b, &sl, &per, &nsp);
  const char* rec0 = ws + (static_cast<int64_t>(b) * a.smax * HQ + head) * kMlaRec;
  const int64_t stride = static_cast<int64_t>(HQ) * kMlaRec;
  float mx = kNegInf;
  for (int s = 0; s < nsp; ++s) mx = fmaxf(mx, reinterpret_cast<const float*>(rec0 + s * stride)[0]);
  const float mu = mx == kNegInf ? 0.f : mx;
  float l = 0.f;
  for (int s = 0; s < nsp; ++s) {
    const float* h = reinterpret_cast<const float*>(rec0 + s * stride);
    l += fast_exp2(h[0] - mu) * h[1];
  }
  const float inv = l > 0.f ? 1.f / l : 0.f;
  for (int d = 2 * threadIdx.x; d < DV; d += 2 * blockDim.x) {
    float o0 = 0.f, o1 = 0.f;
    for (int s = 0; s < nsp; ++s) {
      const char* r = rec0 + s * stride;
      const float w = fast_exp2(reinterpret_cast<const float*>(r)[0] - mu);
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
         a.hkv == 1 && a.slots < (int64_t(1) << 31) / DQK;
}

constexpr int kMlaMaxSplits = 64;

size_t decode_mla_workspace_bytes(const DecodeArgs& a) {
  return static_cast<size_t>(a.batch) * kMlaMaxSplits * HQ * kMlaRec;
}

hipError_t launch_decode_mla(const DecodeArgs& d, const void* ck, const int32_t* state, const void* q,
                             const int32_t* kind, void* out, float* lse, void* ws, hipStream_t s) {
  MlaArgs a;
  a.batch = d.batch;
  a.k = d.k;
  a.C = d.C;
  a.max_summaries = d.max_summaries;
  a.slots = d.slots;
  a.smax = kMlaMaxSplits;
  a.sl = d.scale * kLog2e;
  int dev = 0, ncu = 256;
  if (hipGetDevice(&dev) == hipSuccess)
    hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev);
  a.n_cu = ncu > 0 ? ncu : 256;
  hipLaunchKernelGGL(decode_mla_split_kernel, dim3(kMlaMaxSplits, d.batch), dim3(512), 0, s, a,
                     static_cast<const bf16_t*>(ck), state, static_cast<const bf16_t*>(q), kind,
                     static_cast<char*>(ws));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_mla_merge_kernel, dim3(HQ, d.batch), dim3(256), 0, s, a, state, kind,
                     static_cast<const char*>(ws), static_cast<bf16_t*>(out), lse);
  return hipGetLastError();
}

}  // namespace ksa
