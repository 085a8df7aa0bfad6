// KSA decode cache maintenance: reset, per-step append and bulk fill.
//
// "Kwai Summary Attention Technical Report", Sec. 2.3.1 and Fig. 4.  The
// cache of one (sequence, kv head) is one run of slots,
//   [scratch | current chunk (k) | sliding-chunk ring (C*k) | summary buffer],
// so that every decode read is a single contiguous slice (Fig. 4a).  Text
// keys/values enter the next free current-chunk slot, right to left (4b).
// When the chunk is complete its summary's KV goes to the scratch slot (4c),
// the chunk is copied block-wise over the oldest ring chunk (4d) and the
// summary is appended to the buffer (4e).
#include "ksa_common.h"
#include "ksa_internal.h"

namespace ksa {

// Copy one K row (kw 4-byte words) and, when vd is set, one V row (vw
// words) with the 32 lanes p = 0..31 of a group: every lane loads its words
// of both rows (four per row per pass) before it stores any, so a copy
// costs one memory round trip per pass.
__device__ __forceinline__ void copy_kv_row32(uint32_t* __restrict__ kd, const uint32_t* __restrict__ ks, int kw,
                                              uint32_t* __restrict__ vd, const uint32_t* __restrict__ vs, int vw,
                                              int p) {
  const int mx = kw > vw || !vd ? kw : vw;
  for (int w0 = p; w0 < mx; w0 += 32 * 4) {
    uint32_t a[4], c[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = w0 + 32 * u;
      if (i < kw) a[u] = ks[i];
      if (vd && i < vw) c[u] = vs[i];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int i = w0 + 32 * u;
      if (i < kw) kd[i] = a[u];
      if (vd && i < vw) vd[i] = c[u];
    }
  }
}

__global__ void cache_reset_kernel(int32_t* state, int32_t batch) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    state[4 * b + 0] = 0;
    state[4 * b + 1] = 0;
    state[4 * b + 2] = 0;
    state[4 * b + 3] = 0;
  }
}

// One block per sequence.  Words are 4-byte units of a K or V row.
__global__ void __launch_bounds__(256) cache_append_kernel(CacheArgs a, int kw, int vw,
                                                           uint32_t* __restrict__ ck,
                                                           uint32_t* __restrict__ cv,
                                                           int32_t* __restrict__ state,
                                                           const uint32_t* __restrict__ k_new,
                                                           const uint32_t* __restrict__ v_new,
                                                           const int32_t* __restrict__ kind) {
  const int b = blockIdx.x;
  const int kd = kind[b];
  if (kd < 0) return;
  const int32_t m = state[4 * b + 0];
  const int32_t r = state[4 * b + 1];
  int err = 0;
  if (kd == 0 && r >= a.k) err = KSA_CACHE_ERR_CHUNK_FULL;
  if (kd != 0 && r != a.k) err = KSA_CACHE_ERR_CHUNK_NOT_FULL;
  if (kd != 0 && err == 0 && m >= a.max_summaries) err = KSA_CACHE_ERR_SUMMARY_FULL;
  __syncthreads();  // every thread has read the old state
  if (err) {
    if (threadIdx.x == 0) state[4 * b + 3] |= err;
    return;
  }
  const int64_t kslot = kw, vslot = vw;  // words per slot
  const int lane32 = threadIdx.x & 31;
  for (int h = threadIdx.x >> 5; h < a.hkv; h += blockDim.x >> 5) {  // one 32-lane group per kv head
    const int64_t seq = static_cast<int64_t>(b) * a.hkv + h;
    uint32_t* kc = ck + seq * a.slots * kslot;
    uint32_t* vc = cv ? cv + seq * a.slots * vslot : nullptr;
    const uint32_t* kn = k_new + seq * kslot;
    const uint32_t* vn = v_new ? v_new + seq * vslot : nullptr;
    if (kd == 0) {
      const int64_t slot = a.k - r;  // current chunk fills right to left
      copy_kv_row32(kc + slot * kslot, kn, kw, vc ? vc + slot * vslot : nullptr, vn, vw, lane32);
    } else {
      copy_kv_row32(kc, kn, kw, vc, vn, vw, lane32);  // scratch slot 0 (Fig. 4c)
      if (a.C > 0) {  // finished chunk over the oldest ring chunk (Fig. 4d)
        const int64_t dst = 1 + a.k + static_cast<int64_t>(m % a.C) * a.k;
        for (int p = 0; p < a.k; ++p)
          copy_kv_row32(kc + (dst + p) * kslot, kc + (1 + p) * kslot, kw,
                        vc ? vc + (dst + p) * vslot : nullptr, vc ? vc + (1 + p) * vslot : nullptr, vw, lane32);
      }
      const int64_t sdst = 1 + a.k + static_cast<int64_t>(a.C) * a.k + m;  // Fig. 4e
      copy_kv_row32(kc + sdst * kslot, kn, kw, vc ? vc + sdst * vslot : nullptr, vn, vw, lane32);
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    if (kd == 0) {
      state[4 * b + 1] = r + 1;
    } else {
      state[4 * b + 0] = m + 1;
      state[4 * b + 1] = 0;
    }
  }
}

// Source augmented row of destination slot `slot` after n text tokens were
// appended one by one (with every summary), or -1 if that slot was never
// written.  M = n / k complete chunks, rem = n % k trailing tokens.
__device__ __forceinline__ int64_t fill_source_row(int64_t slot, int64_t M, int64_t rem,
                                                   int32_t k, int32_t C) {
  if (slot == 0) return M >= 1 ? summary_row(M - 1, k) : -1;
  if (slot <= k) {
    const int64_t p = k - slot;  // token offset inside its chunk
    if (p < rem) return text_row(M * k + p, k);
    return M >= 1 ? text_row((M - 1) * k + p, k) : -1;
  }
  const int64_t ring_end = 1 + k + static_cast<int64_t>(C) * k;
  if (slot < ring_end) {
    const int64_t q = (slot - 1 - k) / k;        // ring chunk slot
    const int64_t pp = (slot - 1 - k) - q * k;   // position inside it
    if (M - 1 < q) return -1;
    const int64_t j = q + C * ((M - 1 - q) / C); // last chunk copied there
    return text_row(j * k + (k - 1 - pp), k);
  }
  const int64_t j = slot - ring_end;
  return j < M ? summary_row(j, k) : -1;
}

__global__ void __launch_bounds__(256) cache_fill_kernel(CacheArgs a, int kw, int vw, int64_t n_text,
                                                         uint32_t* __restrict__ ck,
                                                         uint32_t* __restrict__ cv,
                                                         const uint32_t* __restrict__ k_aug,
                                                         const uint32_t* __restrict__ v_aug) {
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t M = n_text / a.k;
  const int64_t rem = n_text - M * a.k;
  const int64_t L = n_text + M;
  const int64_t seq = static_cast<int64_t>(b) * a.hkv + h;
  const int64_t nwrite = 1 + a.k + static_cast<int64_t>(a.C) * a.k + M;
  // 8 slots per block, one 32-lane group each
  const int64_t slot = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  if (slot >= nwrite) return;
  const int64_t row = fill_source_row(slot, M, rem, a.k, a.C);
  if (row < 0) return;
  const int64_t src = (static_cast<int64_t>(b) * L + row) * a.hkv + h;
  copy_kv_row32(ck + (seq * a.slots + slot) * kw, k_aug + src * kw, kw,
                cv ? cv + (seq * a.slots + slot) * vw : nullptr, cv ? v_aug + src * vw : nullptr, vw,
                threadIdx.x & 31);
}

__global__ void cache_fill_state_kernel(int32_t* state, int32_t batch, int64_t n_text, int32_t k) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b < batch) {
    state[4 * b + 0] = static_cast<int32_t>(n_text / k);
    state[4 * b + 1] = static_cast<int32_t>(n_text % k);
    state[4 * b + 2] = 0;
    state[4 * b + 3] = 0;
  }
}

// Appending rows: sequence b continues at augmented row a0 = m (k+1) + r
// (its state) with the R = seg_rows[b+1] - seg_rows[b] rows packed at
// seg_rows[b].  The cache after those single appends is the one after a1 =
// a0 + R rows, i.e. state m' = a1 / (k+1), r' = a1 % (k+1); a slot whose
// source row under that state is a new row (>= a0) takes it, every other
// slot keeps its contents.  Grid x covers scratch, current, ring and the
// summary slots m .. m + max_new_summaries - 1, one 32-lane group per slot.
//
// When the segment completes chunk m, its tokens that arrived before the
// segment (current slots k - o, o < r) belong in ring chunk slot m mod C at
// position k - 1 - o, as the summary append's block copy would move them
// (Fig. 4d), unless a later chunk of the segment lands there too.  The group
// of current slot k - o moves that token before it writes the slot's new
// contents, so no other group reads or writes either slot.
//
// The new state {m', r'} is written by a second, one-thread-per-sequence
// kernel once every block has read the old one.  A segment longer than
// max_rows (the launch covers only max_new_sum summary slots), a negative
// one or a state out of range leaves the sequence untouched; the state
// kernel flags it.
__device__ __forceinline__ bool append_rows_ok(const CacheArgs& a, int64_t m, int64_t r, int64_t R,
                                               int64_t max_rows) {
  return R >= 0 && R <= max_rows && m >= 0 && m <= a.max_summaries && r >= 0 && r <= a.k;
}

__global__ void __launch_bounds__(256) cache_append_rows_kernel(CacheArgs a, int kw, int vw,
                                                                const int64_t* __restrict__ seg_rows,
                                                                int64_t max_rows, int64_t max_new_sum,
                                                                uint32_t* __restrict__ ck,
                                                                uint32_t* __restrict__ cv,
                                                                int32_t* __restrict__ state,
                                                                const uint32_t* __restrict__ k_rows,
                                                                const uint32_t* __restrict__ v_rows) {
  const int h = blockIdx.y;
  const int b = blockIdx.z;
  const int64_t m = state[4 * b + 0], r = state[4 * b + 1];
  const int64_t a0 = m * (a.k + 1) + r;
  const int64_t R = seg_rows[b + 1] - seg_rows[b];
  const int64_t a1 = a0 + R;
  const int64_t m1 = a1 / (a.k + 1), r1 = a1 - m1 * (a.k + 1);
  if (R == 0 || !append_rows_ok(a, m, r, R, max_rows)) return;  // uniform over the sequence's blocks
  if (m1 > a.max_summaries) return;  // flagged by the state kernel; the cache is left as it was
  const int64_t seq = static_cast<int64_t>(b) * a.hkv + h;
  const int64_t sum0 = 1 + a.k + static_cast<int64_t>(a.C) * a.k;
  const int lane32 = threadIdx.x & 31;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 8 + (threadIdx.x >> 5);
  const int64_t slot = e < sum0 ? e : m + (e - sum0) + sum0;
  if (e < sum0 + max_new_sum && !(e >= sum0 && slot >= sum0 + m1)) {
    // the pre-segment token of the completed chunk that sits in this current slot
    if (slot >= 1 && slot <= a.k && a.C > 0 && m1 > m) {
      const int64_t o = a.k - slot;
      const int64_t ring = 1 + a.k + (m % a.C) * a.k + a.k - 1 - o;
      if (o < r && fill_source_row(ring, m1, r1, a.k, a.C) < a0)
        copy_kv_row32(ck + (seq * a.slots + ring) * kw, ck + (seq * a.slots + slot) * kw, kw,
                      cv ? cv + (seq * a.slots + ring) * vw : nullptr, cv ? cv + (seq * a.slots + slot) * vw : nullptr,
                      vw, lane32);
    }
    const int64_t row = fill_source_row(slot, m1, r1, a.k, a.C);
    if (row >= a0) {  // otherwise unchanged (or never written)
      const int64_t src = (seg_rows[b] + row - a0) * a.hkv + h;
      copy_kv_row32(ck + (seq * a.slots + slot) * kw, k_rows + src * kw, kw,
                    cv ? cv + (seq * a.slots + slot) * vw : nullptr, cv ? v_rows + src * vw : nullptr, vw, lane32);
    }
  }
}

__global__ void cache_append_rows_state_kernel(CacheArgs a, int32_t* state, const int64_t* seg_rows,
                                               int64_t max_rows) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.batch) return;
  const int32_t k = a.k, max_summaries = a.max_summaries;
  const int64_t m = state[4 * b], r = state[4 * b + 1];
  const int64_t R = seg_rows[b + 1] - seg_rows[b];
  if (!append_rows_ok(a, m, r, R, max_rows)) {
    state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SEGMENT;
    return;
  }
  const int64_t a1 = m * (k + 1) + r + R;
  const int64_t m1 = a1 / (k + 1);
  if (m1 > max_summaries) {
    state[4 * b + 3] |= KSA_CACHE_ERR_SUMMARY_FULL;
    return;
  }
  state[4 * b + 0] = static_cast<int32_t>(m1);
  state[4 * b + 1] = static_cast<int32_t>(a1 - m1 * (k + 1));
}

static int words_per_row(int d, int32_t dtype) {
  return dtype == KSA_DTYPE_FP32 ? d : d / 2;
}

hipError_t launch_cache_reset(const CacheArgs& a, int32_t* state, hipStream_t s) {
  hipLaunchKernelGGL(cache_reset_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, s, state,
                     a.batch);
  return hipGetLastError();
}

hipError_t launch_cache_append(const CacheArgs& a, int32_t dtype, void* ck, void* cv,
                               int32_t* state, const void* k_new, const void* v_new,
                               const int32_t* kind, hipStream_t s) {
  const int kw = words_per_row(a.dqk, dtype);
  const int vw = words_per_row(a.dv, dtype);
  const bool has_v = !a.v_is_k_prefix;
  hipLaunchKernelGGL(cache_append_kernel, dim3(a.batch), dim3(256), 0, s, a, kw, vw,
                     static_cast<uint32_t*>(ck), has_v ? static_cast<uint32_t*>(cv) : nullptr,
                     state, static_cast<const uint32_t*>(k_new),
                     has_v ? static_cast<const uint32_t*>(v_new) : nullptr, kind);
  return hipGetLastError();
}

hipError_t launch_cache_append_rows(const CacheArgs& a, int32_t dtype, const int64_t* seg_rows, int64_t max_rows,
                                    void* ck, void* cv, int32_t* state, const void* k_rows, const void* v_rows,
                                    hipStream_t s) {
  const int kw = words_per_row(a.dqk, dtype);
  const int vw = words_per_row(a.dv, dtype);
  const bool has_v = !a.v_is_k_prefix;
  const int64_t max_new_sum = max_rows / (a.k + 1) + 1;
  const int64_t n = 1 + a.k + static_cast<int64_t>(a.C) * a.k + max_new_sum;
  hipLaunchKernelGGL(cache_append_rows_kernel, dim3(static_cast<uint32_t>((n + 7) / 8), a.hkv, a.batch),
                     dim3(256), 0, s, a, kw, vw, seg_rows, max_rows, max_new_sum, static_cast<uint32_t*>(ck),
                     has_v ? static_cast<uint32_t*>(cv) : nullptr, state, static_cast<const uint32_t*>(k_rows),
                     has_v ? static_cast<const uint32_t*>(v_rows) : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cache_append_rows_state_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, s, a, state,
                     seg_rows, max_rows);
  return hipGetLastError();
}

hipError_t launch_cache_fill(const CacheArgs& a, int32_t dtype, int64_t n_text, void* ck, void* cv,
                             int32_t* state, const void* k_aug, const void* v_aug, hipStream_t s) {
  const int kw = words_per_row(a.dqk, dtype);
  const int vw = words_per_row(a.dv, dtype);
  const bool has_v = !a.v_is_k_prefix;
  const int64_t M = n_text / a.k;
  const int64_t nwrite = 1 + a.k + static_cast<int64_t>(a.C) * a.k + M;
  const int64_t gx = (nwrite + 7) / 8;
  hipLaunchKernelGGL(cache_fill_kernel, dim3(static_cast<uint32_t>(gx), a.hkv, a.batch), dim3(256),
                     0, s, a, kw, vw, n_text, static_cast<uint32_t*>(ck),
                     has_v ? static_cast<uint32_t*>(cv) : nullptr,
                     static_cast<const uint32_t*>(k_aug),
                     has_v ? static_cast<const uint32_t*>(v_aug) : nullptr);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(cache_fill_state_kernel, dim3((a.batch + 255) / 256), dim3(256), 0, s, state,
                     a.batch, n_text, a.k);
  return hipGetLastError();
}

}  // namespace ksa
