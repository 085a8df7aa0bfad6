// Chunked (and variable-length, batched) KSA prefill against the cache,
// generic path: one wavefront per (sequence, segment row, query head).
//
// A sequence that already holds m committed chunks and r current-chunk
// tokens in its cache ("Kwai Summary Attention Technical Report",
// Sec. 2.3.1, Fig. 4) continues at augmented row a0 = m (k+1) + r of
// Eq. (1).  The segment's rows see exactly what the one-shot prefill would
// give them (Eq. 3 and the summary rule); keys older than a0 are read from
// the cache regions instead of a full K/V:
//   summary s_j, j < m:  summary buffer slot j;
//   text of chunk m:     the current chunk, token o at slot k - o;
//   text of chunk c < m: ring chunk slot c mod C (token o at position k-1-o),
//                        which still holds chunk c whenever c >= m - C,
//                        i.e. whenever some row of the segment can see it;
// keys at or after a0 come from the segment itself.
#include "ksa_attend_wave.h"
#include "ksa_internal.h"

namespace ksa {

template <typename T, int NQ, int NV>
__global__ void __launch_bounds__(256) prefill_chunk_generic_kernel(ChunkArgs a, ChunkPtrs p) {
  const int lane = threadIdx.x & 63;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (wave >= static_cast<int64_t>(a.batch) * a.max_rows * a.hq) return;
  const int h = static_cast<int>(wave % a.hq);
  const int64_t brl = wave / a.hq;
  const int64_t rl = brl % a.max_rows;
  const int b = static_cast<int>(brl / a.max_rows);
  const int64_t off = p.seg_rows[b];
  const int64_t R = p.seg_rows[b + 1] - off;
  const int64_t m = p.state[4 * b], r = p.state[4 * b + 1];
  const int64_t max_sum = a.slots - 1 - a.k - static_cast<int64_t>(a.C) * a.k;
  // state out of range or segment outside 0..max_rows: skipped, and flagged
  // by one wave of the sequence
  if (m < 0 || m > max_sum || r < 0 || r > a.k || R < 0 || R > a.max_rows) {
    if (rl == 0 && h == 0 && lane == 0) p.state[4 * b + 3] |= KSA_CACHE_ERR_BAD_SEGMENT;
    return;
  }
  if (rl >= R) return;
  const int64_t a0 = m * (a.k + 1) + r;
  const int64_t t_seg = a0 - a0 / (a.k + 1);  // first text index of the segment
  const int kvh = h / (a.hq / a.hkv);
  const int64_t sum0 = 1 + a.k + static_cast<int64_t>(a.C) * a.k;
  const T* ck = static_cast<const T*>(p.ck) + (static_cast<int64_t>(b) * a.hkv + kvh) * a.slots * a.dqk;
  const T* cv = p.cv ? static_cast<const T*>(p.cv) + (static_cast<int64_t>(b) * a.hkv + kvh) * a.slots * a.dv
                     : ck;
  const int64_t cvs = p.cv ? a.dv : a.dqk;
  const T* sk = static_cast<const T*>(p.k) + kvh * a.dqk;
  const T* sv = p.v ? static_cast<const T*>(p.v) + kvh * a.dv : sk;
  const int64_t sks = static_cast<int64_t>(a.hkv) * a.dqk;
  const int64_t svs = p.v ? static_cast<int64_t>(a.hkv) * a.dv : sks;

  WaveAttnState<NQ, NV> st;
  const int64_t qrow = off + rl;
  const T* qp = static_cast<const T*>(p.q) + (qrow * a.hq + h) * a.dqk;
  wave_attn_init<T, NQ, NV>(st, qp, a.dqk, a.scale * kLog2e, lane);
  // one key by its augmented row (>= a0: segment) or cache slot
  auto seg = [&](int64_t row) {
    const int64_t sr = off + row - a0;
    wave_attn_step<T, NQ, NV>(st, sk + sr * sks, sv + sr * svs, a.dqk, a.dv, lane);
  };
  auto slot = [&](int64_t s) { wave_attn_step<T, NQ, NV>(st, ck + s * a.dqk, cv + s * cvs, a.dqk, a.dv, lane); };
  auto text_key = [&](int64_t x) {
    if (x >= t_seg) return seg(text_row(x, a.k));
    const int64_t cx = x / a.k, ox = x - cx * a.k;
    if (cx == m) return slot(a.k - ox);
    slot(1 + a.k + (a.C > 0 ? cx % a.C : 0) * a.k + (a.k - 1 - ox));  // chunk c < m needs C > 0
  };

  const int64_t row = a0 + rl;
  const int64_t c = row / (a.k + 1);
  const int64_t o = row - c * (a.k + 1);
  if (o == a.k) {  // summary s_c: its chunk's text and itself
    for (int64_t x = c * a.k; x < c * a.k + a.k; ++x) text_key(x);
    seg(row);
  } else {
    const int64_t i = c * a.k + o;
    for (int64_t j = 0; j < c - a.C; ++j) {
      if (j < m)
        slot(sum0 + j);
      else
        seg(summary_row(j, a.k));
    }
    for (int64_t x = c - a.C > 0 ? (c - a.C) * a.k : 0; x <= i; ++x) text_key(x);
  }
  T* op = static_cast<T*>(p.out) + (qrow * a.hq + h) * a.dv;
  float* lp = p.lse ? p.lse + static_cast<int64_t>(h) * a.total_rows + qrow : nullptr;
  wave_attn_finish<T, NQ, NV>(st, op, a.dv, lp, lane);
}

template <typename T, int N>
static hipError_t launch_t(const ChunkArgs& a, const ChunkPtrs& p, hipStream_t s) {
  const int64_t waves = static_cast<int64_t>(a.batch) * a.max_rows * a.hq;
  if (waves == 0) return hipSuccess;
  hipLaunchKernelGGL((prefill_chunk_generic_kernel<T, N, N>), dim3(static_cast<uint32_t>((waves + 3) / 4)),
                     dim3(256), 0, s, a, p);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_d(const ChunkArgs& a, const ChunkPtrs& p, hipStream_t s) {
  const int d = a.dqk > a.dv ? a.dqk : a.dv;
  if (d <= 64) return launch_t<T, 1>(a, p, s);
  if (d <= 128) return launch_t<T, 2>(a, p, s);
  if (d <= 256) return launch_t<T, 4>(a, p, s);
  if (d <= 576) return launch_t<T, 9>(a, p, s);
  return launch_t<T, 16>(a, p, s);
}

hipError_t launch_prefill_chunk_generic(const ChunkArgs& a, int32_t dtype, const ChunkPtrs& p, hipStream_t s) {
  if (dtype == KSA_DTYPE_FP32) return launch_d<float>(a, p, s);
  return launch_d<bf16_t>(a, p, s);
}

}  // namespace ksa
