// Host-side launch functions of the KSA kernels.  Each returns hipSuccess or
// the launch error; argument validation happens in the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ksa.h"

namespace ksa {

struct RopeArgs {
  int32_t batch;
  int64_t rows;          // rows per batch entry
  int64_t n_text;        // augmented rule (positions == nullptr)
  int32_t chunk;         // k
  const int64_t* positions;  // explicit positions [batch*rows] or nullptr
  int32_t heads, head_dim, rot_off, rot_dim;
  double theta;
};

hipError_t launch_rope(const RopeArgs& a, void* x, int32_t dtype, hipStream_t s);

struct PrefillArgs {
  int32_t batch;
  int64_t n_text, L;
  int32_t k, C, hq, hkv, dqk, dv;
  int32_t v_is_k_prefix;
  float scale;
  int32_t mode;           // KSA_MODE_*
  int64_t window_tokens;  // W of KSA_MODE_SWA
  double rope_theta;      // > 0: q is un-rotated; each row is rotated (half-split over all Dqk
                          // columns, Sec. 2.2.1 positions) as it is loaded.  0: q is rotated.
};

// Generic prefill over a subset of augmented rows: rows_kind selects
// 0 = every row, 1 = summary rows only.
hipError_t launch_prefill_generic(const PrefillArgs& a, int32_t dtype, int rows_kind, const void* q,
                                  const void* k, const void* v, void* out, float* lse,
                                  hipStream_t s);
// bf16 MFMA prefill of all text rows, Dqk = Dv = 128.
hipError_t launch_prefill_mfma_d128(const PrefillArgs& a, const void* q, const void* k,
                                    const void* v, void* out, float* lse, hipStream_t s);
bool prefill_mfma_supported(const PrefillArgs& a, int32_t dtype);
// bf16 absorbed-MLA prefill: Hq = 128, Hkv = 1, Dqk = 576, Dv = 512 (V = K prefix).
bool prefill_mla_supported(const PrefillArgs& a, int32_t dtype);
hipError_t launch_prefill_mla(const PrefillArgs& a, const void* k, const void* q, void* out, float* lse,
                              hipStream_t s);

// Backward of the prefill.  delta[b, h, row] = dot(dout, out) in fp32.
hipError_t launch_bwd_delta(const PrefillArgs& a, int32_t dtype, const void* out, const void* dout,
                            float* delta, hipStream_t s);
// Generic dq / dk / dv kernels (wave per row), any dtype and head dims.
hipError_t launch_prefill_bwd_generic(const PrefillArgs& a, int32_t dtype, const void* q, const void* k,
                                      const void* v, const void* dout, const float* lse, const float* delta,
                                      void* dq, void* dk, void* dv, hipStream_t s);

// bf16 MFMA backward, Dqk = Dv = 128: dq kernel, dk/dv kernel, summary-key
// reduce.  part: fp32 partials of the summary keys (prefill_bwd_mfma_partial_bytes).
bool prefill_bwd_mfma_supported(const PrefillArgs& a, int32_t dtype);
size_t prefill_bwd_mfma_partial_bytes(const PrefillArgs& a);
hipError_t launch_prefill_bwd_mfma(const PrefillArgs& a, const void* q, const void* k, const void* v,
                                   const void* dout, const float* lse, const float* delta, float* part,
                                   void* dq, void* dk, void* dv, hipStream_t s);

// Chunked / varlen prefill against the cache: sequence b's segment is the
// R_b = seg_rows[b+1] - seg_rows[b] augmented rows that follow its cache
// state {m, r} (rows a0 = m (k+1) + r onward), packed at row seg_rows[b].
struct ChunkArgs {
  int32_t batch, k, C, hq, hkv, dqk, dv;
  int32_t v_is_k_prefix;
  float scale;
  int64_t slots;       // cache slots per (sequence, kv head)
  int64_t max_rows;    // >= every R_b
  int64_t total_rows;  // packed rows: the lse row stride
};
struct ChunkPtrs {
  const void* ck;  // cache K [batch, Hkv, slots, Dqk]
  const void* cv;  // cache V (nullptr when V is a K prefix)
  int32_t* state;  // read; only the error word may be written (KSA_CACHE_ERR_BAD_SEGMENT)
  const int64_t* seg_rows;
  const void* q;   // [total_rows, Hq, Dqk]
  const void* k;   // [total_rows, Hkv, Dqk]
  const void* v;   // [total_rows, Hkv, Dv] (nullptr when V is a K prefix)
  void* out;       // [total_rows, Hq, Dv]
  float* lse;      // [Hq, total_rows] or nullptr
};
hipError_t launch_prefill_chunk_generic(const ChunkArgs& a, int32_t dtype, const ChunkPtrs& p, hipStream_t s);
bool prefill_chunk_mfma_supported(const ChunkArgs& a, int32_t dtype);
hipError_t launch_prefill_chunk_mfma(const ChunkArgs& a, const ChunkPtrs& p, hipStream_t s);

struct CacheArgs {
  int32_t batch, k, C, hkv, dqk, dv;
  int32_t v_is_k_prefix;
  int64_t slots;
  int32_t max_summaries;
};

hipError_t launch_cache_reset(const CacheArgs& a, int32_t* state, hipStream_t s);
hipError_t launch_cache_append(const CacheArgs& a, int32_t dtype, void* ck, void* cv,
                               int32_t* state, const void* k_new, const void* v_new,
                               const int32_t* kind, hipStream_t s);
hipError_t launch_cache_append_rows(const CacheArgs& a, int32_t dtype, const int64_t* seg_rows, int64_t max_rows,
                                    void* ck, void* cv, int32_t* state, const void* k_rows, const void* v_rows,
                                    hipStream_t s);
hipError_t launch_cache_fill(const CacheArgs& a, int32_t dtype, int64_t n_text, void* ck, void* cv,
                             int32_t* state, const void* k_aug, const void* v_aug, hipStream_t s);

struct DecodeArgs {
  int32_t batch, k, C, hq, hkv, dqk, dv;
  int32_t v_is_k_prefix;
  int64_t slots;
  int32_t max_summaries;
  float scale;
};

size_t decode_workspace_bytes(const DecodeArgs& a);
// workspace a launch on the current device uses (<= decode_workspace_bytes)
size_t decode_workspace_bytes_used(const DecodeArgs& a, int32_t dtype);
// allocation-free decode: the size of the file-scope scratch array and its
// device address on the current device (looked up once per device)
extern const size_t kDecodeScratchBytes;
hipError_t decode_scratch(void** ptr);
// absorbed-MLA split-K decode: bf16, Hq = 128, Hkv = 1, Dqk = 576, Dv = 512
bool decode_mla_supported(const DecodeArgs& a, int32_t dtype);
size_t decode_mla_workspace_bytes(const DecodeArgs& a);
size_t decode_mla_workspace_bytes_used(const DecodeArgs& a);
hipError_t launch_decode_mla(const DecodeArgs& a, const void* ck, int32_t* state, const void* q,
                             const int32_t* kind, void* out, float* lse, void* ws, hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, int32_t dtype, const void* ck, const void* cv,
                         const int32_t* state, const void* q, const int32_t* kind, void* out,
                         float* lse, void* ws, hipStream_t s);

}  // namespace ksa
