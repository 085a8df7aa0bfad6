// C ABI of the KSA library: argument checks, dispatch to the kernels.
// Every entry point validates on the host before launching anything and
// returns a ksa_status; details go to a thread-local message.
#include <cmath>
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "../../include/ksa.h"
#include "ksa_internal.h"

namespace {

thread_local char g_msg[512] = "";

int32_t fail(ksa_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_msg, sizeof(g_msg), fmt, ap);
  va_end(ap);
  return st;
}

int32_t hip_status(hipError_t e, const char* where) {
  if (e == hipSuccess) return KSA_STATUS_OK;
  return fail(KSA_STATUS_HIP_ERROR, "%s: %s", where, hipGetErrorString(e));
}

int32_t check_params(const ksa_params* p) {
  if (!p) return fail(KSA_STATUS_INVALID_ARGUMENT, "params is NULL");
  if (p->chunk_size < 1) return fail(KSA_STATUS_INVALID_ARGUMENT, "chunk_size must be >= 1");
  if (p->window_chunks < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "window_chunks must be >= 0");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "head counts must be >= 1");
  if (p->num_q_heads % p->num_kv_heads)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)",
                p->num_q_heads, p->num_kv_heads);
  if (p->head_dim_qk < 1 || p->head_dim_qk > 1024 || p->head_dim_v < 1 || p->head_dim_v > 1024)
    return fail(KSA_STATUS_UNSUPPORTED, "head dims must be in [1, 1024]");
  if (p->v_is_k_prefix && p->head_dim_v > p->head_dim_qk)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "head_dim_v exceeds head_dim_qk with v_is_k_prefix");
  if (!(p->softmax_scale > 0.f)) return fail(KSA_STATUS_INVALID_ARGUMENT, "softmax_scale must be > 0");
  if (p->dtype != KSA_DTYPE_BF16 && p->dtype != KSA_DTYPE_FP32)
    return fail(KSA_STATUS_UNSUPPORTED, "dtype must be KSA_DTYPE_BF16 or KSA_DTYPE_FP32");
  if (p->dtype == KSA_DTYPE_BF16 && ((p->head_dim_qk & 1) || (p->head_dim_v & 1)))
    return fail(KSA_STATUS_UNSUPPORTED, "bf16 head dims must be even");
  return KSA_STATUS_OK;
}

int32_t check_cache(const ksa_params* p, const ksa_cache* c) {
  if (!c) return fail(KSA_STATUS_INVALID_ARGUMENT, "cache is NULL");
  if (!c->k || !c->state) return fail(KSA_STATUS_INVALID_ARGUMENT, "cache k/state is NULL");
  if (!p->v_is_k_prefix && !c->v) return fail(KSA_STATUS_INVALID_ARGUMENT, "cache v is NULL");
  if (c->max_summaries < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "max_summaries < 0");
  return KSA_STATUS_OK;
}

ksa::CacheArgs cache_args(const ksa_params* p, const ksa_cache* c, int32_t batch) {
  ksa::CacheArgs a;
  a.batch = batch;
  a.k = p->chunk_size;
  a.C = p->window_chunks;
  a.hkv = p->num_kv_heads;
  a.dqk = p->head_dim_qk;
  a.dv = p->head_dim_v;
  a.v_is_k_prefix = p->v_is_k_prefix;
  a.max_summaries = c->max_summaries;
  a.slots = 1 + static_cast<int64_t>(p->chunk_size) + static_cast<int64_t>(p->window_chunks) * p->chunk_size +
            c->max_summaries;
  return a;
}

ksa::DecodeArgs decode_args(const ksa_params* p, int32_t batch, int32_t max_summaries) {
  ksa::DecodeArgs a;
  a.batch = batch;
  a.k = p->chunk_size;
  a.C = p->window_chunks;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.dqk = p->head_dim_qk;
  a.dv = p->head_dim_v;
  a.v_is_k_prefix = p->v_is_k_prefix;
  a.max_summaries = max_summaries;
  a.slots = 1 + static_cast<int64_t>(p->chunk_size) + static_cast<int64_t>(p->window_chunks) * p->chunk_size +
            max_summaries;
  a.scale = p->softmax_scale;
  return a;
}

}  // namespace

extern "C" {

const char* ksa_status_string(int32_t s) {
  switch (s) {
    case KSA_STATUS_OK: return "ok";
    case KSA_STATUS_INVALID_ARGUMENT: return "invalid argument";
    case KSA_STATUS_UNSUPPORTED: return "unsupported";
    case KSA_STATUS_CAPACITY: return "capacity exceeded";
    case KSA_STATUS_WORKSPACE_TOO_SMALL: return "workspace too small";
    case KSA_STATUS_HIP_ERROR: return "hip error";
    default: return "unknown status";
  }
}

const char* ksa_last_error_message(void) { return g_msg; }

int64_t ksa_augmented_len(int64_t n_text, int32_t k) {
  if (n_text < 0 || k < 1) return -1;
  return n_text + n_text / k;
}

static int32_t rope_common(const ksa_params* p, ksa::RopeArgs& ra, void* x, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (ra.heads < 1 || ra.head_dim < 1) return fail(KSA_STATUS_INVALID_ARGUMENT, "bad heads/head_dim");
  if (ra.rot_dim < 2 || (ra.rot_dim & 1) || ra.rot_off < 0 || ra.rot_off + ra.rot_dim > ra.head_dim)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "rotary block [%d, %d) does not fit head_dim %d (even width)",
                ra.rot_off, ra.rot_off + ra.rot_dim, ra.head_dim);
  if (!(ra.theta > 1.0)) return fail(KSA_STATUS_INVALID_ARGUMENT, "theta must be > 1");
  g_msg[0] = 0;
  if (ra.batch == 0 || ra.rows == 0) return KSA_STATUS_OK;  // empty input: nothing to rotate
  if (!x) return fail(KSA_STATUS_INVALID_ARGUMENT, "x is NULL");
  return hip_status(ksa::launch_rope(ra, x, p->dtype, static_cast<hipStream_t>(stream)), "rope");
}

int32_t ksa_rope_augmented(const ksa_params* p, int32_t batch, int64_t n_text, void* x,
                           int32_t num_heads, int32_t head_dim, int32_t rot_off, int32_t rot_dim,
                           double theta, void* stream) {
  if (batch < 0 || n_text < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/n_text");
  if (int32_t st = check_params(p)) return st;
  ksa::RopeArgs ra;
  ra.batch = batch;
  ra.rows = ksa_augmented_len(n_text, p->chunk_size);
  ra.n_text = n_text;
  ra.chunk = p->chunk_size;
  ra.positions = nullptr;
  ra.heads = num_heads;
  ra.head_dim = head_dim;
  ra.rot_off = rot_off;
  ra.rot_dim = rot_dim;
  ra.theta = theta;
  return rope_common(p, ra, x, stream);
}

int32_t ksa_rope_positions(const ksa_params* p, int64_t rows, const int64_t* positions, void* x,
                           int32_t num_heads, int32_t head_dim, int32_t rot_off, int32_t rot_dim,
                           double theta, void* stream) {
  if (rows < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative rows");
  if (rows > 0 && !positions) return fail(KSA_STATUS_INVALID_ARGUMENT, "positions is NULL");
  if (int32_t st = check_params(p)) return st;
  ksa::RopeArgs ra;
  ra.batch = 1;
  ra.rows = rows;
  ra.n_text = 0;
  ra.chunk = p->chunk_size;
  ra.positions = positions;
  ra.heads = num_heads;
  ra.head_dim = head_dim;
  ra.rot_off = rot_off;
  ra.rot_dim = rot_dim;
  ra.theta = theta;
  return rope_common(p, ra, x, stream);
}

namespace {

int32_t check_mode(int32_t mode, int64_t window_tokens) {
  if (mode != KSA_MODE_KSA && mode != KSA_MODE_SCA && mode != KSA_MODE_SWA)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "unknown prefill mode");
  if (mode == KSA_MODE_SWA && window_tokens < 1)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "token window must be at least 1");
  return KSA_STATUS_OK;
}

ksa::PrefillArgs prefill_args(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch,
                              int64_t n_text) {
  ksa::PrefillArgs a;
  a.batch = batch;
  a.n_text = n_text;
  a.L = ksa_augmented_len(n_text, p->chunk_size);
  a.k = p->chunk_size;
  a.C = p->window_chunks;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.dqk = p->head_dim_qk;
  a.dv = p->head_dim_v;
  a.v_is_k_prefix = p->v_is_k_prefix;
  a.scale = p->softmax_scale;
  a.mode = mode;
  // a window wider than the sequence is the whole causal prefix
  a.window_tokens = mode == KSA_MODE_SWA ? (window_tokens < n_text ? window_tokens : n_text) : 0;
  a.rope_theta = 0.0;
  return a;
}

}  // namespace

namespace {

int32_t prefill_launch(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch, int64_t n_text,
                       const void* q, const void* k, const void* v, void* out, float* lse, double rope_theta,
                       void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_mode(mode, window_tokens)) return st;
  if (batch < 0 || n_text < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/n_text");
  if (n_text > (int64_t(1) << 40)) return fail(KSA_STATUS_UNSUPPORTED, "n_text too large");
  if (batch == 0 || n_text == 0) return KSA_STATUS_OK;
  if (!q || !k || !out || (!p->v_is_k_prefix && !v))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "q/k/v/out pointer is NULL");
  ksa::PrefillArgs a = prefill_args(p, mode, window_tokens, batch, n_text);
  a.rope_theta = rope_theta;
  g_msg[0] = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ksa::prefill_mfma_supported(a, p->dtype))
    return hip_status(ksa::launch_prefill_mfma_d128(a, q, k, v, out, lse, s), "prefill");
  if (ksa::prefill_mla_supported(a, p->dtype))
    return hip_status(ksa::launch_prefill_mla(a, k, q, out, lse, s), "prefill");
  return hip_status(ksa::launch_prefill_generic(a, p->dtype, 0, q, k, v, out, lse, s), "prefill");
}

}  // namespace

int32_t ksa_prefill_attn_mode(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch,
                              int64_t n_text, const void* q, const void* k, const void* v, void* out,
                              float* lse, void* stream) {
  return prefill_launch(p, mode, window_tokens, batch, n_text, q, k, v, out, lse, 0.0, stream);
}

int32_t ksa_prefill_attn_qrope(const ksa_params* p, int32_t batch, int64_t n_text, const void* q, const void* k,
                               const void* v, void* out, float* lse, double rope_theta, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (!(rope_theta > 0.0) || !std::isfinite(rope_theta))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "rope_theta must be positive and finite");
  if (p->head_dim_qk % 2) return fail(KSA_STATUS_INVALID_ARGUMENT, "head_dim_qk must be even for RoPE");
  if (p->v_is_k_prefix)
    return fail(KSA_STATUS_UNSUPPORTED, "fused query RoPE of the absorbed (v_is_k_prefix) form");
  return prefill_launch(p, KSA_MODE_KSA, 0, batch, n_text, q, k, v, out, lse, rope_theta, stream);
}

// [delta: batch * Hq * L fp32, 256-byte aligned][MFMA path: summary-key partials]
static size_t bwd_delta_bytes(const ksa::PrefillArgs& a) {
  return (static_cast<size_t>(a.batch) * a.hq * a.L * sizeof(float) + 255) / 256 * 256;
}
static size_t bwd_workspace(const ksa::PrefillArgs& a, int32_t dtype) {
  size_t n = bwd_delta_bytes(a);
  if (ksa::prefill_bwd_mfma_supported(a, dtype)) n += ksa::prefill_bwd_mfma_partial_bytes(a);
  return n;
}

size_t ksa_prefill_bwd_workspace_bytes(const ksa_params* p, int32_t batch, int64_t n_text) {
  if (check_params(p) || batch < 0 || n_text < 0 || n_text > (int64_t(1) << 40)) return 0;
  return bwd_workspace(prefill_args(p, KSA_MODE_KSA, 0, batch, n_text), p->dtype);
}

int32_t ksa_prefill_attn_bwd(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch,
                             int64_t n_text, const void* q, const void* k, const void* v, const void* out,
                             const void* dout, const float* lse, void* dq, void* dk, void* dv,
                             void* workspace, size_t workspace_bytes, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_mode(mode, window_tokens)) return st;
  if (p->v_is_k_prefix) return fail(KSA_STATUS_UNSUPPORTED, "backward of the absorbed (v_is_k_prefix) form");
  if (batch < 0 || n_text < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/n_text");
  if (n_text > (int64_t(1) << 40)) return fail(KSA_STATUS_UNSUPPORTED, "n_text too large");
  if (batch == 0 || n_text == 0) return KSA_STATUS_OK;
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "a tensor pointer is NULL");
  const ksa::PrefillArgs a = prefill_args(p, mode, window_tokens, batch, n_text);
  const size_t need = bwd_workspace(a, p->dtype);
  if (!workspace || workspace_bytes < need)
    return fail(KSA_STATUS_WORKSPACE_TOO_SMALL, "workspace needs %zu bytes, got %zu", need,
                workspace ? workspace_bytes : size_t(0));
  g_msg[0] = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  float* delta = static_cast<float*>(workspace);
  if (int32_t st = hip_status(ksa::launch_bwd_delta(a, p->dtype, out, dout, delta, s), "prefill_bwd"))
    return st;
  if (ksa::prefill_bwd_mfma_supported(a, p->dtype)) {
    float* part = reinterpret_cast<float*>(static_cast<char*>(workspace) + bwd_delta_bytes(a));
    return hip_status(ksa::launch_prefill_bwd_mfma(a, q, k, v, dout, lse, delta, part, dq, dk, dv, s),
                      "prefill_bwd");
  }
  return hip_status(ksa::launch_prefill_bwd_generic(a, p->dtype, q, k, v, dout, lse, delta, dq, dk, dv, s),
                    "prefill_bwd");
}

int32_t ksa_prefill_attn(const ksa_params* p, int32_t batch, int64_t n_text, const void* q,
                         const void* k, const void* v, void* out, float* lse, void* stream) {
  return ksa_prefill_attn_mode(p, KSA_MODE_KSA, 0, batch, n_text, q, k, v, out, lse, stream);
}

int64_t ksa_cache_slots(const ksa_params* p, int32_t max_summaries) {
  if (check_params(p) || max_summaries < 0) return -1;
  return 1 + static_cast<int64_t>(p->chunk_size) + static_cast<int64_t>(p->window_chunks) * p->chunk_size +
         max_summaries;
}

int32_t ksa_cache_reset(const ksa_params* p, const ksa_cache* c, int32_t batch, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch");
  if (batch == 0) return KSA_STATUS_OK;
  g_msg[0] = 0;
  return hip_status(ksa::launch_cache_reset(cache_args(p, c, batch), c->state,
                                            static_cast<hipStream_t>(stream)),
                    "cache_reset");
}

int32_t ksa_cache_append(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* k_new,
                         const void* v_new, const int32_t* kind, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch");
  if (batch == 0) return KSA_STATUS_OK;
  if (!k_new || !kind || (!p->v_is_k_prefix && !v_new))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "k_new/v_new/kind is NULL");
  g_msg[0] = 0;
  return hip_status(ksa::launch_cache_append(cache_args(p, c, batch), p->dtype, c->k, c->v, c->state,
                                             k_new, v_new, kind, static_cast<hipStream_t>(stream)),
                    "cache_append");
}

int32_t ksa_cache_fill(const ksa_params* p, const ksa_cache* c, int32_t batch, int64_t n_text,
                       const void* k_aug, const void* v_aug, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0 || n_text < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/n_text");
  if (n_text / p->chunk_size > c->max_summaries)
    return fail(KSA_STATUS_CAPACITY, "%lld complete chunks exceed max_summaries %d",
                static_cast<long long>(n_text / p->chunk_size), c->max_summaries);
  if (batch == 0) return KSA_STATUS_OK;
  if (n_text > 0 && (!k_aug || (!p->v_is_k_prefix && !v_aug)))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "k_aug/v_aug is NULL");
  g_msg[0] = 0;
  return hip_status(ksa::launch_cache_fill(cache_args(p, c, batch), p->dtype, n_text, c->k, c->v,
                                           c->state, k_aug, v_aug, static_cast<hipStream_t>(stream)),
                    "cache_fill");
}

int32_t ksa_cache_append_rows(const ksa_params* p, const ksa_cache* c, int32_t batch, const int64_t* seg_rows,
                              int64_t max_rows, const void* k_rows, const void* v_rows, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0 || max_rows < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/max_rows");
  if (batch == 0 || max_rows == 0) return KSA_STATUS_OK;
  if (!seg_rows || !k_rows || (!p->v_is_k_prefix && !v_rows))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "seg_rows/k_rows/v_rows is NULL");
  g_msg[0] = 0;
  return hip_status(ksa::launch_cache_append_rows(cache_args(p, c, batch), p->dtype, seg_rows, max_rows, c->k,
                                                  c->v, c->state, k_rows, v_rows,
                                                  static_cast<hipStream_t>(stream)),
                    "cache_append_rows");
}

int32_t ksa_prefill_chunk(const ksa_params* p, const ksa_cache* c, int32_t batch, const int64_t* seg_rows,
                          int64_t max_rows, int64_t total_rows, const void* q, const void* k, const void* v,
                          void* out, float* lse, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0 || max_rows < 0 || total_rows < 0)
    return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch/max_rows/total_rows");
  if (batch == 0 || max_rows == 0 || total_rows == 0) return KSA_STATUS_OK;
  if (!seg_rows || !q || !k || !out || (!p->v_is_k_prefix && !v))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "seg_rows/q/k/v/out is NULL");
  const int64_t slots = 1 + static_cast<int64_t>(p->chunk_size) +
                        static_cast<int64_t>(p->window_chunks) * p->chunk_size + c->max_summaries;
  // augmented rows of a whole sequence stay below the summary capacity's reach
  const int64_t max_seq_rows = static_cast<int64_t>(c->max_summaries + 1) * (p->chunk_size + 1);
  if (max_seq_rows + max_rows > (int64_t(1) << 30) || total_rows > (int64_t(1) << 31))
    return fail(KSA_STATUS_UNSUPPORTED, "sequence or packed rows too long");
  ksa::ChunkArgs a;
  a.batch = batch;
  a.k = p->chunk_size;
  a.C = p->window_chunks;
  a.hq = p->num_q_heads;
  a.hkv = p->num_kv_heads;
  a.dqk = p->head_dim_qk;
  a.dv = p->head_dim_v;
  a.v_is_k_prefix = p->v_is_k_prefix;
  a.scale = p->softmax_scale;
  a.slots = slots;
  a.max_rows = max_rows;
  a.total_rows = total_rows;
  ksa::ChunkPtrs ptrs{c->k, p->v_is_k_prefix ? nullptr : c->v, c->state, seg_rows, q, k,
                      p->v_is_k_prefix ? nullptr : v, out, lse};
  g_msg[0] = 0;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (ksa::prefill_chunk_mfma_supported(a, p->dtype))
    return hip_status(ksa::launch_prefill_chunk_mfma(a, ptrs, s), "prefill_chunk");
  return hip_status(ksa::launch_prefill_chunk_generic(a, p->dtype, ptrs, s), "prefill_chunk");
}

size_t ksa_decode_workspace_bytes(const ksa_params* p, int32_t batch, int32_t max_summaries) {
  if (check_params(p) || batch < 0 || max_summaries < 0) return 0;
  return ksa::decode_workspace_bytes(decode_args(p, batch, max_summaries));
}

int32_t ksa_decode_attn(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* q,
                        const int32_t* kind, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch");
  if (batch == 0) return KSA_STATUS_OK;
  if (!q || !kind || !out) return fail(KSA_STATUS_INVALID_ARGUMENT, "q/kind/out is NULL");
  const ksa::DecodeArgs a = decode_args(p, batch, c->max_summaries);
  const size_t need = ksa::decode_workspace_bytes(a);
  if (workspace_bytes < need || (need > 0 && !workspace))
    return fail(KSA_STATUS_WORKSPACE_TOO_SMALL, "decode needs %zu workspace bytes, got %zu", need,
                workspace_bytes);
  g_msg[0] = 0;
  return hip_status(ksa::launch_decode(a, p->dtype, c->k, c->v, c->state, q, kind, out, lse, workspace,
                                       static_cast<hipStream_t>(stream)),
                    "decode");
}

int32_t ksa_decode_attn_noalloc(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* q,
                                const int32_t* kind, void* out, float* lse, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0) return fail(KSA_STATUS_INVALID_ARGUMENT, "negative batch");
  if (batch == 0) return KSA_STATUS_OK;
  if (!q || !kind || !out) return fail(KSA_STATUS_INVALID_ARGUMENT, "q/kind/out is NULL");
  const ksa::DecodeArgs a = decode_args(p, batch, c->max_summaries);
  const size_t need = ksa::decode_workspace_bytes_used(a, p->dtype);
  if (need > ksa::kDecodeScratchBytes)
    return fail(KSA_STATUS_WORKSPACE_TOO_SMALL,
                "this decode needs %zu scratch bytes, above the allocation-free limit of %zu; "
                "use ksa_decode_attn with a workspace",
                need, ksa::kDecodeScratchBytes);
  void* scratch = nullptr;
  if (need > 0) {
    if (int32_t st = hip_status(ksa::decode_scratch(&scratch), "decode_noalloc scratch lookup")) return st;
  }
  g_msg[0] = 0;
  return hip_status(ksa::launch_decode(a, p->dtype, c->k, c->v, c->state, q, kind, out, lse, scratch,
                                       static_cast<hipStream_t>(stream)),
                    "decode_noalloc");
}

int32_t ksa_cache_read_errors(const ksa_params* p, const ksa_cache* c, int32_t batch,
                              int32_t* host_error_bits, void* stream) {
  if (int32_t st = check_params(p)) return st;
  if (int32_t st = check_cache(p, c)) return st;
  if (batch < 0 || (batch > 0 && !host_error_bits))
    return fail(KSA_STATUS_INVALID_ARGUMENT, "bad batch or host buffer");
  if (batch == 0) return KSA_STATUS_OK;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (int32_t st = hip_status(hipStreamSynchronize(s), "cache_read_errors")) return st;
  return hip_status(hipMemcpy2D(host_error_bits, sizeof(int32_t), c->state + 3, 4 * sizeof(int32_t),
                                sizeof(int32_t), batch, hipMemcpyDeviceToHost),
                    "cache_read_errors");
}

}  // extern "C"
