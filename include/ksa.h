/*
 * ksa.h - C ABI of the Kwai Summary Attention (KSA) hot path for AMD gfx950.
 *
 * Method source: "Kwai Summary Attention Technical Report" (arXiv:2604.24432).
 * The report defines:
 *   - the augmented sequence: after every k text tokens one summary token,
 *     chunk j = [t_jk .. t_jk+k-1, s_j]                     (Sec. 2.2.1, Eq. 1)
 *   - summary visibility: a summary reads only its own chunk; its position
 *     id equals the chunk's last text token's id           (Sec. 2.2.1)
 *   - text visibility: the text of chunks floor(i/k)-C .. floor(i/k) up to
 *     t_i, plus the summaries s_0 .. s_{floor(i/k)-C-1}     (Sec. 2.2.2, Eq. 2-3)
 *   - masked softmax attention over that rule               (Sec. 4.1.4, Eq. 10)
 *   - a block-sparse prefill kernel that loads only visible
 *     blocks and never builds the mask                      (Sec. 2.3)
 *   - a decode cache of three adjacent regions (current chunk | sliding
 *     chunk ring | summary buffer) read as one contiguous slice, with the
 *     lifecycle of Fig. 4b-4e                               (Sec. 2.3.1, Fig. 4)
 *
 * Readings fixed by this library where the report is silent:
 *   - a summary token also sees itself (k+1 keys);
 *   - C ("window_chunks") counts complete past chunks; the query's own chunk
 *     is always visible; chunks with negative index do not exist;
 *   - n need not be a multiple of k: the trailing partial chunk has no summary;
 *   - query head h reads key/value head h / (Hq / Hkv);
 *   - RoPE is half-split, angle = pos * theta^(-2f/rot_dim).
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers unless a comment says "host".
 *     Tensors are dense, row-major, in the layout given beside each argument.
 *   - The caller owns every buffer.  The library allocates nothing, frees
 *     nothing and does not synchronise, except ksa_cache_read_errors (which
 *     is documented as synchronous).
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch is asynchronous on that stream.
 *   - Every function returning int32_t returns a ksa_status.  Host-detectable
 *     problems (NULL pointers, bad sizes, unsupported shapes) are reported
 *     before anything is launched; ksa_last_error_message() then holds a
 *     thread-local description.  A failed launch returns KSA_STATUS_HIP_ERROR.
 *   - Outputs are fully overwritten; inputs are never modified except the
 *     in-place rotary calls and the cache state/regions.
 */
#ifndef KSA_H_
#define KSA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define KSA_API __attribute__((visibility("default")))
#else
#define KSA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  KSA_STATUS_OK = 0,
  KSA_STATUS_INVALID_ARGUMENT = 1,
  KSA_STATUS_UNSUPPORTED = 2,
  KSA_STATUS_CAPACITY = 3,
  KSA_STATUS_WORKSPACE_TOO_SMALL = 4,
  KSA_STATUS_HIP_ERROR = 5
} ksa_status;

typedef enum { KSA_DTYPE_BF16 = 0, KSA_DTYPE_FP32 = 1 } ksa_dtype;

/* Shape and rule parameters shared by every call. */
typedef struct {
  int32_t chunk_size;    /* k >= 1 (Eq. 1) */
  int32_t window_chunks; /* C >= 0 complete past chunks seen as text (Eq. 2) */
  int32_t num_q_heads;   /* Hq, a multiple of num_kv_heads */
  int32_t num_kv_heads;  /* Hkv >= 1 */
  int32_t head_dim_qk;   /* Dqk: 1..1024 generic; 128 and 576 have tuned kernels */
  int32_t head_dim_v;    /* Dv <= Dqk when v_is_k_prefix */
  int32_t v_is_k_prefix; /* 1: absorbed latent form, V = K[..., :Dv]; v pointers ignored */
  float softmax_scale;   /* > 0; Eq. 10 uses 1/sqrt(d) */
  int32_t dtype;         /* ksa_dtype of q/k/v/out/cache */
} ksa_params;

/* Decode cache of one layer.  Physical slot order of every (sequence, kv
 * head), left to right (Fig. 4a):
 *   slot 0                       scratch slot for the pending summary (Fig. 4c)
 *   slots 1 .. k                 current chunk, filled right to left (Fig. 4b)
 *   slots k+1 .. k+C*k           sliding-chunk ring, chunk j in ring slot j mod C (Fig. 4d)
 *   slots k+1+C*k ..             summary buffer, s_0, s_1, ... (Fig. 4e)
 * state[b*4 + 0] = m, committed chunks; state[b*4 + 1] = r, tokens in the
 * current chunk (0..k); state[b*4 + 2] reserved (0); state[b*4 + 3] =
 * error bits (KSA_CACHE_ERR_*).  Keys are stored
 * after RoPE. */
typedef struct {
  void* k;               /* [batch, Hkv, slots, Dqk] */
  void* v;               /* [batch, Hkv, slots, Dv]; NULL when v_is_k_prefix */
  int32_t* state;        /* [batch, 4] int32 */
  int32_t max_summaries; /* capacity of the summary buffer */
} ksa_cache;

enum {
  KSA_CACHE_ERR_CHUNK_FULL = 1,      /* text append with r == k */
  KSA_CACHE_ERR_CHUNK_NOT_FULL = 2,  /* summary append with r != k */
  KSA_CACHE_ERR_SUMMARY_FULL = 4,    /* summary append with m == max_summaries */
  KSA_CACHE_ERR_BAD_SUMMARY_READ = 8, /* summary decode without a just-committed chunk */
  KSA_CACHE_ERR_BAD_SEGMENT = 16      /* row-wise append or chunked prefill whose segment
                                         length is negative or above max_rows, or whose
                                         state {m, r} is out of range */
};

KSA_API const char* ksa_status_string(int32_t status);
KSA_API const char* ksa_last_error_message(void);

/* L = n + floor(n/k) (Eq. 1).  Returns -1 for n < 0 or k < 1. */
KSA_API int64_t ksa_augmented_len(int64_t n_text, int32_t chunk_size);

/* Half-split RoPE in place over the augmented sequence, positions by the
 * KSA rule: text t_i -> i, summary s_j -> j*k + k - 1 (Sec. 2.2.1).
 * x: [batch, L, num_heads, head_dim] in p->dtype.  Dims [rot_off,
 * rot_off+rot_dim) are rotated, rot_dim even.  Angles are formed in fp64.
 * batch == 0 or n_text == 0 is a no-op (x may then be NULL). */
KSA_API int32_t ksa_rope_augmented(const ksa_params* p, int32_t batch, int64_t n_text, void* x,
                           int32_t num_heads, int32_t head_dim, int32_t rot_off, int32_t rot_dim,
                           double theta, void* stream);

/* Same rotation with explicit positions: x [rows, num_heads, head_dim],
 * positions [rows] int64 (device).  Used for decode tokens.  rows == 0 is a
 * no-op (x and positions may then be NULL). */
KSA_API int32_t ksa_rope_positions(const ksa_params* p, int64_t rows, const int64_t* positions, void* x,
                           int32_t num_heads, int32_t head_dim, int32_t rot_off, int32_t rot_dim,
                           double theta, void* stream);

/* KSA prefill attention (Eq. 10 with the Eq. 1-3 rule), block-sparse:
 * visible key tiles are enumerated from the chunk indices; no mask exists.
 * Rows are in Eq. 1 order: row j*(k+1)+o is t_{jk+o} for o < k and s_j for
 * o == k; the trailing n%k rows are text with no summary.
 *   q   [batch, L, Hq,  Dqk]
 *   k   [batch, L, Hkv, Dqk]
 *   v   [batch, L, Hkv, Dv ]   (ignored when v_is_k_prefix)
 *   out [batch, L, Hq,  Dv ]
 *   lse [batch, Hq, L] fp32 natural-log normaliser, or NULL.
 * bf16 with Dqk = Dv = 128 runs the MFMA kernel; other shapes the generic one. */
KSA_API int32_t ksa_prefill_attn(const ksa_params* p, int32_t batch, int64_t n_text, const void* q,
                         const void* k, const void* v, void* out, float* lse, void* stream);

/* ksa_prefill_attn with the query's rotary embedding applied as the kernel
 * loads each query row (Sec. 2.2.1: a text token's position id is its text
 * index, a summary token's is that of its chunk's last text token).  q holds
 * the un-rotated queries and is not written; each row is rotated half-split
 * over all Dqk columns, pair (f, f + Dqk/2) by pos * rope_theta^(-2f/Dqk)
 * radians, as ksa_rope_augmented(q, rot_off 0, rot_dim Dqk, rope_theta)
 * would store it (rotation in fp32 or better, rounded to the dtype).  k must
 * already be rotated: the cache keeps post-RoPE keys (Sec. 2.3.1), so the
 * keys' pass stays separate.  Same shapes, kernels and errors as
 * ksa_prefill_attn, plus: rope_theta not positive and finite, or Dqk odd,
 * is KSA_STATUS_INVALID_ARGUMENT; v_is_k_prefix (whose rotary part is a
 * column block, not the whole head) is KSA_STATUS_UNSUPPORTED. */
KSA_API int32_t ksa_prefill_attn_qrope(const ksa_params* p, int32_t batch, int64_t n_text, const void* q,
                               const void* k, const void* v, void* out, float* lse, double rope_theta,
                               void* stream);

/* Summary-free baselines the report compares KSA with (Fig. 3; the
 * Hybrid-SCA / Hybrid-SWA comparisons), laid over the same Eq. 1 layout so
 * that the same inputs can be timed against KSA:
 *   KSA_MODE_KSA  the KSA rule (same as ksa_prefill_attn);
 *   KSA_MODE_SCA  sliding chunk attention: text t_i (c = i / k) sees text
 *                 t_{max(0,(c-C)k)} .. t_i and no summary;
 *   KSA_MODE_SWA  token sliding window: text t_i sees text
 *                 t_{max(0,i-W+1)} .. t_i and no summary, W = window_tokens.
 * Summary rows keep the KSA rule (own chunk and itself) in every mode. */
enum { KSA_MODE_KSA = 0, KSA_MODE_SCA = 1, KSA_MODE_SWA = 2 };

/* ksa_prefill_attn with a visibility mode.  window_tokens (W >= 1) is used
 * by KSA_MODE_SWA only.  Same shapes, kernels and errors as
 * ksa_prefill_attn; an unknown mode or W < 1 with SWA is
 * KSA_STATUS_INVALID_ARGUMENT. */
KSA_API int32_t ksa_prefill_attn_mode(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch,
                              int64_t n_text, const void* q, const void* k, const void* v, void* out,
                              float* lse, void* stream);

/* Bytes of workspace ksa_prefill_attn_bwd needs for this shape (it depends
 * on the kernel the shape runs on); 0 on bad input. */
KSA_API size_t ksa_prefill_bwd_workspace_bytes(const ksa_params* p, int32_t batch, int64_t n_text);

/* Backward of ksa_prefill_attn_mode: gradients of the attention output with
 * respect to q, k and v (the report trains with its block-sparse kernel,
 * Sec. 2.3; the gradient is the chain rule through Eq. 10 over the same
 * visible pairs).  Inputs are those of the forward call plus
 *   out  [batch, L, Hq, Dv]  the forward output
 *   dout [batch, L, Hq, Dv]  gradient of the loss with respect to out
 *   lse  [batch, Hq, L] fp32 the forward's natural-log normaliser (required)
 * and outputs (every element written; dk/dv of a kv head sum its query heads)
 *   dq [batch, L, Hq, Dqk], dk [batch, L, Hkv, Dqk], dv [batch, L, Hkv, Dv]
 * in the params' dtype.  workspace (device, >= ksa_prefill_bwd_workspace_bytes)
 * holds per-row dot(dout, out) and, on the MFMA path, per-segment partial
 * gradients of the summary keys; its contents on entry do not matter.
 * v_is_k_prefix (absorbed MLA) is KSA_STATUS_UNSUPPORTED.  Rows that see no
 * key do not exist under these rules. */
KSA_API int32_t ksa_prefill_attn_bwd(const ksa_params* p, int32_t mode, int64_t window_tokens, int32_t batch,
                             int64_t n_text, const void* q, const void* k, const void* v,
                             const void* out, const void* dout, const float* lse, void* dq, void* dk,
                             void* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Slots per (sequence, kv head): 1 + k + C*k + max_summaries; -1 on bad input. */
KSA_API int64_t ksa_cache_slots(const ksa_params* p, int32_t max_summaries);

/* Empty every sequence: state := {0, 0, 0, 0}.  Regions are not cleared. */
KSA_API int32_t ksa_cache_reset(const ksa_params* p, const ksa_cache* c, int32_t batch, void* stream);

/* One decode-step cache update per sequence (Fig. 4b-4e).
 *   k_new [batch, Hkv, Dqk], v_new [batch, Hkv, Dv] (post-RoPE keys)
 *   kind  [batch] int32: 0 text token -> current-chunk slot k - r, r += 1;
 *         1 summary -> scratch slot, copy the chunk into ring slot m mod C,
 *           append at summary-buffer slot m, m += 1, r = 0;
 *         -1 skip.
 * Misuse (text into a full chunk, summary into a non-full chunk, summary
 * buffer full) leaves that sequence untouched and sets its error bit. */
KSA_API int32_t ksa_cache_append(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* k_new,
                         const void* v_new, const int32_t* kind, void* stream);

/* Bulk hand-off from prefill to decode (Sec. 2.3.1: the cache that decoding
 * reads holds the keys and values the prefill produced, in the regions of
 * Fig. 4a): the result equals appending the L augmented rows one by one
 * (text rows as kind 0, summary rows as kind 1, Fig. 4b-4e), starting from
 * an empty cache, for every sequence.  Slots that those appends would never
 * write are left as they were.
 *   k_aug [batch, L, Hkv, Dqk], v_aug [batch, L, Hkv, Dv] (post-RoPE). */
KSA_API int32_t ksa_cache_fill(const ksa_params* p, const ksa_cache* c, int32_t batch, int64_t n_text,
                       const void* k_aug, const void* v_aug, void* stream);

/* Append the next augmented rows of each sequence (chunked prefill hand-off,
 * Sec. 2.3.1): sequence b continues at row m (k+1) + r of Eq. 1 (its state)
 * with R_b = seg_rows[b+1] - seg_rows[b] rows; text rows act as kind-0
 * appends and summary rows (every (k+1)-th row) as kind-1 appends, in order,
 * and the result equals those single appends.
 *   seg_rows [batch + 1] device int64, non-decreasing packed row offsets
 *   k_rows [seg_rows[batch], Hkv, Dqk], v_rows [.., Hkv, Dv] (post-RoPE)
 *   max_rows >= every R_b (sizes the launch).
 * A sequence whose summaries would exceed max_summaries is left untouched
 * and gets KSA_CACHE_ERR_SUMMARY_FULL; one whose R_b is negative or above
 * max_rows, or whose state is out of range (r outside 0..k, m outside
 * 0..max_summaries), is left untouched and gets KSA_CACHE_ERR_BAD_SEGMENT.
 * R_b = 0 is a no-op. */
KSA_API int32_t ksa_cache_append_rows(const ksa_params* p, const ksa_cache* c, int32_t batch,
                              const int64_t* seg_rows, int64_t max_rows, const void* k_rows,
                              const void* v_rows, void* stream);

/* Chunked and variable-length (batched) prefill against the cache (the
 * serving path next to the prefill hand-off of Sec. 2.3.1).  Sequence b's
 * segment is the R_b = seg_rows[b+1] - seg_rows[b] augmented rows that
 * follow its cache state {m, r}: rows m (k+1) + r onward of Eq. 1, text and
 * summary rows interleaved as in the one-shot layout.  Every segment row
 * gets the output the one-shot ksa_prefill_attn gives that row of the whole
 * sequence (KSA rule); keys before the segment are read from the cache
 * regions (summary buffer, ring, current chunk), which hold every key a
 * segment row can see, and keys in the segment from k / v.
 *   seg_rows [batch + 1] device int64, non-decreasing, seg_rows[0] = 0
 *   q   [total_rows, Hq, Dqk]   k [total_rows, Hkv, Dqk]   v [total_rows, Hkv, Dv]
 *   out [total_rows, Hq, Dv]    lse [Hq, total_rows] fp32 natural log, or NULL
 *   max_rows >= every R_b, total_rows = seg_rows[batch].
 * The cache regions are read only; ksa_cache_append_rows with the same
 * seg_rows and k / v then moves the segment into it.  A sequence whose cache
 * state is out of range (m > max_summaries, r > k) or whose R_b is negative
 * or above max_rows is skipped (its rows are not written) and gets
 * KSA_CACHE_ERR_BAD_SEGMENT in its state's error word, the only state word
 * this call may write. */
KSA_API int32_t ksa_prefill_chunk(const ksa_params* p, const ksa_cache* c, int32_t batch,
                          const int64_t* seg_rows, int64_t max_rows, int64_t total_rows, const void* q,
                          const void* k, const void* v, void* out, float* lse, void* stream);

/* Bytes of workspace ksa_decode_attn needs for this batch and capacity. */
KSA_API size_t ksa_decode_workspace_bytes(const ksa_params* p, int32_t batch, int32_t max_summaries);

/* Split-K decode attention over one contiguous cache slice per sequence
 * (Sec. 2.3.1): text query -> [current fill | ring | s_0 .. s_{m-C-1}],
 * summary query -> [scratch | full current chunk].
 *   q    [batch, Hq, Dqk] (post-RoPE)
 *   kind [batch] int32: 0 text, 1 summary, -1 skip (outputs not written)
 *   out  [batch, Hq, Dv];  lse [batch, Hq] fp32 or NULL
 * An empty text slice yields out = 0, lse = -inf. */
KSA_API int32_t ksa_decode_attn(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* q,
                        const int32_t* kind, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream);

/* ksa_decode_attn for callers that cannot allocate (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and results, with the split partials kept in a scratch array of
 * the library instead of a caller workspace.  The array (128 MiB) is device
 * memory of the library's code object: each GPU the library runs on holds
 * its own copy from the first launch until the process ends; its address is
 * looked up on the first call on each device.  The call allocates and frees
 * nothing.  Every call on a GPU shares that GPU's copy, so calls that
 * overlap on one GPU (different streams, threads) race: serialise them.  A
 * shape whose partials exceed the array returns
 * KSA_STATUS_WORKSPACE_TOO_SMALL before anything is launched.  Arguments,
 * layouts and errors otherwise as ksa_decode_attn. */
KSA_API int32_t ksa_decode_attn_noalloc(const ksa_params* p, const ksa_cache* c, int32_t batch, const void* q,
                                const int32_t* kind, void* out, float* lse, void* stream);

/* Synchronous: copies each sequence's error bits into host_error_bits[batch]
 * (host memory) after the work queued on `stream` has finished. */
KSA_API int32_t ksa_cache_read_errors(const ksa_params* p, const ksa_cache* c, int32_t batch,
                              int32_t* host_error_bits, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* KSA_H_ */
