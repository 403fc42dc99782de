/*
 * dsa.h -- C ABI of the MI355X (gfx950) DeepSeek Sparse Attention hot path.
 *
 * The operation (Keye-VL-2.0 summary page, gsyq.cn):
 *   section 一: a lightweight, MQA-shared "Lightning Indexer" scans every position and
 *     scores which ones deserve attention (one indexer key per token, shared by all
 *     indexer heads);
 *   section 一 and the second Q&A: every current token keeps the 2048 most relevant positions
 *     of its context, so attention costs O(Lk) instead of O(L^2);
 *   section 一: attention then runs only among the kept positions, on a GQA base model;
 *   section 一: prefill and decode costs are quoted against standard full attention;
 *   section 八: the selection is deterministic.
 *
 * Readings fixed by this library where the pages are silent:
 *   score  I[t,s] = sum_h w[t,h] * max(0, q_I[t,h,:] . k_I[s,:])  for keys s <= t of t's own
 *     sequence (the token sees itself); fp32, exact for integer-valued inputs;
 *   selection: the first min(k, t+1) keys in the order (score descending, index ascending),
 *     written in ascending index order, -1 padded; index = position within the sequence;
 *   attention: one index set per token shared by all query heads; query head h reads KV
 *     head h / (q_heads / kv_heads); softmax scale given; fp32 softmax, bf16 output (RNE).
 *
 * Conventions for every entry point:
 *   - all tensor pointers are DEVICE pointers, row-major and contiguous, 16-byte aligned,
 *     owned by the caller; the library never allocates or frees device memory;
 *   - `stream` is a hipStream_t (NULL = the default stream); every call only enqueues work on
 *     it and returns without synchronising; nothing is copied between host and device;
 *   - bf16 tensors are uint16 bit patterns; fp8 tensors are OCP E4M3 ("e4m3fn") codes;
 *   - a prefill batch with total_tokens == 0 is valid and does nothing (tensor pointers may
 *     then be NULL);
 *   - return DSA_OK (0) or a positive dsa_status.  Argument checks happen on the host
 *     before anything is enqueued; on error nothing is enqueued.  Contents of device arrays
 *     (cu_seqlens, cache_lens) are the caller's contract and are not checked;
 *   - identical inputs give bit-identical outputs (no float atomics anywhere);
 *   - the library keeps no mutable global state (except the device scratch array of
 *     dsa_decode_noalloc, below); calls on different streams may overlap as long as they do
 *     not share output or workspace buffers.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum dsa_status {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARGUMENT = 1,   /* null pointer, bad size, inconsistent shape */
  DSA_ERR_UNSUPPORTED = 2,        /* valid but not compiled (e.g. head_dim != 128), or past a size
                                     limit: calls that run attention address K/V rows with 32-bit
                                     byte offsets, so total_tokens (prefill) or cache_capacity
                                     (decode) x Hkv x head_dim x 2 bytes must stay below 4 GiB */
  DSA_ERR_WORKSPACE_TOO_SMALL = 3,
  DSA_ERR_HIP = 4,                /* a HIP launch failed; see dsa_last_hip_error() */
  DSA_ERR_SCRATCH_TOO_SMALL = 5   /* dsa_decode_noalloc: the shape needs more than its scratch */
};

enum dsa_idx_dtype { DSA_IDX_BF16 = 0, DSA_IDX_FP8_E4M3 = 1 };

/* One packed prefill batch of num_seqs causal sequences (block-diagonal causal mask). */
typedef struct dsa_prefill_shape {
  int32_t num_seqs;           /* B >= 1 */
  const int32_t* cu_seqlens;  /* DEVICE int32 [B+1]: 0 = cu[0] <= cu[1] <= ... <= cu[B] = total_tokens */
  int64_t total_tokens;       /* T >= 0 */
  int32_t max_seqlen;         /* host-known bound on every sequence length (sizes the grids) */
  int32_t topk;               /* k: 1..4096 */
  int32_t idx_heads;          /* H_I: multiple of 16, 16..64 */
  int32_t idx_dim;            /* d_I: 64 or 128 (fp8 needs 128) */
  int32_t idx_dtype;          /* enum dsa_idx_dtype */
  int32_t q_heads;            /* Hq */
  int32_t kv_heads;           /* Hkv: 1..8, Hq % Hkv == 0, Hq / Hkv <= 16 */
  int32_t head_dim;           /* d: 128 */
  float softmax_scale;        /* > 0, e.g. 1/sqrt(d) */
} dsa_prefill_shape;

/* A batch of decode sequences, each with its own cache of `cache_capacity` rows. */
typedef struct dsa_decode_shape {
  int32_t batch;              /* B >= 1 */
  int32_t cache_capacity;     /* rows per sequence in every cache */
  const int32_t* cache_lens;  /* DEVICE int32 [B]: valid rows, the newest token included, 1..capacity */
  int32_t max_cache_len;      /* host-known bound on cache_lens (<= cache_capacity) */
  int32_t topk, idx_heads, idx_dim, idx_dtype, q_heads, kv_heads, head_dim;  /* as for prefill */
  float softmax_scale;
} dsa_decode_shape;

/* Text of a status code (static storage). */
const char* dsa_status_string(int status);
/* hipError_t of the last DSA_ERR_HIP returned on the calling thread (0 if none). */
int dsa_last_hip_error(void);

/* ---------------------------------------------------------------------------------------
 * Prefill
 * ------------------------------------------------------------------------------------- */

/* Workspace bytes needed by dsa_index_scores / dsa_index_topk / dsa_prefill /
 * dense_causal_attention for `shape`.  cu_seqlens_host (HOST int32 [B+1], nullable) gives the
 * exact size; without it a bound from total_tokens, num_seqs and max_seqlen is returned.
 * The workspace holds the causal indexer score triangle (fp32, in 16-row blocks), a work
 * schedule, for dsa_prefill with topk_idx == NULL the index array, the gather's row order,
 * and for dense_causal_attention an fp16 copy of V (T * Hkv * 128 halves). */
int dsa_prefill_workspace_size(const dsa_prefill_shape* shape, const int32_t* cu_seqlens_host,
                               size_t* bytes);

/* Debug/verification export of the Lightning Indexer scores (summary page section 一).
 * q_idx [T, H_I, d_I], k_idx [T, d_I] (bf16 or fp8 per idx_dtype), w_idx fp32 [T, H_I].
 * scores fp32 [T, max_seqlen]: row t holds I[t, s] for s = 0..i (i = t's position in its
 * sequence) and -inf for s > i. */
int dsa_index_scores(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                     const float* w_idx, float* scores, void* workspace, size_t workspace_bytes,
                     void* stream);

/* Lightning Indexer + per-token top-k (summary page sections 一 and 八).
 * topk_idx int32 [T, k]: the min(k, i+1) selected positions of each token, ascending,
 * then -1. */
int dsa_index_topk(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                   const float* w_idx, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                   void* stream);

/* Sparse GQA attention over given index sets (summary page section 一: attention only among
 * the selected positions).  q bf16 [T, Hq, d], k/v bf16 [T, Hkv, d], topk_idx int32 [T, k]
 * as produced by dsa_index_topk (entries < 0 are ignored; valid entries must be in
 * 0..i); out bf16 [T, Hq, d].  No workspace. */
int dsa_sparse_attention(const dsa_prefill_shape* shape, const uint16_t* q, const uint16_t* k,
                         const uint16_t* v, const int32_t* topk_idx, uint16_t* out, void* stream);

/* The whole prefill hot path (summary page section 一: the indexer scores every causal pair,
 * each token keeps its 2048 most relevant positions, and attention runs only among them; the
 * prefill cost is quoted against full attention): dsa_index_topk then dsa_sparse_attention.
 * Arguments as those two calls take them; out bf16 [T, Hq, d].  topk_idx may be
 * NULL (the workspace then holds the indices).  Between the two, the rows are ordered by the
 * key block most of their selection falls in, and the attention takes them in that order
 * (better cache reuse; the results are those of the natural order, bit for bit). */
int dsa_prefill(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                const float* w_idx, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                uint16_t* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                void* stream);

/* Number of timing events dsa_prefill_timed and dsa_prefill_dedup record: 3 + 2 n, where n is
 * the number of indexer chunks (the indexer scores 512 blocks of 16 query rows at a time -- the
 * next 256 longest blocks of the schedule and 256 from its short end -- into a reusable buffer
 * of 512 x 16 x max_seqlen scores, and the top-k selects each chunk's rows before the next chunk
 * reuses it). */
int dsa_prefill_timing_events(const dsa_prefill_shape* shape, int32_t* count);

/* dsa_prefill that also records caller-created hipEvent_t events on `stream` (count from
 * dsa_prefill_timing_events): events[0] after the work schedule; for chunk c, events[1 + 2c]
 * after its indexer scores and events[2 + 2c] after its top-k; events[1 + 2n] after the row
 * ordering, events[2 + 2n] after the attention (per-stage timing). */
int dsa_prefill_timed(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                      const float* w_idx, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                      void* stream, void* const* events);

/* ---------------------------------------------------------------------------------------
 * Adjacent-query dedup (summary page section 八: the top-k sets of adjacent queries overlap,
 * so each block of 16 adjacent rows attends over the union of its rows' sets once, with a
 * per-(row, key) mask).  Same results as dsa_sparse_attention / dsa_prefill up to the order of
 * fp32 sums; fastest when adjacent rows' selections overlap.  Needs Hq/Hkv in {2, 4, 8, 16}
 * (DSA_ERR_UNSUPPORTED otherwise).  A separate "dedup workspace" (DEVICE, 16-byte aligned)
 * holds the block schedule, the unions (about T * k * 6 bytes) and an fp16 copy of V
 * (T * Hkv * 256 bytes).
 * ------------------------------------------------------------------------------------- */

/* Dedup workspace bytes for this shape (host only). */
int dsa_dedup_workspace_size(const dsa_prefill_shape* shape, size_t* bytes);

/* dsa_sparse_attention through the union of each 16-row block's index sets. */
int dsa_sparse_attention_dedup(const dsa_prefill_shape* shape, const uint16_t* q, const uint16_t* k,
                               const uint16_t* v, const int32_t* topk_idx, uint16_t* out,
                               void* dedup_workspace, size_t dedup_workspace_bytes, void* stream);

/* dsa_prefill whose attention stage runs through the unions.  events (nullable): as
 * dsa_prefill_timed, caller-created hipEvent_t recorded after each stage as there. */
int dsa_prefill_dedup(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                      const float* w_idx, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      uint16_t* out, int32_t* topk_idx, void* workspace, size_t workspace_bytes,
                      void* dedup_workspace, size_t dedup_workspace_bytes, void* stream,
                      void* const* events);

/* ---------------------------------------------------------------------------------------
 * Indexer dense warm-up objective (summary page section 一: with the full attention frozen, the
 * indexer is trained so that its distribution follows the full attention's, minimising a KL
 * divergence).  Per query token t over its keys s <= t:
 *   p_t = mean over the Hq heads of softmax_s(scale q[t,h] . k[s, g(h)])  (target, constant)
 *   r_t = softmax_s(I[t, :]) with I the Lightning Indexer scores (as dsa_index_scores)
 *   kl[t] = sum_s p log(p / r)
 * and the gradients of sum_t kl[t] with respect to the indexer inputs, with g = r - p and
 * c = q_I[t,h] . k_I[s]:  dw[t,h] = sum_s g max(0, c);  dq_I[t,h] = w[t,h] sum_s g [c>0] k_I[s];
 * dk_I[s] = sum_{t>=s} sum_h g w[t,h] [c>0] q_I[t,h].
 * Inputs as dsa_prefill (q, k bf16; V is not used); indexer e4m3 with d_I = 128 and
 * H_I in {16, 32, 64}; Hkv in {1, 2, 4} (DSA_ERR_UNSUPPORTED otherwise).
 * Outputs (DEVICE fp32): kl [T], dq_idx [T, H_I, d_I], dk_idx [T, d_I], dw_idx [T, H_I].
 * Deterministic (no float atomics).  Workspace: dsa_indexer_kl_workspace_size.
 * ------------------------------------------------------------------------------------- */
int dsa_indexer_kl_workspace_size(const dsa_prefill_shape* shape, size_t* bytes);
int dsa_indexer_kl(const dsa_prefill_shape* shape, const void* q_idx, const void* k_idx,
                   const float* w_idx, const uint16_t* q, const uint16_t* k, float* kl,
                   float* dq_idx, float* dk_idx, float* dw_idx, void* workspace,
                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Sparse attention backward (summary page section 一: the "sparse adaptation" stage trains the
 * whole model in sparse mode, which needs this attention's gradients).  With P = softmax over
 * the selected keys of scale q.k, O = P V, upstream gradient dO and D = rowsum(dO * O):
 *   dS = P (dO . v - D);  dq = scale sum_s dS k[s];  dk[s] = scale sum_{(t,h) selecting s} dS q;
 *   dv[s] = sum_{(t,h) selecting s} P dO.
 * Deterministic: no float atomics; every key's sums run over its rows in a fixed order.
 * Needs Hq/Hkv in {2, 4, 8, 16} (DSA_ERR_UNSUPPORTED otherwise).
 * ------------------------------------------------------------------------------------- */

/* dsa_sparse_attention that also writes lse (DEVICE fp32 [T, Hq]): the natural-log
 * log-sum-exp of each row's scaled scores over its selected keys (the backward's statistics). */
int dsa_sparse_attention_fwd_lse(const dsa_prefill_shape* shape, const uint16_t* q, const uint16_t* k,
                                 const uint16_t* v, const int32_t* topk_idx, uint16_t* out,
                                 float* lse, void* stream);

/* Workspace bytes for dsa_sparse_attention_bwd (host only). */
int dsa_sparse_attention_bwd_workspace_size(const dsa_prefill_shape* shape, size_t* bytes);

/* Gradients of sum <d_out, O> with respect to q, k and v.  q, k, v, topk_idx as given to the
 * forward; out and lse from dsa_sparse_attention_fwd_lse; d_out bf16 [T, Hq, d].  Outputs
 * (DEVICE fp32): dq [T, Hq, d], dk [T, Hkv, d], dv [T, Hkv, d]. */
int dsa_sparse_attention_bwd(const dsa_prefill_shape* shape, const uint16_t* q, const uint16_t* k,
                             const uint16_t* v, const int32_t* topk_idx, const uint16_t* out,
                             const float* lse, const uint16_t* d_out, float* dq, float* dk,
                             float* dv, void* workspace, size_t workspace_bytes, void* stream);

/* Standard full causal GQA attention (the cost reference of summary page section 一), same
 * tensors as dsa_sparse_attention without indices.  Uses the prefill workspace. */
int dense_causal_attention(const dsa_prefill_shape* shape, const uint16_t* q, const uint16_t* k,
                           const uint16_t* v, uint16_t* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Decode
 * ------------------------------------------------------------------------------------- */

/* Workspace bytes for dsa_decode / dense_decode_attention. */
int dsa_decode_workspace_size(const dsa_decode_shape* shape, size_t* bytes);

/* Append one token per sequence to the caches and count it: with n = cache_lens[b] (DEVICE
 * int32 [B], in/out), row n of each cache receives the token and cache_lens[b] becomes n + 1.
 * k_idx_new [B, d_I] -> k_idx_cache [B, cap, d_I]; k_new/v_new bf16 [B, Hkv, d] ->
 * k_cache/v_cache bf16 [B, cap, Hkv, d].  A sequence whose cache is full (n >= cap) is left
 * unchanged, lengths included, so the caller detects it by reading cache_lens back.
 * cache_lens is normally the same buffer as shape->cache_lens; the shape's max_cache_len is
 * not read here, so the caller raises it for the following dsa_decode. */
int dsa_kv_append(const dsa_decode_shape* shape, const void* k_idx_new, const uint16_t* k_new,
                  const uint16_t* v_new, int32_t* cache_lens, void* k_idx_cache,
                  uint16_t* k_cache, uint16_t* v_cache, void* stream);

/* One DSA decode step (summary page sections 一 and 八): for each sequence b the newest token
 * (cache row cache_lens[b]-1, already appended) scores cache rows 0..n-1 with the indexer,
 * keeps the top-k and attends over them.  q_idx [B, H_I, d_I], w_idx fp32 [B, H_I],
 * q bf16 [B, Hq, d]; out bf16 [B, Hq, d]; topk_idx int32 [B, k] (nullable).
 * max_cache_len up to 2^20 rows and cache_capacity x Hkv x head_dim x 2 bytes below 4 GiB
 * (DSA_ERR_UNSUPPORTED beyond). */
int dsa_decode(const dsa_decode_shape* shape, const void* q_idx, const float* w_idx,
               const uint16_t* q, const void* k_idx_cache, const uint16_t* k_cache,
               const uint16_t* v_cache, uint16_t* out, int32_t* topk_idx, void* workspace,
               size_t workspace_bytes, void* stream);

/* dsa_decode that also records caller-created hipEvent_t events[0..2] on `stream` after the
 * indexer, the top-k and the attention kernels (per-stage timing). */
int dsa_decode_timed(const dsa_decode_shape* shape, const void* q_idx, const float* w_idx,
                     const uint16_t* q, const void* k_idx_cache, const uint16_t* k_cache,
                     const uint16_t* v_cache, uint16_t* out, int32_t* topk_idx, void* workspace,
                     size_t workspace_bytes, void* stream, void* const* events);

/* Bytes of the device scratch array behind dsa_decode_noalloc (one array per GPU). */
#define DSA_DECODE_NOALLOC_SCRATCH_BYTES (64u << 20)

/* dsa_decode without a workspace argument, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid allocation).
 * Same arguments, results and error checks as dsa_decode; the workspace is instead a
 * file-scope device array of DSA_DECODE_NOALLOC_SCRATCH_BYTES that every GPU the library runs
 * on holds until the process ends.  Its address on the current device is looked up on the
 * first call on that device (hipGetSymbolAddress); nothing is allocated or freed, ever.
 * `stream` must belong to the current device.  A shape whose dsa_decode_workspace_size exceeds
 * the scratch returns DSA_ERR_SCRATCH_TOO_SMALL before anything is enqueued (16 sequences of
 * 131136 cached rows with k = 2048 fit).  All calls on one GPU share its scratch: calls that
 * overlap in time on one GPU (different streams or threads without ordering) race and must
 * not be made; calls ordered on one stream are fine.  The decode kernels write every scratch
 * byte they read within the call, so nothing carries over from the previous call. */
int dsa_decode_noalloc(const dsa_decode_shape* shape, const void* q_idx, const float* w_idx,
                       const uint16_t* q, const void* k_idx_cache, const uint16_t* k_cache,
                       const uint16_t* v_cache, uint16_t* out, int32_t* topk_idx, void* stream);

/* Full attention of the newest token over its whole cache (decode cost reference). */
int dense_decode_attention(const dsa_decode_shape* shape, const uint16_t* q,
                           const uint16_t* k_cache, const uint16_t* v_cache, uint16_t* out,
                           void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------------------------
 * Standalone deterministic top-k
 * ------------------------------------------------------------------------------------- */

/* The deterministic replacement of torch.topk in the DSA selection (summary page section 八),
 * as an op over arbitrary float32 rows.  Row r of scores (DEVICE fp32) starts at
 * scores + r*ld and holds n candidates, or its first row_lens[r] (DEVICE int32 [rows],
 * nullable; clamped to [0, n]).  NaN (any payload) and -inf are never selected; +0 and -0 are
 * equal.  out (DEVICE int32 [rows, k]) receives the first min(k, #selectable) positions in
 * the order (score descending, index ascending), written in ascending position order and
 * padded with -1.  Deterministic (no float atomics), no workspace, enqueued on `stream`.
 * rows == 0 is a no-op; n == 0 writes all -1.  Requires 1 <= k <= 2^24 and ld >= n. */
int dsa_topk(const float* scores, int64_t rows, int32_t n, int64_t ld, const int32_t* row_lens,
             int32_t k, int32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* DSA_H */
