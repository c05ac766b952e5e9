/*
 * pa.h — C ABI of the MI355X (gfx950) paged-attention engine (libpa.so).
 *
 * The engine computes causal softmax(scale * Q K^T) V for a continuous batch
 * of requests whose keys and values live in fixed-size pages of a KV cache.
 * Sources of the operations (web pages the method is described on):
 *   [TDD] "vLLM Triton Attention Backend Deep Dive"
 *   [ROC] "vLLM AMD ROCm Attention Backend Optimization"
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every pointer argument except the `pa_dims` descriptor and the stream is
 *    a DEVICE pointer owned by the caller.  The library never allocates,
 *    frees or synchronises on these calls; work is enqueued on `stream`
 *    (a hipStream_t; NULL means the null stream) and the call returns at
 *    once.  Scratch memory comes from the caller as `workspace`, sized with
 *    the matching *_workspace_size() function.  Its contents need no
 *    initialisation.  pa_forward leaves a little state in the first 256
 *    bytes of its workspace for the next call on it (queue counters left at
 *    zero and a marker that says so; a workspace without the marker is run
 *    without the counters); a caller that writes into a workspace between
 *    calls, or reuses one after a PA_ERR_HIP, must zero those 256 bytes or
 *    overwrite them as a whole.
 *  - Sizes, dtypes and capacities are checked on the host before anything is
 *    launched; a failed check returns an error code and launches nothing.
 *    A launch failure returns PA_ERR_HIP (pa_last_hip_error() gives the
 *    hipError_t).  Nothing throws across this boundary.
 *  - DEVICE CONTENTS ARE NOT CHECKED by the compute calls of libpa.so (a
 *    block-table entry outside [0, num_pages), seq_len < q_len, a
 *    non-monotone query_start_loc ...): they are undefined behaviour there.
 *    pa_validate() checks them synchronously; the debug build libpa_debug.so
 *    checks block-table entries as it reads them (see "Debug build" below).
 *  - Calls are graph-capture safe: each call is a fixed sequence of kernel
 *    launches whose grids depend only on the pa_dims capacities, never on
 *    device contents, and no call issues a memset or a host synchronisation
 *    (in libpa.so; the debug build waits for its stream after every call
 *    that reads a block table).
 *    A captured call may be replayed after the caller rewrites seq_lens,
 *    query_start_loc and block_table in place (within the capacities).
 *
 * Data layouts (row-major, element strides in brackets)
 * -----------------------------------------------------
 *  q            [T, Hq, Dqk]            T >= query_start_loc[B]; rows past
 *               query_start_loc[B] are neither read nor written
 *  k_cache      [num_pages, Hkv, P, Dqk]      key of (page, head, slot)
 *  v_cache      [num_pages, Hkv, Dv, P]       value, stored column-major per
 *               page so that consecutive slots of one column are adjacent
 *               (a layout chosen for the matrix cores: [ROC] section
 *               "ROCM_AITER_FA", bullet on the hardware-optimised cache layout)
 *  MLA latent   [num_pages, P, 576]           key = the whole row,
 *               value = its first 512 columns
 *  block_table  int32 [B, max_pages_per_seq]  logical page -> physical page;
 *               token t of request b is at page block_table[b][t / P], slot
 *               t % P.  Entries past ceil(seq_len / P) are never read.
 *  seq_lens     int32 [B]     total keys of request b INCLUDING its new tokens
 *  query_start_loc int32 [B + 1]  request b owns query rows
 *               [qsl[b], qsl[b+1]); q_len = qsl[b+1] - qsl[b] may be 0.
 *  out          [T, Hq, Dv]   same dtype as q
 *  lse          float32 [T, Hq]   natural-log log-sum-exp of the scaled
 *               scores of the row (optional: NULL skips it)
 *
 * Causality: the q_len new tokens of a request are its LAST q_len positions;
 * new token j (0-based) sees keys 0 .. seq_len - q_len + j.  The new tokens'
 * keys and values must already be written into the cache.
 * GQA: query head h reads KV head h / (Hq / Hkv).
 */
#ifndef PA_H_
#define PA_H_

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define PA_API __attribute__((visibility("default")))
#else
#define PA_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pa_status {
  PA_OK = 0,
  PA_ERR_INVALID_ARG = 1,  /* null pointer, inconsistent sizes, bad range       */
  PA_ERR_UNSUPPORTED = 2,  /* valid but not implemented (head dim, page size ...) */
  PA_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than required            */
  PA_ERR_HIP = 4,          /* a HIP call or kernel launch failed                 */
  PA_ERR_DEVICE_DATA = 5   /* device contents are invalid (pa_validate, and the  */
                           /* debug build below)                                 */
} pa_status;

/*
 * Debug build.  libpa_debug.so is this library compiled with PA_DEBUG: its
 * kernels check every block-table entry they read against [0, num_pages); an
 * entry outside it is replaced by page 0 (so nothing outside the pool is
 * read) and recorded in a per-GPU device flag.  Every call that reads a block
 * table (pa_forward, pa_forward_masked, pa_forward_noalloc, pa_decode_split,
 * pa_forward_chunked, mla_decode) then waits for its stream and returns
 * PA_ERR_DEVICE_DATA if the flag was set (its outputs are then garbage).
 * The release libpa.so does neither: block-table contents are the caller's
 * contract there (pa_validate checks them on request).
 */

typedef enum pa_dtype { PA_F32 = 0, PA_BF16 = 1 } pa_dtype;

/*
 * Which keys a new token sees (pa_forward_masked).  With c_b = seq_lens[b] -
 * q_b cached keys, new token j of request b sits at position c_b + j.
 *   PA_MASK_CAUSAL  keys 0 .. c_b + j (pa_forward)
 *   PA_MASK_FULL    every key of the request (encoder / decoder attention)
 *   PA_MASK_PREFIX  keys 0 .. max(c_b + j, prefix_lens[b] - 1), at most
 *                   seq_lens[b] - 1: the first prefix_lens[b] positions are
 *                   a bidirectional prefix (multimodal prefix attention)
 */
typedef enum pa_mask { PA_MASK_CAUSAL = 0, PA_MASK_FULL = 1, PA_MASK_PREFIX = 2 } pa_mask;

/*
 * Position bias of pa_forward_masked ([TDD] section on the backend's use
 * cases, which names "ALiBi sqrt", used by a StepFun audio model, without a
 * formula; read as ALiBi, Press et al., "Train Short, Test Long", 2022).  With
 * p the query's position and t the key's, the scaled score of query head h
 * gets
 *   PA_ALIBI_LINEAR  - alibi_slopes[h] * |p - t|
 *   PA_ALIBI_SQRT    - alibi_slopes[h] * sqrt(|p - t|)
 * before the softmax (the slopes are the caller's: ALiBi's own are the
 * geometric sequence 2^(-8 (h + 1) / Hq) for Hq a power of two).
 */
typedef enum pa_alibi { PA_ALIBI_NONE = 0, PA_ALIBI_LINEAR = 1, PA_ALIBI_SQRT = 2 } pa_alibi;

/* Shapes and host-side capacities of one call.  Capacities (max_*) size the
 * workspace and the launch grids without reading device memory. */
typedef struct pa_dims {
  int32_t num_seqs;          /* B                                              */
  int32_t num_tokens;        /* T, rows of q / out (>= query_start_loc[B])      */
  int32_t num_q_heads;       /* Hq, a multiple of num_kv_heads                 */
  int32_t num_kv_heads;      /* Hkv                                            */
  int32_t head_dim_qk;       /* Dqk                                            */
  int32_t head_dim_v;        /* Dv                                             */
  int32_t page_size;         /* P                                              */
  int32_t num_pages;         /* pages in the cache pool                        */
  int32_t max_pages_per_seq; /* block_table row stride                         */
  int32_t max_seq_len;       /* >= every seq_len                               */
  int32_t max_q_len;         /* >= every q_len                                 */
  int32_t dtype;             /* pa_dtype of q, caches and out                  */
} pa_dims;

/*
 * Bytes of workspace pa_forward needs for these dims (0 if the dims are
 * invalid).  Pure host function.
 */
PA_API size_t pa_workspace_size(const pa_dims* dims);

/*
 * pa_forward — paged causal attention over a varlen continuous batch of
 * prefill, extend and decode requests in one call ([TDD] sections
 * "Technical implementation of paged attention", "Q-block optimization",
 * "Persistent kernels and CUDA graphs"; [ROC] section "The challenge of
 * mixed inference workloads").  seq_lens and query_start_loc are turned into
 * work items (query tokens x the query heads of one KV head, over a key
 * range) on the device: by a planner kernel, or, for calls whose requests all
 * decode (max_q_len x Hq / Hkv <= 16) and number at most 1024, by the
 * persistent kernel itself.  One persistent kernel with a fixed grid runs the
 * items; decode rows whose key range was split are then merged by
 * log-sum-exp ([TDD] section "Parallel tiled softmax (3D kernel)").  A bf16
 * call whose prefill-mode items could not fill the GPU (decided from the dims:
 * at most 128 (request, KV head, 256-row block) items, max_seq_len >= 8192)
 * runs instead as the chunk partials of pa_forward_chunked plus their merge
 * ([ROC] bullet "Chunked context processing"); pa_workspace_size then
 * includes those partials.
 *
 * Supported: bf16 with (Dqk, Dv) = (64, 64), (128, 128) or (192, 128) (the
 * last is MLA's prefill / extend on the uncompressed representation, query
 * and key 128 + 64 rotary columns, value 128: [ROC] sections "Hybrid
 * processing strategy" and "Prefill/Extend (Non-Absorbed)"), P a multiple of 8
 * up to 256; fp32 with Dqk, Dv <= 256 and any P >= 1.  Requires
 * Hq % Hkv == 0.
 * Returns PA_OK, PA_ERR_INVALID_ARG, PA_ERR_UNSUPPORTED, PA_ERR_WORKSPACE or
 * PA_ERR_HIP.
 */
PA_API pa_status pa_forward(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* query_start_loc, float scale, void* out,
                     float* lse, const pa_dims* dims, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_forward_masked — pa_forward with another mask than causal and / or
 * sink tokens ([TDD] section on the backend's use cases, which names
 * encoder / decoder attention, multimodal prefix attention and sink tokens).
 * mask is a pa_mask; prefix_lens is an int32 [B] device array for
 * PA_MASK_PREFIX (any values; negative ones act as 0) and must be NULL for
 * the other masks.  sinks (nullable) is a float32 [Hq] device array of sink
 * logits: for query head h, one more softmax key with logit sinks[h] (in
 * the units of the scaled scores, natural log) and a zero value, so
 *   out = sum_t e^{s_t} v_t / (e^{sinks[h]} + sum_t e^{s_t}),
 *   lse = ln(e^{sinks[h]} + sum_t e^{s_t});  -inf means no sink.
 * alibi_mode is a pa_alibi; with PA_ALIBI_LINEAR or PA_ALIBI_SQRT,
 * alibi_slopes is a float32 [Hq] device array of per-head slopes (else it must
 * be NULL).  ALiBi needs Dqk <= 128 in bf16 (PA_ERR_UNSUPPORTED otherwise); an
 * ALiBi call always runs on the persistent kernel, also where pa_forward would
 * take the chunked route.
 * Everything else, including the workspace, is as for pa_forward, which is
 * this call with PA_MASK_CAUSAL, no sinks and no ALiBi.  Returns
 * PA_ERR_INVALID_ARG for an unknown mask or ALiBi mode, or a prefix_lens or
 * alibi_slopes that does not match it.
 */
PA_API pa_status pa_forward_masked(const void* q, const void* k_cache, const void* v_cache,
                                   const int32_t* block_table, const int32_t* seq_lens,
                                   const int32_t* query_start_loc, int32_t mask,
                                   const int32_t* prefix_lens, const float* sinks,
                                   const float* alibi_slopes, int32_t alibi_mode, float scale,
                                   void* out, float* lse, const pa_dims* dims, void* workspace,
                                   size_t workspace_bytes, void* stream);

/*
 * pa_forward_noalloc — pa_forward for callers that cannot allocate device
 * memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation.  Same arguments, results and
 * kernels as pa_forward, but the workspace is a device array inside the
 * library of pa_noalloc_max_workspace() bytes (64 MiB), one copy per GPU, held
 * until the process ends; the call itself allocates and frees nothing.
 * Returns PA_ERR_WORKSPACE when pa_workspace_size(dims) exceeds that size
 * (for instance a long-context call that pa_forward would run as chunk
 * partials of several hundred MiB).  Every call on one GPU shares that GPU's
 * array: calls that can overlap on one GPU (other streams, other threads)
 * race on it and must be serialised by the caller.  The array keeps the last
 * call's contents, which the next call needs no clearing of.
 */
PA_API pa_status pa_forward_noalloc(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, float scale, void* out,
                                    float* lse, const pa_dims* dims, void* stream);

/* Size in bytes of pa_forward_noalloc's per-GPU workspace. */
PA_API size_t pa_noalloc_max_workspace(void);

/*
 * pa_decode_split — first launch of split-KV decode ([TDD] section
 * "Parallel tiled softmax (3D kernel)"): every request has exactly one query
 * token (T == B, q is [B, Hq, Dqk]; query_start_loc is not taken).  The keys
 * of request b are cut into num_splits contiguous, page-aligned partitions of
 * P * ceil(ceil(L / P) / num_splits) keys each (L = seq_lens[b]; trailing
 * partitions may be short or empty).  Partition s yields
 *   part_out[b, h, s, :]  float32 [B, Hq, S, Dv]  softmax-normalised within
 *                         the partition (zeros if empty)
 *   part_lse[b, h, s]     float32 [B, Hq, S]      its log-sum-exp (-inf if empty)
 * num_splits in [1, 256].  Same dtype / shape support as pa_forward; a bf16
 * call also needs Hq / Hkv <= 256 (one partition runs as one work item of at
 * most 256 rows), else PA_ERR_UNSUPPORTED.  Every seq_len must be >= 1.
 */
PA_API pa_status pa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens,
                          float scale, int32_t num_splits, float* part_out,
                          float* part_lse, const pa_dims* dims, void* stream);

/*
 * pa_forward_chunked — chunked-context processing of a varlen batch ([ROC]
 * bullet "Chunked context processing"): the keys of every request are taken
 * a fixed budget of chunk_keys at a time, and each chunk yields per-row
 * partials that pa_merge_lse combines.  Chunk s of request b covers keys
 * [s * chunk_keys, (s + 1) * chunk_keys); new token j of request b (at
 * position c_b + j, c_b = seq_lens[b] - q_b, causal as in pa_forward) sees
 * the keys of the chunk below c_b + j + 1.  For output row i * Hq + h
 * (token i = query_start_loc[b] + j, query head h):
 *   part_out[i, h, s, :]  float32 [T, Hq, num_chunks, Dv]  attention over the
 *                         keys of chunk s the token sees (zeros if none)
 *   part_lse[i, h, s]     float32 [T, Hq, num_chunks]      their log-sum-exp
 *                         (-inf if none)
 * pa_merge_lse(part_out, part_lse, T * Hq, num_chunks, Dv, out, lse, PA_BF16)
 * then gives pa_forward's out and lse.  One workgroup runs each (request, KV
 * head, block of up to 256 rows, chunk), so a long context is spread over
 * num_chunks workgroups whatever its number of new tokens.
 * mask / prefix_lens as for pa_forward_masked (PA_MASK_CAUSAL and NULL for
 * causal attention): a token sees the chunk's keys below its mask's limit.
 * chunk_keys: a positive multiple of 64; num_chunks in [1, 256] with
 * chunk_keys * num_chunks >= dims->max_seq_len.  bf16 only, with the head
 * dims and page sizes of pa_forward.  Rows of requests with no new token
 * or with seq_len < q_len are not written.  Buffers are caller-owned device
 * memory; nothing is allocated.  Returns PA_OK, PA_ERR_INVALID_ARG,
 * PA_ERR_UNSUPPORTED or PA_ERR_HIP.
 */
PA_API pa_status pa_forward_chunked(const void* q, const void* k_cache, const void* v_cache,
                                    const int32_t* block_table, const int32_t* seq_lens,
                                    const int32_t* query_start_loc, float scale,
                                    int32_t chunk_keys, int32_t num_chunks, float* part_out,
                                    float* part_lse, int32_t mask, const int32_t* prefix_lens,
                                    const pa_dims* dims, void* stream);

/*
 * pa_merge_lse — second launch: log-sum-exp merge of split partials ([TDD]
 * section "Parallel tiled softmax (3D kernel)"; [ROC] bullet "Chunked context
 * processing").  For each of num_rows rows:
 *   M = max_s lse_s,  w_s = exp(lse_s - M) (0 for lse_s = -inf),
 *   out = sum_s w_s o_s / sum_s w_s,  lse = M + ln sum_s w_s;
 * a row whose partitions are all empty gives zeros and -inf.
 *   part_out float32 [num_rows, S, Dv], part_lse float32 [num_rows, S]
 *   out      [num_rows, Dv] in out_dtype (pa_dtype), lse float32 [num_rows] or NULL
 * sinks (nullable): float32 [num_q_heads] sink logits as in pa_forward_masked;
 * row r belongs to query head r % num_q_heads (rows ordered [T, Hq]) and
 * gets sinks[r % num_q_heads] folded in as one more zero-valued key.
 * num_splits in [1, 256], head_dim_v in [1, 1024].
 */
PA_API pa_status pa_merge_lse(const float* part_out, const float* part_lse, int32_t num_rows,
                       int32_t num_splits, int32_t head_dim_v, void* out, float* lse,
                       int32_t out_dtype, const float* sinks, int32_t num_q_heads,
                       void* stream);

/*
 * Bytes of workspace mla_decode needs for these dims and num_splits
 * (0 = the automatic choice mla_decode makes); 0 if the dims are invalid.
 */
PA_API size_t mla_workspace_size(const pa_dims* dims, int32_t num_splits);

/*
 * mla_decode — absorbed multi-head latent attention decode ([ROC] sections
 * "AITER MLA backend" and "Hybrid processing strategy"): one query token per
 * request; all Hq heads share one cached 576-wide latent row per token, which
 * is the key (576 columns) and, through its first 512 columns, the value.
 *   q        bf16 [B, Hq, 576]
 *   kv_cache bf16 [num_pages, P, 576]
 *   out      bf16 [B, Hq, 512];  lse float32 [B, Hq] or NULL
 * num_splits > 0: the keys of each request are split into num_splits
 * page-aligned partitions (as in pa_decode_split), one workgroup each, and
 * merged by log-sum-exp.  num_splits == 0 (the default): balanced schedule;
 * every request is cut into pieces of at most c key tiles of 32, c chosen on
 * the device from seq_lens so that all pieces run at once, one per compute
 * unit, whatever the length mix; requests in several pieces are merged by
 * log-sum-exp ([TDD] section "Parallel tiled softmax (3D kernel)").
 * Requires bf16, Hkv == 1, Dqk == 576, Dv == 512, Hq a multiple of 16 up to
 * 128, P a power of two in [8, 256], seq_len >= 1.
 */
PA_API pa_status mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                     const int32_t* seq_lens, float scale, void* out, float* lse,
                     int32_t num_splits, const pa_dims* dims, void* workspace,
                     size_t workspace_bytes, void* stream);

/*
 * pa_validate — synchronous debug check of the device contents a pa_forward
 * call would read: query_start_loc[0] == 0, non-decreasing, query_start_loc[B]
 * <= num_tokens, 0 <= q_len <= max_q_len, q_len <= seq_len <= max_seq_len,
 * ceil(seq_len / P) <= max_pages_per_seq and every used block-table entry in
 * [0, num_pages).  query_start_loc may be NULL (then every q_len is 1).
 * Returns PA_OK, PA_ERR_DEVICE_DATA (with the first bad request in
 * *bad_seq when bad_seq is not NULL), PA_ERR_INVALID_ARG or PA_ERR_HIP.
 * Copies the three index arrays to the host and waits for `stream`.
 */
PA_API pa_status pa_validate(const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, const pa_dims* dims,
                      int32_t* bad_seq, void* stream);

/*
 * pa_set_kernel_events — measurement hook.  When both events are non-NULL
 * (hipEvent_t, created by the caller), every later pa_forward, pa_decode_split
 * and mla_decode call made from THIS thread records `start` on its stream
 * immediately before launching its attention kernel and `stop` immediately
 * after it, so the caller can time that one kernel without the planner or the
 * merge.  Passing NULL for either turns the hook off.  Returns PA_OK.
 */
PA_API pa_status pa_set_kernel_events(void* start, void* stop);

/* Static, human-readable name of a status code (any integer: values that are
 * no pa_status give "unknown status"). */
PA_API const char* pa_status_string(int32_t status);

/* hipError_t of the last PA_ERR_HIP returned on this thread (0 if none). */
PA_API int32_t pa_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PA_H_ */
