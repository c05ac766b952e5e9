// pa_internal.h — host-side interface between the C ABI (pa_api.hip) and the
// kernel files.  Each kernel file owns its kernels and the launcher that
// starts them; launchers only enqueue work and return the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pa_device.h"

namespace pa {

// Tunables shared by the planner, the workspace sizing and the kernels.
constexpr int kThreads = 256;          // threads of a decode-only MHA workgroup (4 waves)
constexpr int kPrefillWaves = 8;       // waves of a workgroup that runs prefill-mode items
constexpr int kPrefillThreads = 64 * kPrefillWaves;
constexpr int kDecodeRows = 16;        // rows of one decode-mode item (one MFMA tile)
constexpr int kPrefillRows = 32 * kPrefillWaves;  // rows of a prefill-mode item (32 per wave)
constexpr int kXcdRun = 32;           // consecutive prefill-mode items per queue run (CUs per XCD)
constexpr int kMaxFwdSplits = 64;      // key partitions per decode row in pa_forward
constexpr int kMinChunk = 256;         // smallest key partition pa_forward makes ...
constexpr int kMinChunkWide = 512;     // ... or, for calls whose (request, KV head) pairs fill the grid, this
constexpr int kTailFraction = 4;       // the last 1 / kTailFraction of the requests ...
constexpr int kTailDivisor = 2;        // ... get decode partitions kTailDivisor times smaller
constexpr int kItemsPerWorkgroup = 4;  // decode work is cut into ~this many items per workgroup,
constexpr int kItemsPerWorkgroupWide = 2;  // or this many in decode-only calls of more than 8
                                           // rows per (request, KV head) pair
constexpr int kMaxSplits = 256;        // pa_decode_split / pa_merge_lse / mla_decode limit
constexpr int kItemInts = 12;          // int32 words of one pa_forward work item
constexpr int kFusedPlanMax = 1024;    // decode-only calls up to this many requests plan in-kernel
constexpr int kLongKeys = 100000;      // prefill-mode requests of at least this many keys ...
constexpr int kLongChunk = 32768;      // ... are cut into chunks of this many keys (a multiple of 64)
constexpr int64_t kLongBudgetBytes = 256ll << 20;  // partials of such chunks, at most

// Masks (pa_mask in include/pa.h).
constexpr int kMaskCausal = 0, kMaskFull = 1, kMaskPrefix = 2;

// End (exclusive) of the keys new token t of a request with ctx cached keys
// sees: ctx + t + 1 under the causal mask; every key under the full mask
// (the caller caps it at the key count); under the prefix mask at least the
// request's first `prefix` keys.
__device__ __forceinline__ int visible_end(int mask, int ctx, int t, int prefix) {
  const int causal = ctx + t + 1;
  if (mask == kMaskFull) return 0x7fffffff;
  return mask == kMaskPrefix ? (prefix > causal ? prefix : causal) : causal;
}

// Physical page read from a block table.  In a PA_DEBUG build an entry
// outside [0, num_pages) is recorded in *dbg (kept nonzero) and replaced by
// page 0, so the kernel only reads pages of the pool and the calling entry
// point reports PA_ERR_DEVICE_DATA; in a release build the entry is used as
// it is (device contents are the caller's contract).
__device__ __forceinline__ int checked_page(int pg, int num_pages, int32_t* dbg) {
#ifdef PA_DEBUG
  if ((unsigned)pg >= (unsigned)num_pages) {
    if (dbg) *dbg = 1;
    return 0;
  }
#else
  (void)num_pages;
  (void)dbg;
#endif
  return pg;
}

// ALiBi term of a score, in the units of the raw (unscaled) dot product:
// m_raw * f(|d|) is subtracted, with m_raw = slope / scale and f the distance
// (linear) or its square root (sqrt) between the query's and the key's
// positions.  The caller scales the result like any raw score.
__device__ __forceinline__ float alibi_term(float m_raw, int sqrt_mode, int dist) {
  const float d = (float)(dist < 0 ? -dist : dist);
  return m_raw * (sqrt_mode ? __builtin_amdgcn_sqrtf(d) : d);
}

// Folds a sink logit s (natural-log units, -inf for none) into a finished
// row whose keys gave log-sum-exp *lse (-inf if it saw no key): the sink is
// one more softmax key with a zero value.  Returns the factor the row's
// normalised output is multiplied by; *lse becomes that of keys and sink.
__device__ __forceinline__ float fold_sink(float s, float* lse) {
  const float mx = fmaxf(*lse, s);
  if (mx == kNegInf) return 1.f;
  const float wr = __expf(*lse - mx), ws = __expf(s - mx);
  *lse = mx + __logf(wr + ws);
  return wr / (wr + ws);
}

struct MhaArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* qsl;        // NULL: one query token per request (token index == request)
  void* out;
  float* lse;                // may be NULL
  float* part_o;             // partial outputs (split items)
  float* part_lse;
  const ReqPlan* req;        // pa_forward planner output
  const int32_t* pre_off;    // [B + 1] first prefill-mode item of each request
  const int32_t* dec_items;  // decode-mode items (relative to n_pre), kItemInts int32 each
  int32_t* merges;           // merge entry of each (request, KV head) pair, 4 int32 each:
                             // first slot, S | nrows << 16, q0, kvh (S <= 1: not split)
                             // (written by the kernel that plans the call)
  Control* ctrl;
  float scale;
  int32_t num_seqs;
  int32_t Hq, Hkv, G, P, max_pages;
  int32_t num_splits;        // pa_decode_split: partitions; pa_forward_chunked: chunks
  int32_t target_items;      // pa_forward decode-only calls planned in the kernel
  int32_t single_pass;       // ... 1: one item per (request, KV head) over all its keys,
                             // no plan, no split, no queue (see pa_forward)
  int32_t chunk_keys;        // pa_forward_chunked: keys per chunk
  int32_t row_blocks;        // pa_forward_chunked: row blocks of the longest request
  int32_t merge_groups;      // pa_forward's merge: groups of 4 rows of the widest split pair
  int32_t mask;              // kMaskCausal / kMaskFull / kMaskPrefix
  const int32_t* prefix_lens;  // [B], read under kMaskPrefix only
  const int32_t* cmerge;     // pa_forward: chunked requests, 4 int32 each: request,
                             // first output row among them, chunks, first partial row
  float* cpart_o;            // pa_forward: chunk partials [rows, chunks, Dv] ...
  float* cpart_lse;          // ... and their log-sum-exps
  const float* sinks;        // [Hq] sink logits or NULL (pa_forward_masked only)
  const float* alibi;        // [Hq] ALiBi slopes (kernels built with ALiBi only)
  int32_t alibi_sqrt;        // 1: square root of the distance, 0: the distance
  int32_t num_pages;         // pages in the pool (checked_page)
  int32_t* dbg;              // PA_DEBUG builds: bad block-table entry flag (else NULL)
};

struct PlanArgs {
  const int32_t* seq_lens;
  const int32_t* qsl;
  ReqPlan* req;
  int32_t* pre_off;
  int32_t* dec_items;
  int32_t* merges;
  int32_t* cmerge;           // chunked prefill-mode requests (see MhaArgs::cmerge)
  Control* ctrl;
  int32_t B, Hkv, G;
  int32_t P, max_pages;
  int32_t target_items;
  int32_t long_keys;         // prefill-mode requests of >= long_keys keys are cut (0: never)
  int32_t chunk_keys;        // ... into chunks of this many keys
  int32_t crow_budget;       // ... while their partial rows x chunks stay within this
};

struct F32Args {
  const float* q;
  const float* k_cache;
  const float* v_cache;
  const int32_t* block_table;
  const int32_t* seq_lens;
  const int32_t* qsl;        // NULL in split mode
  float* out;                // forward mode
  float* lse;
  float* part_o;             // split mode [B, Hq, S, Dv]
  float* part_lse;
  float scale;
  int32_t B, T, Hq, Hkv, G, Dqk, Dv, P, max_pages, num_splits;
  int32_t mask;                // forward mode: kMaskCausal / kMaskFull / kMaskPrefix
  const int32_t* prefix_lens;  // [B], read under kMaskPrefix only
  const float* sinks;          // forward mode: [Hq] sink logits or NULL
  const float* alibi;          // forward mode: [Hq] ALiBi slopes or NULL
  int32_t alibi_sqrt;          // 1: square root of the distance, 0: the distance
  int32_t num_pages;           // pages in the pool (checked_page)
  int32_t* dbg;                // PA_DEBUG builds: bad block-table entry flag (else NULL)
};

struct MlaArgs {
  const void* q;             // bf16 [B, Hq, 576]
  const void* kv;            // bf16 [pages, P, 576]
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* out;                 // bf16 [B, Hq, 512] (num_splits == 1)
  float* lse;
  float* part_o;             // [B, Hq, S, 512] (num_splits > 1); balanced: [max_pieces, Hq, 512]
  float* part_lse;           // [B, Hq, S]; balanced: [max_pieces, Hq]
  int32_t* merge_info;       // balanced: [B, 2] first partial slot and piece count of each request
  float scale;
  int32_t B, Hq, P, log2_page, max_pages, num_splits;
  int32_t max_pieces;        // balanced: partial slots (two per workgroup, one workgroup per CU)
  int32_t num_pages;         // pages in the pool (checked_page)
  int32_t* dbg;              // PA_DEBUG builds: bad block-table entry flag (else NULL)
};

// Workspace layout of pa_forward.
struct FwdWorkspace {
  size_t ctrl_off, req_off, pre_off, items_off, merges_off, plse_off, po_off;
  size_t cmerge_off, cpl_off, cpo_off, total;
  int64_t cap_slots;
  int32_t crow_budget;  // chunk partial rows x chunks the workspace holds (0: no chunking)
};
// target_items: the decode work of a call is cut into about this many items
// (kItemsPerWorkgroup, or kItemsPerWorkgroupWide, x the persistent grid).
// long_rows: rows x chunks of per-request chunk partials to provide for (0: none).
FwdWorkspace fwd_workspace_layout(int B, int Hkv, int D, int target_items, int64_t long_rows);

hipError_t launch_plan(const PlanArgs& a, hipStream_t s);
// bf16 MHA kernels exist for (Dqk, Dv) = (64, 64), (128, 128) and (192, 128):
// variant 0, 1, 2; mha_variant gives -1 for other pairs.
constexpr int kMhaVariants = 3;
int mha_variant(int dk, int dv);
// alibi: launch the kernels built with the ALiBi term (variants 0 and 1 only).
hipError_t launch_mha_forward(const MhaArgs& a, int variant, bool decode_only, bool alibi,
                              int grid, hipStream_t s);
hipError_t launch_mha_forward_fused(const MhaArgs& a, int variant, bool alibi, int grid,
                                    hipStream_t s);
hipError_t launch_mha_forward_merge(const MhaArgs& a, int Dv, int grid, hipStream_t s);
hipError_t launch_mha_chunk_merge(const MhaArgs& a, int Dv, int grid, hipStream_t s);
hipError_t launch_mha_split(const MhaArgs& a, int variant, hipStream_t s);
hipError_t launch_mha_chunked(const MhaArgs& a, int variant, hipStream_t s);
hipError_t mha_occupancy(int variant, bool decode_only, int* blocks_per_cu);
// Rows are ordered [token, head] with Hq heads per token; tok_end (a device
// int, may be NULL) stops the merge at token *tok_end: later rows are left
// untouched.
hipError_t launch_merge(const float* po, const float* pl, int rows, int S, int Dv, void* out,
                        bool out_bf16, float* lse, hipStream_t s, const float* sinks = nullptr,
                        int Hq = 1, const int32_t* tok_end = nullptr);
hipError_t launch_f32_forward(const F32Args& a, hipStream_t s);
hipError_t launch_f32_split(const F32Args& a, hipStream_t s);
hipError_t launch_mla_split(const MlaArgs& a, hipStream_t s);
hipError_t launch_mla_balanced(const MlaArgs& a, int grid, hipStream_t s);
hipError_t launch_mla_balanced_merge(const MlaArgs& a, hipStream_t s);

}  // namespace pa
