// pa_api.hip — the C ABI declared in include/pa.h: host-side argument checks,
// workspace sizing, per-device launch configuration and the launch sequences.
// Nothing here synchronises, allocates or touches device memory except
// pa_validate, which is documented as a synchronous debug call.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <vector>

#include "pa.h"
#include "pa_internal.h"

namespace {

thread_local int32_t g_last_hip_error = 0;
thread_local hipEvent_t g_ev_start = nullptr;
thread_local hipEvent_t g_ev_stop = nullptr;

// Records the measurement hook's event (if set) on stream s.
hipError_t mark(hipEvent_t ev, hipStream_t s) {
  return (g_ev_start && g_ev_stop) ? hipEventRecord(ev, s) : hipSuccess;
}

pa_status hip_fail(hipError_t e) {
  g_last_hip_error = (int32_t)e;
  return PA_ERR_HIP;
}

struct DevCfg {
  int cu_count = 0;
  int occ[pa::kMhaVariants][2] = {};  // persistent workgroups per CU [variant][decode_only]
};

std::mutex g_mu;
std::map<int, DevCfg> g_cfg;

// Workspace of pa_forward_noalloc: a device array of the library, one copy on
// every GPU it runs on, held until the process ends.  Host code never uses
// the array's name as an address (on the host it only stands for the device
// symbol): the per-device address comes from hipGetSymbolAddress, called
// once per device with that device current.
constexpr size_t kScratchBytes = 64ull << 20;
__device__ __align__(256) char scratch[kScratchBytes];
std::map<int, void*> g_scratch;  // device -> address of its copy (under g_mu)

#ifdef PA_DEBUG
// Debug builds: one flag per GPU, set by a kernel that met a block-table entry
// outside the pool (checked_page).  It starts at zero; every call that reads
// a block table waits for its stream, reads it and clears it when set.
__device__ int32_t debug_bad_page;
std::map<int, int32_t*> g_debug;  // device -> address of its flag (under g_mu)
int32_t* debug_flag() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_debug.find(dev);
  if (it == g_debug.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(debug_bad_page)) != hipSuccess) return nullptr;
    it = g_debug.emplace(dev, (int32_t*)ptr).first;
  }
  return it->second;
}
#else
int32_t* debug_flag() { return nullptr; }
#endif

// Debug builds: after a call's launches, wait for its stream and report
// PA_ERR_DEVICE_DATA if a kernel set the flag (then cleared again; it starts
// at zero).  Release builds: nothing.
pa_status debug_end(pa_status st, hipStream_t s) {
#ifdef PA_DEBUG
  if (st != PA_OK) return st;
  int32_t* f = debug_flag();
  if (!f) return PA_ERR_HIP;
  int32_t v = 0;
  hipError_t e = hipMemcpyAsync(&v, f, sizeof(int32_t), hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e == hipSuccess && v) e = hipMemsetAsync(f, 0, sizeof(int32_t), s);  // clear for the next call
  if (e == hipSuccess && v) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  return v ? PA_ERR_DEVICE_DATA : PA_OK;
#else
  (void)s;
  return st;
#endif
}

pa_status scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_scratch.find(dev);
  if (it == g_scratch.end()) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    if (!ptr) return hip_fail(hipErrorInvalidSymbol);
    it = g_scratch.emplace(dev, ptr).first;
  }
  *out = it->second;
  return PA_OK;
}

pa_status device_config(DevCfg* out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  std::lock_guard<std::mutex> lk(g_mu);
  auto it = g_cfg.find(dev);
  if (it == g_cfg.end()) {
    DevCfg c;
    e = hipDeviceGetAttribute(&c.cu_count, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e);
    for (int di = 0; di < pa::kMhaVariants; ++di)
      for (int dd = 0; dd < 2; ++dd) {
        e = pa::mha_occupancy(di, dd != 0, &c.occ[di][dd]);
        if (e != hipSuccess) return hip_fail(e);
        if (c.occ[di][dd] < 1) c.occ[di][dd] = 1;
      }
    it = g_cfg.emplace(dev, c).first;
  }
  *out = it->second;
  return PA_OK;
}

// Shape checks common to every call.  Returns PA_OK or PA_ERR_INVALID_ARG.
pa_status check_dims(const pa_dims* d) {
  if (!d) return PA_ERR_INVALID_ARG;
  if (d->num_seqs < 0 || d->num_tokens < 0 || d->num_q_heads <= 0 || d->num_kv_heads <= 0 ||
      d->head_dim_qk <= 0 || d->head_dim_v <= 0 || d->page_size <= 0 || d->num_pages <= 0 ||
      d->max_pages_per_seq <= 0 || d->max_seq_len < 0 || d->max_q_len < 0)
    return PA_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_F32 && d->dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  if ((int64_t)d->max_pages_per_seq * d->page_size < d->max_seq_len) return PA_ERR_INVALID_ARG;
  if (d->max_q_len > d->max_seq_len) return PA_ERR_INVALID_ARG;
  if ((int64_t)d->num_tokens * d->num_q_heads > INT32_MAX) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

// Support check for the MHA kernels (pa_forward / pa_decode_split).
pa_status check_mha_support(const pa_dims* d) {
  if (d->dtype == PA_BF16) {
    if (pa::mha_variant(d->head_dim_qk, d->head_dim_v) < 0) return PA_ERR_UNSUPPORTED;
    if (d->page_size % 8 != 0 || d->page_size > 256) return PA_ERR_UNSUPPORTED;
  } else {
    if (d->head_dim_qk > 256 || d->head_dim_v > 256) return PA_ERR_UNSUPPORTED;
  }
  return PA_OK;
}

// Balanced schedule with at most `pieces` split pieces: partial log-sum-exps
// [pieces, Hq], merge info [B, 2], partial rows [pieces, Hq, 512].
struct MlaBalancedWs {
  size_t lse_off, info_off, po_off, total;
};
MlaBalancedWs mla_balanced_ws(const pa_dims* d, int pieces) {
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  const size_t slots = (size_t)pieces * d->num_q_heads;
  MlaBalancedWs w;
  w.lse_off = 0;
  w.info_off = align(slots * sizeof(float));
  w.po_off = w.info_off + align((size_t)2 * d->num_seqs * sizeof(int32_t));
  w.total = w.po_off + slots * 512 * sizeof(float);
  return w;
}

size_t mla_ws_bytes(const pa_dims* d, int S) {
  if (S <= 1) return 256;  // nothing needed; keep a non-zero size
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads;
  const size_t lse_bytes = ((rows * S * sizeof(float)) + 255) & ~(size_t)255;
  return lse_bytes + rows * S * 512 * sizeof(float);
}

// Chunked route of a pa_forward call (chunked-context processing, "vLLM AMD
// ROCm Attention Backend Optimization", bullet "Chunked context
// processing"), decided from the dims alone so that pa_workspace_size can
// size it.  A bf16 call with prefill-mode rows whose prefill items
// cannot fill the GPU (at most kRouteItems (request, KV head, 256-row block)
// items by the capacities) and whose contexts reach kRouteMinKeys keys runs
// as chunk partials plus a merge: S chunks of C keys, S chosen so that
// items x S is about kRouteTargetItems (one per compute unit: measured 3% faster
// than two for 256 new tokens on 131072 keys, with half the partial rows) while
// the fp32 partials stay under kRouteMaxBytes.
constexpr int64_t kRouteItems = 128, kRouteTargetItems = 256, kRouteMinKeys = 8192,
                  kRouteMinChunk = 2048, kRouteMaxBytes = 256ll << 20;
struct ChunkRoute {
  bool on = false;
  int C = 0, S = 0, row_blocks = 0;
  size_t po_bytes = 0, pl_bytes = 0;
};
ChunkRoute chunk_route(const pa_dims* d) {
  ChunkRoute r;
  if (d->dtype != PA_BF16 || pa::mha_variant(d->head_dim_qk, d->head_dim_v) < 0) return r;
  const int G = d->num_q_heads / d->num_kv_heads;
  if ((int64_t)d->max_q_len * G <= pa::kDecodeRows) return r;  // decode-only calls split their own way
  if (d->max_seq_len < kRouteMinKeys) return r;
  const int64_t blocks = ((int64_t)d->max_q_len * G + pa::kPrefillRows - 1) / pa::kPrefillRows;
  const int64_t items = (int64_t)d->num_seqs * d->num_kv_heads * blocks;
  if (items < 1 || items > kRouteItems) return r;
  const int64_t rows = (int64_t)d->num_tokens * d->num_q_heads;
  const int64_t row_bytes = ((int64_t)d->head_dim_v + 1) * 4;
  int64_t S = (kRouteTargetItems + items - 1) / items;
  S = std::min<int64_t>(S, kRouteMaxBytes / std::max<int64_t>(1, rows * row_bytes));
  S = std::min<int64_t>(S, pa::kMaxSplits);
  if (S < 2) return r;
  int64_t C = (d->max_seq_len + S - 1) / S;
  C = std::max<int64_t>(kRouteMinChunk, (C + 63) & ~63LL);
  S = (d->max_seq_len + C - 1) / C;
  if (S < 2 || items * S > INT32_MAX) return r;
  auto align = [](int64_t x) { return (size_t)((x + 255) & ~255LL); };
  r.on = true;
  r.C = (int)C;
  r.S = (int)S;
  r.row_blocks = (int)blocks;
  r.po_bytes = align(rows * S * d->head_dim_v * 4);
  r.pl_bytes = align(rows * S * 4);
  return r;
}

// Persistent grid of a bf16 pa_forward call and the number of decode items its
// planner aims at (the workspace is sized from the same numbers).
struct FwdGeom {
  bool decode_only = false;
  int grid = 0, target = 0;
};
pa_status fwd_geometry(const pa_dims* d, FwdGeom* g) {
  DevCfg cfg;
  const pa_status st = device_config(&cfg);
  if (st != PA_OK) return st;
  const int G = d->num_q_heads / d->num_kv_heads;
  g->decode_only = (int64_t)d->max_q_len * G <= pa::kDecodeRows;
  g->grid = cfg.cu_count * cfg.occ[pa::mha_variant(d->head_dim_qk, d->head_dim_v)]
                                   [g->decode_only ? 1 : 0];
  // A split item writes its rows as fp32 partials that the merge reads back:
  // with 16 rows per pair (G = 16) that is 4 times the partial bytes per split of
  // G = 4, so decode-only calls of more than 8 rows per pair aim at fewer, longer
  // items (the Qwen3 decode share, 48 requests, 64/4 heads: 0.172 -> 0.168 ms;
  // with 512 pairs the two targets measured the same).
  const bool wide = g->decode_only && (int64_t)d->max_q_len * G > 8;
  g->target = std::max(1, (wide ? pa::kItemsPerWorkgroupWide : pa::kItemsPerWorkgroup) * g->grid);
  return PA_OK;
}

// Partial rows x chunks of the requests pa_forward's planner may cut into
// key chunks (prefill-mode requests of at least kLongKeys keys, "vLLM AMD ROCm
// Attention Backend Optimization", bullet "Chunked context processing"):
// zero unless the dims allow such a request on the persistent path (the
// chunked route takes whole calls of few long requests instead), at most
// kLongBudgetBytes of partials.
int64_t long_rows(const pa_dims* d, const ChunkRoute& route) {
  if (route.on || d->dtype != PA_BF16) return 0;
  if (pa::mha_variant(d->head_dim_qk, d->head_dim_v) < 0) return 0;
  const int G = d->num_q_heads / d->num_kv_heads;
  if ((int64_t)d->max_q_len * G <= pa::kDecodeRows || d->max_seq_len < pa::kLongKeys) return 0;
  const int64_t chunks = (d->max_seq_len + pa::kLongChunk - 1) / pa::kLongChunk;
  const int64_t want = (int64_t)d->num_tokens * d->num_q_heads * chunks;
  return std::min<int64_t>(want, pa::kLongBudgetBytes / (((int64_t)d->head_dim_v + 1) * 4));
}

pa_status check_mla(const pa_dims* d) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  if (d->dtype != PA_BF16 || d->num_kv_heads != 1 || d->head_dim_qk != 576 ||
      d->head_dim_v != 512)
    return PA_ERR_UNSUPPORTED;
  if (d->num_q_heads % 16 != 0 || d->num_q_heads > 128) return PA_ERR_UNSUPPORTED;
  // page size: a power of two in [8, 256]
  if (d->page_size < 8 || d->page_size > 256 || (d->page_size & (d->page_size - 1)) != 0)
    return PA_ERR_UNSUPPORTED;
  if (d->num_tokens != d->num_seqs) return PA_ERR_INVALID_ARG;
  return PA_OK;
}

}  // namespace

extern "C" {

const char* pa_status_string(int32_t status) {
  switch (status) {
    case PA_OK: return "ok";
    case PA_ERR_INVALID_ARG: return "invalid argument";
    case PA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PA_ERR_WORKSPACE: return "workspace missing or too small";
    case PA_ERR_HIP: return "HIP error";
    case PA_ERR_DEVICE_DATA: return "invalid device data";
  }
  return "unknown status";
}

int32_t pa_last_hip_error(void) { return g_last_hip_error; }

pa_status pa_set_kernel_events(void* start, void* stop) {
  g_ev_start = (start && stop) ? (hipEvent_t)start : nullptr;
  g_ev_stop = (start && stop) ? (hipEvent_t)stop : nullptr;
  return PA_OK;
}

size_t pa_workspace_size(const pa_dims* d) {
  if (check_dims(d) != PA_OK) return 0;
  if (d->dtype == PA_F32) return 256;
  // the decode-item bound needs the current device's grid; without a device
  // the bound of kMaxFwdSplits partitions per (request, KV head) is used
  FwdGeom geo;
  const int target = fwd_geometry(d, &geo) == PA_OK ? geo.target : INT32_MAX / 4;
  const ChunkRoute r = chunk_route(d);
  return pa::fwd_workspace_layout(d->num_seqs, d->num_kv_heads, d->head_dim_v, target,
                                  long_rows(d, r))
             .total +
         r.po_bytes + r.pl_bytes;
}

pa_status pa_forward(const void* q, const void* k_cache, const void* v_cache,
                     const int32_t* block_table, const int32_t* seq_lens,
                     const int32_t* query_start_loc, float scale, void* out, float* lse,
                     const pa_dims* d, void* workspace, size_t workspace_bytes, void* stream) {
  return pa_forward_masked(q, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                           PA_MASK_CAUSAL, nullptr, nullptr, nullptr, PA_ALIBI_NONE, scale, out,
                           lse, d, workspace, workspace_bytes, stream);
}

static_assert(PA_MASK_CAUSAL == pa::kMaskCausal && PA_MASK_FULL == pa::kMaskFull &&
                  PA_MASK_PREFIX == pa::kMaskPrefix,
              "mask codes");

static pa_status forward_masked_impl(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t mask,
                            const int32_t* prefix_lens, const float* sinks,
                            const float* alibi_slopes, int32_t alibi_mode, float scale,
                            void* out, float* lse, const pa_dims* d, void* workspace,
                            size_t workspace_bytes, void* stream) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start_loc || !out)
    return PA_ERR_INVALID_ARG;
  if (mask != PA_MASK_CAUSAL && mask != PA_MASK_FULL && mask != PA_MASK_PREFIX)
    return PA_ERR_INVALID_ARG;
  if ((mask == PA_MASK_PREFIX) != (prefix_lens != nullptr)) return PA_ERR_INVALID_ARG;
  if (alibi_mode != PA_ALIBI_NONE && alibi_mode != PA_ALIBI_LINEAR && alibi_mode != PA_ALIBI_SQRT)
    return PA_ERR_INVALID_ARG;
  if ((alibi_mode != PA_ALIBI_NONE) != (alibi_slopes != nullptr)) return PA_ERR_INVALID_ARG;
  const bool alibi = alibi_mode != PA_ALIBI_NONE;
  st = check_mha_support(d);
  if (st != PA_OK) return st;
  if (alibi && d->dtype == PA_BF16 && d->head_dim_qk > 128) return PA_ERR_UNSUPPORTED;
  hipStream_t s = (hipStream_t)stream;
  const int G = d->num_q_heads / d->num_kv_heads;
  if (d->num_seqs == 0 || d->num_tokens == 0) return PA_OK;

  if (d->dtype == PA_F32) {
    pa::F32Args a{};
    a.q = (const float*)q;
    a.k_cache = (const float*)k_cache;
    a.v_cache = (const float*)v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.qsl = query_start_loc;
    a.out = (float*)out;
    a.lse = lse;
    a.scale = scale;
    a.B = d->num_seqs;
    a.T = d->num_tokens;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = G;
    a.Dqk = d->head_dim_qk;
    a.Dv = d->head_dim_v;
    a.P = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.num_pages = d->num_pages;
    a.dbg = debug_flag();
    a.num_splits = 1;
    a.mask = mask;
    a.prefix_lens = prefix_lens;
    a.sinks = sinks;
    a.alibi = alibi_slopes;
    a.alibi_sqrt = alibi_mode == PA_ALIBI_SQRT;
    hipError_t e = mark(g_ev_start, s);
    if (e == hipSuccess) e = pa::launch_f32_forward(a, s);
    if (e == hipSuccess) e = mark(g_ev_stop, s);
    return e == hipSuccess ? PA_OK : hip_fail(e);
  }

  const int variant = pa::mha_variant(d->head_dim_qk, d->head_dim_v);
  // (without a device the workspace is checked against the device-free bound
  // pa_workspace_size gives, and the device error is reported after the
  // host checks)
  FwdGeom geo;
  const pa_status geo_st = fwd_geometry(d, &geo);
  // (ALiBi calls stay on the persistent path: the chunk kernel has no ALiBi term)
  const ChunkRoute route = chunk_route(d);
  const pa::FwdWorkspace w =
      pa::fwd_workspace_layout(d->num_seqs, d->num_kv_heads, d->head_dim_v,
                               geo_st == PA_OK ? geo.target : INT32_MAX / 4, long_rows(d, route));
  if (route.on && !alibi) {
    // few long requests: chunk partials and their merge instead of the
    // persistent kernel, whose prefill items alone could not fill the GPU
    if (!workspace || workspace_bytes < w.total + route.po_bytes + route.pl_bytes)
      return PA_ERR_WORKSPACE;
    char* ws = (char*)workspace;
    pa::MhaArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.qsl = query_start_loc;
    a.part_o = (float*)(ws + w.total);
    a.part_lse = (float*)(ws + w.total + route.po_bytes);
    a.scale = scale;
    a.num_seqs = d->num_seqs;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = G;
    a.P = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.num_pages = d->num_pages;
    a.dbg = debug_flag();
    a.num_splits = route.S;
    a.chunk_keys = route.C;
    a.row_blocks = route.row_blocks;
    a.mask = mask;
    a.prefix_lens = prefix_lens;
    hipError_t e = mark(g_ev_start, s);
    if (e == hipSuccess) e = pa::launch_mha_chunked(a, variant, s);
    if (e == hipSuccess) e = mark(g_ev_stop, s);
    if (e == hipSuccess)
      e = pa::launch_merge(a.part_o, a.part_lse, d->num_tokens * d->num_q_heads, route.S,
                           d->head_dim_v, out, true, lse, s, sinks, d->num_q_heads,
                           query_start_loc + d->num_seqs);
    return e == hipSuccess ? PA_OK : hip_fail(e);
  }
  if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
  if (geo_st != PA_OK) return geo_st;
  DevCfg cfg;
  st = device_config(&cfg);
  if (st != PA_OK) return st;
  const bool decode_only = geo.decode_only;
  const int grid = geo.grid;

  char* ws = (char*)workspace;
  pa::Control* ctrl = (pa::Control*)(ws + w.ctrl_off);
  pa::ReqPlan* req = (pa::ReqPlan*)(ws + w.req_off);
  int32_t* pre_off = (int32_t*)(ws + w.pre_off);
  int32_t* dec_items = (int32_t*)(ws + w.items_off);
  int32_t* merges = (int32_t*)(ws + w.merges_off);

  pa::PlanArgs pl{};
  pl.seq_lens = seq_lens;
  pl.qsl = query_start_loc;
  pl.req = req;
  pl.pre_off = pre_off;
  pl.dec_items = dec_items;
  pl.merges = merges;
  pl.ctrl = ctrl;
  pl.B = d->num_seqs;
  pl.Hkv = d->num_kv_heads;
  pl.G = G;
  pl.P = d->page_size;
  pl.max_pages = d->max_pages_per_seq;
  pl.target_items = geo.target;
  pl.cmerge = (int32_t*)(ws + w.cmerge_off);
  pl.long_keys = w.crow_budget > 0 ? pa::kLongKeys : 0;
  pl.chunk_keys = pa::kLongChunk;
  pl.crow_budget = w.crow_budget;
  // decode-only calls of up to kFusedPlanMax requests: the persistent kernel
  // plans itself, so the call is two launches (attention kernel, merge)
  const bool fused = decode_only && d->num_seqs <= pa::kFusedPlanMax;
  hipError_t e = hipSuccess;
  if (!fused && (e = pa::launch_plan(pl, s)) != hipSuccess) return hip_fail(e);

  pa::MhaArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.out = out;
  a.lse = lse;
  a.part_o = (float*)(ws + w.po_off);
  a.part_lse = (float*)(ws + w.plse_off);
  a.req = req;
  a.pre_off = pre_off;
  a.dec_items = dec_items;
  a.merges = merges;
  a.cmerge = (const int32_t*)(ws + w.cmerge_off);
  a.cpart_o = (float*)(ws + w.cpo_off);
  a.cpart_lse = (float*)(ws + w.cpl_off);
  a.chunk_keys = pa::kLongChunk;
  a.ctrl = ctrl;
  a.scale = scale;
  a.num_seqs = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.G = G;
  a.P = d->page_size;
  a.max_pages = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.dbg = debug_flag();
  a.num_splits = 1;
  a.target_items = pl.target_items;
  // A decode-only call whose requests are no longer than the smallest
  // partition the plan would make for a filled grid, and whose (request, KV
  // head) pairs do not outnumber the workgroups, needs neither a plan nor a
  // split nor the queue: workgroup j runs pair j over all its keys.  The merge
  // launch then has no rows to merge and no counters to reset, so it is left
  // out and the call is one launch.
  const bool single_launch = fused && d->max_seq_len <= pa::kMinChunkWide &&
                             (int64_t)d->num_seqs * d->num_kv_heads <= grid;
  a.single_pass = single_launch ? 1 : 0;
  a.mask = mask;
  a.prefix_lens = prefix_lens;
  a.sinks = sinks;
  a.alibi = alibi_slopes;
  a.alibi_sqrt = alibi_mode == PA_ALIBI_SQRT;
  if ((e = mark(g_ev_start, s)) != hipSuccess) return hip_fail(e);
  e = fused ? pa::launch_mha_forward_fused(a, variant, alibi, grid, s)
            : pa::launch_mha_forward(a, variant, decode_only, alibi, grid, s);
  if (e != hipSuccess) return hip_fail(e);
  if ((e = mark(g_ev_stop, s)) != hipSuccess) return hip_fail(e);
  // the merge also leaves the queue counters zeroed for the next call; one
  // wave per 4 rows of each (request, KV head) pair (B * Hkv pairs of up to
  // 16 rows; the waves of unsplit pairs stop at the pair's entry), four waves
  // per workgroup
  if (single_launch) return PA_OK;
  const int64_t pairs = (int64_t)d->num_seqs * d->num_kv_heads;
  a.merge_groups =
      (int)((std::min<int64_t>(std::max(1, d->max_q_len) * (int64_t)G, pa::kDecodeRows) + 3) / 4);
  const int64_t units = pairs * a.merge_groups;
  e = pa::launch_mha_forward_merge(
      a, d->head_dim_v, (int)std::max<int64_t>(1, std::min<int64_t>(cfg.cu_count * 4, (units + 3) / 4)), s);
  if (e != hipSuccess) return hip_fail(e);
  // rows of requests the planner cut into key chunks (dims that allow them only)
  if (!fused && w.crow_budget > 0) {
    e = pa::launch_mha_chunk_merge(a, d->head_dim_v, std::max(1, cfg.cu_count * 4), s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return PA_OK;
}

size_t pa_noalloc_max_workspace(void) { return kScratchBytes; }

pa_status pa_forward_noalloc(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, float scale, void* out, float* lse,
                             const pa_dims* d, void* stream) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  const size_t need = pa_workspace_size(d);
  if (need == 0 || need > kScratchBytes) return PA_ERR_WORKSPACE;
  void* ws = nullptr;
  st = scratch_address(&ws);
  if (st != PA_OK) return st;
  return pa_forward_masked(q, k_cache, v_cache, block_table, seq_lens, query_start_loc,
                           PA_MASK_CAUSAL, nullptr, nullptr, nullptr, PA_ALIBI_NONE, scale, out,
                           lse, d, ws, kScratchBytes, stream);
}

static pa_status decode_split_impl(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, float scale,
                          int32_t num_splits, float* part_out, float* part_lse,
                          const pa_dims* d, void* stream) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !part_out || !part_lse)
    return PA_ERR_INVALID_ARG;
  if (num_splits < 1 || num_splits > pa::kMaxSplits) return PA_ERR_INVALID_ARG;
  if (d->num_tokens != d->num_seqs) return PA_ERR_INVALID_ARG;
  st = check_mha_support(d);
  if (st != PA_OK) return st;
  const int G = d->num_q_heads / d->num_kv_heads;
  // a bf16 partition runs one work item, which holds at most kPrefillRows rows
  if (d->dtype == PA_BF16 && G > pa::kPrefillRows) return PA_ERR_UNSUPPORTED;
  if (d->num_seqs == 0) return PA_OK;
  if ((int64_t)d->num_seqs * d->num_q_heads * num_splits > INT32_MAX) return PA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = mark(g_ev_start, s);
  if (e != hipSuccess) return hip_fail(e);
  if (d->dtype == PA_F32) {
    pa::F32Args a{};
    a.q = (const float*)q;
    a.k_cache = (const float*)k_cache;
    a.v_cache = (const float*)v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.qsl = nullptr;
    a.part_o = part_out;
    a.part_lse = part_lse;
    a.scale = scale;
    a.B = d->num_seqs;
    a.T = d->num_seqs;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = G;
    a.Dqk = d->head_dim_qk;
    a.Dv = d->head_dim_v;
    a.P = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.num_pages = d->num_pages;
    a.dbg = debug_flag();
    a.num_splits = num_splits;
    e = pa::launch_f32_split(a, s);
  } else {
    pa::MhaArgs a{};
    a.q = q;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.qsl = nullptr;
    a.part_o = part_out;
    a.part_lse = part_lse;
    a.scale = scale;
    a.num_seqs = d->num_seqs;
    a.Hq = d->num_q_heads;
    a.Hkv = d->num_kv_heads;
    a.G = G;
    a.P = d->page_size;
    a.max_pages = d->max_pages_per_seq;
    a.num_pages = d->num_pages;
    a.dbg = debug_flag();
    a.num_splits = num_splits;
    e = pa::launch_mha_split(a, pa::mha_variant(d->head_dim_qk, d->head_dim_v), s);
  }
  if (e == hipSuccess) e = mark(g_ev_stop, s);
  return e == hipSuccess ? PA_OK : hip_fail(e);
}

static pa_status forward_chunked_impl(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, float scale, int32_t chunk_keys,
                             int32_t num_chunks, float* part_out, float* part_lse,
                             int32_t mask, const int32_t* prefix_lens, const pa_dims* d,
                             void* stream) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  if (!q || !k_cache || !v_cache || !block_table || !seq_lens || !query_start_loc || !part_out ||
      !part_lse)
    return PA_ERR_INVALID_ARG;
  if (chunk_keys < 64 || chunk_keys % 64 != 0) return PA_ERR_INVALID_ARG;
  if (mask != PA_MASK_CAUSAL && mask != PA_MASK_FULL && mask != PA_MASK_PREFIX)
    return PA_ERR_INVALID_ARG;
  if ((mask == PA_MASK_PREFIX) != (prefix_lens != nullptr)) return PA_ERR_INVALID_ARG;
  if (num_chunks < 1 || num_chunks > pa::kMaxSplits) return PA_ERR_INVALID_ARG;
  if ((int64_t)chunk_keys * num_chunks < d->max_seq_len) return PA_ERR_INVALID_ARG;
  if (d->dtype != PA_BF16) return PA_ERR_UNSUPPORTED;
  st = check_mha_support(d);
  if (st != PA_OK) return st;
  if (d->num_seqs == 0 || d->num_tokens == 0 || d->max_q_len == 0) return PA_OK;
  if ((int64_t)d->num_tokens * d->num_q_heads * num_chunks > INT32_MAX) return PA_ERR_INVALID_ARG;
  const int G = d->num_q_heads / d->num_kv_heads;
  const int64_t row_blocks = ((int64_t)d->max_q_len * G + pa::kPrefillRows - 1) / pa::kPrefillRows;
  if ((int64_t)d->num_seqs * d->num_kv_heads * row_blocks * num_chunks > INT32_MAX)
    return PA_ERR_INVALID_ARG;
  hipStream_t s = (hipStream_t)stream;
  pa::MhaArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.qsl = query_start_loc;
  a.part_o = part_out;
  a.part_lse = part_lse;
  a.scale = scale;
  a.num_seqs = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.Hkv = d->num_kv_heads;
  a.G = G;
  a.P = d->page_size;
  a.max_pages = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.dbg = debug_flag();
  a.num_splits = num_chunks;
  a.chunk_keys = chunk_keys;
  a.row_blocks = (int32_t)row_blocks;
  a.mask = mask;
  a.prefix_lens = prefix_lens;
  hipError_t e = mark(g_ev_start, s);
  if (e == hipSuccess)
    e = pa::launch_mha_chunked(a, pa::mha_variant(d->head_dim_qk, d->head_dim_v), s);
  if (e == hipSuccess) e = mark(g_ev_stop, s);
  return e == hipSuccess ? PA_OK : hip_fail(e);
}

pa_status pa_merge_lse(const float* part_out, const float* part_lse, int32_t num_rows,
                       int32_t num_splits, int32_t head_dim_v, void* out, float* lse,
                       int32_t out_dtype, const float* sinks, int32_t num_q_heads,
                       void* stream) {
  if (!part_out || !part_lse || !out) return PA_ERR_INVALID_ARG;
  if (sinks && num_q_heads < 1) return PA_ERR_INVALID_ARG;
  if (num_rows < 0 || num_splits < 1 || num_splits > pa::kMaxSplits || head_dim_v < 1 ||
      head_dim_v > 1024)
    return PA_ERR_INVALID_ARG;
  if (out_dtype != PA_F32 && out_dtype != PA_BF16) return PA_ERR_INVALID_ARG;
  hipError_t e = pa::launch_merge(part_out, part_lse, num_rows, num_splits, head_dim_v, out,
                                  out_dtype == PA_BF16, lse, (hipStream_t)stream, sinks,
                                  num_q_heads);
  return e == hipSuccess ? PA_OK : hip_fail(e);
}

size_t mla_workspace_size(const pa_dims* d, int32_t num_splits) {
  if (check_mla(d) != PA_OK || num_splits < 0 || num_splits > 64) return 0;
  if (num_splits == 0) {
    DevCfg cfg;
    if (device_config(&cfg) != PA_OK) return 0;
    return mla_balanced_ws(d, 2 * cfg.cu_count).total;
  }
  return mla_ws_bytes(d, num_splits);
}

static pa_status mla_decode_impl(const void* q, const void* kv_cache, const int32_t* block_table,
                     const int32_t* seq_lens, float scale, void* out, float* lse,
                     int32_t num_splits, const pa_dims* d, void* workspace,
                     size_t workspace_bytes, void* stream) {
  pa_status st = check_mla(d);
  if (st != PA_OK) return st;
  if (!q || !kv_cache || !block_table || !seq_lens || !out) return PA_ERR_INVALID_ARG;
  if (num_splits < 0 || num_splits > 64) return PA_ERR_INVALID_ARG;
  if (d->num_seqs == 0) return PA_OK;
  hipStream_t s = (hipStream_t)stream;
  if (num_splits == 0) {
    // balanced schedule: one workgroup per compute unit
    DevCfg cfg;
    st = device_config(&cfg);
    if (st != PA_OK) return st;
    const MlaBalancedWs w = mla_balanced_ws(d, 2 * cfg.cu_count);
    if (!workspace || workspace_bytes < w.total) return PA_ERR_WORKSPACE;
    char* ws = (char*)workspace;
    pa::MlaArgs a{};
    a.q = q;
    a.kv = kv_cache;
    a.block_table = block_table;
    a.seq_lens = seq_lens;
    a.out = out;
    a.lse = lse;
    a.part_lse = (float*)(ws + w.lse_off);
    a.merge_info = (int32_t*)(ws + w.info_off);
    a.part_o = (float*)(ws + w.po_off);
    a.scale = scale;
    a.B = d->num_seqs;
    a.Hq = d->num_q_heads;
    a.P = d->page_size;
    a.log2_page = __builtin_ctz((unsigned)d->page_size);
    a.max_pages = d->max_pages_per_seq;
    a.num_pages = d->num_pages;
    a.dbg = debug_flag();
    a.num_splits = 0;
    a.max_pieces = 2 * cfg.cu_count;
    hipError_t e = mark(g_ev_start, s);
    if (e == hipSuccess) e = pa::launch_mla_balanced(a, cfg.cu_count, s);
    if (e == hipSuccess) e = mark(g_ev_stop, s);
    if (e == hipSuccess) e = pa::launch_mla_balanced_merge(a, s);
    return e == hipSuccess ? PA_OK : hip_fail(e);
  }
  const int S = num_splits;
  if ((int64_t)d->num_seqs * S > INT32_MAX) return PA_ERR_INVALID_ARG;
  const size_t need = mla_ws_bytes(d, S);
  if (S > 1 && (!workspace || workspace_bytes < need)) return PA_ERR_WORKSPACE;
  const size_t rows = (size_t)d->num_seqs * d->num_q_heads;
  const size_t lse_bytes = ((rows * S * sizeof(float)) + 255) & ~(size_t)255;
  pa::MlaArgs a{};
  a.q = q;
  a.kv = kv_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.out = out;
  a.lse = lse;
  a.part_lse = S > 1 ? (float*)workspace : nullptr;
  a.part_o = S > 1 ? (float*)((char*)workspace + lse_bytes) : nullptr;
  a.scale = scale;
  a.B = d->num_seqs;
  a.Hq = d->num_q_heads;
  a.P = d->page_size;
  a.log2_page = __builtin_ctz((unsigned)d->page_size);
  a.max_pages = d->max_pages_per_seq;
  a.num_pages = d->num_pages;
  a.dbg = debug_flag();
  a.num_splits = S;
  hipError_t e = mark(g_ev_start, s);
  if (e == hipSuccess) e = pa::launch_mla_split(a, s);
  if (e == hipSuccess) e = mark(g_ev_stop, s);
  if (e != hipSuccess) return hip_fail(e);
  if (S > 1) {
    e = pa::launch_merge(a.part_o, a.part_lse, (int)rows, S, 512, out, true, lse, s);
    if (e != hipSuccess) return hip_fail(e);
  }
  return PA_OK;
}

// The entry points that read a block table (debug builds check it there).
pa_status pa_forward_masked(const void* q, const void* k_cache, const void* v_cache,
                            const int32_t* block_table, const int32_t* seq_lens,
                            const int32_t* query_start_loc, int32_t mask,
                            const int32_t* prefix_lens, const float* sinks,
                            const float* alibi_slopes, int32_t alibi_mode, float scale,
                            void* out, float* lse, const pa_dims* d, void* workspace,
                            size_t workspace_bytes, void* stream) {
  return debug_end(forward_masked_impl(q, k_cache, v_cache, block_table, seq_lens,
                                       query_start_loc, mask, prefix_lens, sinks, alibi_slopes,
                                       alibi_mode, scale, out, lse, d, workspace, workspace_bytes,
                                       stream),
                   (hipStream_t)stream);
}

pa_status pa_decode_split(const void* q, const void* k_cache, const void* v_cache,
                          const int32_t* block_table, const int32_t* seq_lens, float scale,
                          int32_t num_splits, float* part_out, float* part_lse,
                          const pa_dims* d, void* stream) {
  return debug_end(decode_split_impl(q, k_cache, v_cache, block_table, seq_lens, scale,
                                     num_splits, part_out, part_lse, d, stream),
                   (hipStream_t)stream);
}

pa_status pa_forward_chunked(const void* q, const void* k_cache, const void* v_cache,
                             const int32_t* block_table, const int32_t* seq_lens,
                             const int32_t* query_start_loc, float scale, int32_t chunk_keys,
                             int32_t num_chunks, float* part_out, float* part_lse,
                             int32_t mask, const int32_t* prefix_lens, const pa_dims* d,
                             void* stream) {
  return debug_end(forward_chunked_impl(q, k_cache, v_cache, block_table, seq_lens,
                                        query_start_loc, scale, chunk_keys, num_chunks, part_out,
                                        part_lse, mask, prefix_lens, d, stream),
                   (hipStream_t)stream);
}

pa_status mla_decode(const void* q, const void* kv_cache, const int32_t* block_table,
                     const int32_t* seq_lens, float scale, void* out, float* lse,
                     int32_t num_splits, const pa_dims* d, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return debug_end(mla_decode_impl(q, kv_cache, block_table, seq_lens, scale, out, lse,
                                   num_splits, d, workspace, workspace_bytes, stream),
                   (hipStream_t)stream);
}

pa_status pa_validate(const int32_t* block_table, const int32_t* seq_lens,
                      const int32_t* query_start_loc, const pa_dims* d, int32_t* bad_seq,
                      void* stream) {
  pa_status st = check_dims(d);
  if (st != PA_OK) return st;
  if (!block_table || !seq_lens) return PA_ERR_INVALID_ARG;
  if (bad_seq) *bad_seq = -1;
  const int B = d->num_seqs;
  if (B == 0) return PA_OK;
  hipStream_t s = (hipStream_t)stream;
  std::vector<int32_t> bt((size_t)B * d->max_pages_per_seq), sl(B), qs(B + 1);
  hipError_t e = hipMemcpyAsync(bt.data(), block_table, bt.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipMemcpyAsync(sl.data(), seq_lens, sl.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess && query_start_loc)
    e = hipMemcpyAsync(qs.data(), query_start_loc, qs.size() * 4, hipMemcpyDeviceToHost, s);
  if (e == hipSuccess) e = hipStreamSynchronize(s);
  if (e != hipSuccess) return hip_fail(e);
  if (!query_start_loc)
    for (int b = 0; b <= B; ++b) qs[b] = b;
  int bad = -1;
  if (qs[0] != 0) bad = 0;
  for (int b = 0; b < B && bad < 0; ++b) {
    const int nq = qs[b + 1] - qs[b], L = sl[b];
    bool ok = nq >= 0 && nq <= d->max_q_len && L >= nq && L <= d->max_seq_len;
    if (!query_start_loc && L < 1) ok = false;
    if (ok) {
      const int64_t np = ((int64_t)L + d->page_size - 1) / d->page_size;
      if (np > d->max_pages_per_seq) ok = false;
      for (int64_t i = 0; i < np && ok; ++i) {
        const int32_t pg = bt[(size_t)b * d->max_pages_per_seq + i];
        if (pg < 0 || pg >= d->num_pages) ok = false;
      }
    }
    if (!ok) bad = b;
  }
  if (bad < 0 && qs[B] > d->num_tokens) bad = B - 1;
  if (bad >= 0) {
    if (bad_seq) *bad_seq = bad;
    return PA_ERR_DEVICE_DATA;
  }
  return PA_OK;
}

}  // extern "C"
