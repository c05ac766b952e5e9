// pa_merge.hip — log-sum-exp merge of split partials.
//
// Merge ("vLLM Triton Attention Backend Deep Dive", section "Parallel tiled
// softmax (3D kernel)": a second launch combines the partial results;
// "vLLM AMD ROCm Attention Backend Optimization", bullet "Chunked context
// processing": the pieces are combined by log-sum-exp for stability):
//   M = max_s lse_s;  w_s = exp(lse_s - M), 0 for an empty partition;
//   out = sum_s w_s o_s / sum_s w_s;  lse = M + ln sum_s w_s.
// With sink logits (pa_forward's chunked route), row r of head r % Hq folds
// sinks[r % Hq] in as one more zero-valued key (fold_sink).
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMergeThreads = 256;

// One wave per row; partials of a row are contiguous: part_o [rows, S, Dv].
__global__ __launch_bounds__(kMergeThreads) void merge_kernel(const float* __restrict__ po,
                                                              const float* __restrict__ pl,
                                                              int rows, int S, int Dv, void* out,
                                                              int out_bf16, float* lse,
                                                              const float* __restrict__ sinks,
                                                              int Hq,
                                                              const int32_t* __restrict__ tok_end) {
  __shared__ float wts[kMergeThreads / 64][kMaxSplits];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int64_t row = (int64_t)blockIdx.x * (kMergeThreads / 64) + wv;
  // rows of tokens at or past *tok_end (when given) are left untouched
  const bool valid = row < rows && (!tok_end || row < (int64_t)tok_end[0] * Hq);
  // (every wave reaches the barrier below)
  const float* ls = pl + (valid ? row : 0) * S;
  float M = kNegInf;
  if (valid)
    for (int s = lane; s < S; s += 64) M = fmaxf(M, ls[s]);
  M = wave_max(M);
  float wsum = 0.f;
  if (valid)
    for (int s = lane; s < S; s += 64) {
      const float v = ls[s];
      const float w = (M != kNegInf && v != kNegInf) ? __expf(v - M) : 0.f;
      wts[wv][s] = w;
      wsum += w;
    }
  wsum = wave_sum(wsum);
  __syncthreads();
  if (!valid) return;
  float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  float lrow = wsum > 0.f ? M + __logf(wsum) : kNegInf;
  if (sinks) inv *= fold_sink(sinks[row % Hq], &lrow);
  const float* o = po + row * S * Dv;
  for (int d = lane; d < Dv; d += 64) {
    float acc = 0.f;
    for (int s = 0; s < S; ++s) {
      const float w = wts[wv][s];
      if (w != 0.f) acc = fmaf(w, o[(int64_t)s * Dv + d], acc);
    }
    acc *= inv;
    if (out_bf16) ((__bf16*)out)[row * Dv + d] = (__bf16)acc;
    else ((float*)out)[row * Dv + d] = acc;
  }
  if (lane == 0 && lse) lse[row] = lrow;
}

}  // namespace

hipError_t launch_merge(const float* po, const float* pl, int rows, int S, int Dv, void* out,
                        bool out_bf16, float* lse, hipStream_t s, const float* sinks, int Hq,
                        const int32_t* tok_end) {
  if (rows <= 0) return hipSuccess;
  const int blocks = (rows + kMergeThreads / 64 - 1) / (kMergeThreads / 64);
  hipLaunchKernelGGL(merge_kernel, dim3(blocks), dim3(kMergeThreads), 0, s, po, pl, rows, S, Dv,
                     out, out_bf16 ? 1 : 0, lse, sinks, Hq > 0 ? Hq : 1, tok_end);
  return hipGetLastError();
}

}  // namespace pa
