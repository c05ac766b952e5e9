// pa_f32.hip — fp32 paged attention on the vector ALUs.
//
// fp32 inputs keep full fp32 products, which the bf16 matrix cores would
// not, so this path computes on VALU: one wave per query row.  The keys of
// the row are walked in 64-key steps (one key per lane for the score, then
// one output column per lane for the value sum) with an online softmax
// ("vLLM Triton Attention Backend Deep Dive", sections "Technical
// implementation of paged attention" and "Parallel tiled softmax (3D
// kernel)").  Used for fp32 caches (the pages name fp32 attention as a use of
// the unified backend, section "Usage scenarios").
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kF32MaxD = 256;

// One query row over keys [k0, k1) (k1 already capped by the row's visible limit).
// Writes out[0..Dv) (normalised) and *lse; an empty range gives 0 and -inf.
// sink: a sink logit folded into the row (-inf: none).  alibi_slope (0: none):
// the ALiBi term slope * f(|qpos - t|) is subtracted from the score of key t.
__device__ void f32_row(const F32Args& a, int b, int kvh, const float* qrow, int k0, int k1,
                        float* out, float* lse_out, float sink, float alibi_slope, int qpos) {
  __shared__ float qs[kF32MaxD];
  __shared__ float ps[64];
  const int lane = threadIdx.x;
  for (int d = lane; d < a.Dqk; d += 64) qs[d] = qrow[d];
  __syncthreads();
  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const int P = a.P, Dqk = a.Dqk, Dv = a.Dv;
  float m = kNegInf, l = 0.f;
  float acc[kF32MaxD / 64];
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) acc[c] = 0.f;
  for (int t0 = k0; t0 < k1; t0 += 64) {
    const int t = t0 + lane;
    float s = kNegInf;
    if (t < k1) {
      const int page = checked_page(bt[t / P], a.num_pages, a.dbg);
      const float* kr = a.k_cache + (((int64_t)page * a.Hkv + kvh) * P + (t % P)) * Dqk;
      float dot = 0.f;
      for (int d = 0; d < Dqk; ++d) dot = fmaf(qs[d], kr[d], dot);
      s = dot * a.scale;
      if (alibi_slope != 0.f) {
        const float d = fabsf((float)(qpos - t));
        s -= alibi_slope * (a.alibi_sqrt ? sqrtf(d) : d);
      }
    }
    const float mnew = fmaxf(m, wave_max(s));  // finite: key t0 < k1 is valid
    const float alpha = __expf(m - mnew);
    const float p = t < k1 ? __expf(s - mnew) : 0.f;
    l = l * alpha + wave_sum(p);
    m = mnew;
    ps[lane] = p;
    __syncthreads();
    const int n = min(64, k1 - t0);
#pragma unroll
    for (int c = 0; c < kF32MaxD / 64; ++c) acc[c] *= alpha;
    for (int j = 0; j < n; ++j) {
      const int tt = t0 + j;
      const int page = checked_page(bt[tt / P], a.num_pages, a.dbg);
      const float* vp = a.v_cache + ((int64_t)page * a.Hkv + kvh) * Dv * P + (tt % P);
      const float pj = ps[j];
#pragma unroll
      for (int c = 0; c < kF32MaxD / 64; ++c) {
        const int d = lane + 64 * c;
        if (d < Dv) acc[c] = fmaf(pj, vp[(int64_t)d * P], acc[c]);
      }
    }
    __syncthreads();
  }
  float inv = l > 0.f ? 1.f / l : 0.f;
  float lse = l > 0.f ? m + __logf(l) : kNegInf;
  if (sink != kNegInf) inv *= fold_sink(sink, &lse);
#pragma unroll
  for (int c = 0; c < kF32MaxD / 64; ++c) {
    const int d = lane + 64 * c;
    if (d < Dv) out[d] = acc[c] * inv;
  }
  if (lane == 0 && lse_out) *lse_out = lse;
}

// pa_forward, fp32: one workgroup (one wave) per (query row, head).
__global__ __launch_bounds__(64) void f32_forward_kernel(F32Args a) {
  const int64_t row = blockIdx.x;  // token * Hq + head
  const int i = (int)(row / a.Hq), h = (int)(row % a.Hq);
  if (i >= a.qsl[a.B]) return;  // rows past the batch's tokens are left untouched
  // request of token i: largest b with qsl[b] <= i (qsl non-decreasing)
  int lo = 0, hi = a.B - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.qsl[mid] <= i) lo = mid; else hi = mid - 1;
  }
  const int b = lo;
  const int nq = a.qsl[b + 1] - a.qsl[b];
  const int L = a.seq_lens[b];
  const int pfx = a.mask == kMaskPrefix ? a.prefix_lens[b] : 0;
  const int end = min(visible_end(a.mask, L - nq, i - a.qsl[b], pfx), L);
  f32_row(a, b, h / a.G, a.q + row * a.Dqk, 0, end, a.out + row * a.Dv,
          a.lse ? a.lse + row : nullptr, a.sinks ? a.sinks[h] : kNegInf,
          a.alibi ? a.alibi[h] : 0.f, L - nq + (i - a.qsl[b]));
}

// pa_decode_split, fp32: one workgroup per (request, head, partition).
__global__ __launch_bounds__(64) void f32_split_kernel(F32Args a) {
  const int S = a.num_splits;
  const int64_t id = blockIdx.x;
  const int s = (int)(id % S);
  const int64_t bh = id / S;  // b * Hq + h
  const int b = (int)(bh / a.Hq), h = (int)(bh % a.Hq);
  const int L = a.seq_lens[b];
  const int pages = (L + a.P - 1) / a.P;
  const long long per = (long long)a.P * ((pages + S - 1) / S);
  const long long a0 = per * s, a1 = a0 + per;
  const int t0 = a0 < L ? (int)a0 : L, t1 = a1 < L ? (int)a1 : L;
  f32_row(a, b, h / a.G, a.q + bh * a.Dqk, t0, t1, a.part_o + id * a.Dv, a.part_lse + id, kNegInf,
          0.f, L - 1);
}

}  // namespace

hipError_t launch_f32_forward(const F32Args& a, hipStream_t s) {
  const int64_t rows = (int64_t)a.T * a.Hq;
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_forward_kernel, dim3(rows), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_f32_split(const F32Args& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.Hq * a.num_splits;
  if (blocks <= 0) return hipSuccess;
  hipLaunchKernelGGL(f32_split_kernel, dim3(blocks), dim3(64), 0, s, a);
  return hipGetLastError();
}

}  // namespace pa
