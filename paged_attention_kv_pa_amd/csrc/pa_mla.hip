// pa_mla.hip — absorbed multi-head latent attention decode on gfx950.
//
// All query heads of a request attend to one cached latent row per token;
// the row (576 columns) is the key and its first 512 columns are the value
// ("vLLM AMD ROCm Attention Backend Optimization", sections "AITER MLA
// backend" and "Hybrid processing strategy").  With 128 heads on one latent
// head the work per cached byte is high, so a workgroup of 8 waves takes all
// heads of one request (wave w owns the kMNT 16-row MFMA tiles of heads
// 16 kMNT w ..) and each latent tile is read from HBM once.
//
// Per 32-key tile:
//   * the tile is copied to LDS row-major (the key operand), then transposed
//     inside LDS into [column][key] (the value operand), so that each of the
//     waves reads 16-byte MFMA operands for both products;
//   * S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 with the same
//     lane-local row statistics as the MHA kernel (key rows of the K operand
//     permuted so lane group g holds keys 8g .. 8g+7);
//   * online softmax in base 2, probabilities rounded to bf16.
// The keys of a request are split into page-aligned partitions, one
// workgroup each, and merged by log-sum-exp in a second launch.
#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMlaThreads = 512;
constexpr int kMNT = 1;                  // 16-row tiles per wave
constexpr int kDqk = 576, kDv = 512;
constexpr int kMTK = 32;                 // keys per tile
constexpr int kMKRow = kDqk + 8;         // bf16 per K row in LDS
constexpr int kMVRow = kMTK + 8;         // bf16 per V^T row in LDS
constexpr int kMChunks = kMTK * kDqk / 8;  // 16-byte chunks per tile (2304)
constexpr int kMLoads = (kMChunks + kMlaThreads - 1) / kMlaThreads;  // 5

struct alignas(16) MlaLds {
  __bf16 k[2][kMTK * kMKRow];
  __bf16 v[2][kDv * kMVRow];
};

__device__ __forceinline__ int kperm(int mt, int m) { return 8 * (m >> 2) + 4 * mt + (m & 3); }

__global__ __launch_bounds__(kMlaThreads) void mla_split_kernel(MlaArgs a) {
  extern __shared__ __align__(16) char mla_smem[];
  MlaLds& sm = *reinterpret_cast<MlaLds*>(mla_smem);
  constexpr int KS = kDqk / 32, DT = kDv / 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int S = a.num_splits;
  const int s = blockIdx.x % S, b = blockIdx.x / S;
  const int L = a.seq_lens[b], P = a.P;
  const int pages = (L + P - 1) / P;
  const long long per = (long long)P * ((pages + S - 1) / S);
  const long long a0 = per * s, a1 = a0 + per;
  const int t0k = a0 < L ? (int)a0 : L, t1k = a1 < L ? (int)a1 : L;

  int head[kMNT];
  bool row_ok[kMNT];
  bf16x8 qf[kMNT][KS];
#pragma unroll
  for (int nt = 0; nt < kMNT; ++nt) {
    head[nt] = 16 * (kMNT * wave + nt) + r;
    row_ok[nt] = head[nt] < a.Hq;
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)b * a.Hq + head[nt]) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[nt][ks] = row_ok[nt] ? as_bf16x8(load16(qp + 32 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  const float sc = a.scale * kLog2e;
  float m[kMNT], l[kMNT];
  floatx4 acc[kMNT][DT];
#pragma unroll
  for (int nt = 0; nt < kMNT; ++nt) {
    m[nt] = kNegInf;
    l[nt] = 0.f;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[nt][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }

  const int32_t* bt = a.block_table + (int64_t)b * a.max_pages;
  const __bf16* kv = (const __bf16*)a.kv;
  u32x4 reg[kMLoads];
  auto gload = [&](int t0) {
#pragma unroll
    for (int j = 0; j < kMLoads; ++j) {
      const int c = j * kMlaThreads + tid;
      if (c < kMChunks) {
        const int key = min(t0 + c / (kDqk / 8), t1k - 1);  // clamped: real data
        const int page = bt[key / P];
        reg[j] = load16(kv + ((int64_t)page * P + (key % P)) * kDqk + (c % (kDqk / 8)) * 8);
      }
    }
  };
  auto kstore = [&](int buf) {
#pragma unroll
    for (int j = 0; j < kMLoads; ++j) {
      const int c = j * kMlaThreads + tid;
      if (c < kMChunks) store16(&sm.k[buf][(c / (kDqk / 8)) * kMKRow + (c % (kDqk / 8)) * 8], reg[j]);
    }
  };
  // V^T[col][key] for col < 512 from the row-major tile: thread task u covers
  // column u % 512 and keys 8 (u / 512) .. +7.
  auto transpose = [&](int buf) {
    const unsigned short* kt = reinterpret_cast<const unsigned short*>(sm.k[buf]);
#pragma unroll
    for (int j = 0; j < kDv * (kMTK / 8) / kMlaThreads; ++j) {
      const int u = j * kMlaThreads + tid;
      const int col = u % kDv, kg = u / kDv;
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = kt[(8 * kg + 2 * e) * kMKRow + col];
        const uint32_t hi = kt[(8 * kg + 2 * e + 1) * kMKRow + col];
        w[e] = lo | (hi << 16);
      }
      store16(&sm.v[buf][col * kMVRow + 8 * kg], u32x4{w[0], w[1], w[2], w[3]});
    }
  };

  const int ntiles = (t1k - t0k + kMTK - 1) / kMTK;
  if (ntiles > 0) {
    gload(t0k);
    kstore(0);
  }
  __syncthreads();
  if (ntiles > 0) transpose(0);
  __syncthreads();
  for (int ti = 0; ti < ntiles; ++ti) {
    const int t0 = t0k + ti * kMTK;
    const int buf = ti & 1;
    {
      const __bf16* kt = sm.k[buf];
      const __bf16* vt = sm.v[buf];
      floatx4 sacc[kMNT][2];
#pragma unroll
      for (int nt = 0; nt < kMNT; ++nt) sacc[nt][0] = sacc[nt][1] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const bf16x8 k0 = as_bf16x8(load16(kt + kperm(0, r) * kMKRow + 32 * ks + 8 * g));
        const bf16x8 k1 = as_bf16x8(load16(kt + kperm(1, r) * kMKRow + 32 * ks + 8 * g));
#pragma unroll
        for (int nt = 0; nt < kMNT; ++nt) {
          sacc[nt][0] = mfma_bf16(k0, qf[nt][ks], sacc[nt][0]);
          sacc[nt][1] = mfma_bf16(k1, qf[nt][ks], sacc[nt][1]);
        }
      }
      bf16x8 pf[kMNT];
      float alpha[kMNT];
#pragma unroll
      for (int nt = 0; nt < kMNT; ++nt) {
        float x[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float v = j < 4 ? sacc[nt][0][j] : sacc[nt][1][j - 4];
          x[j] = (t0 + 8 * g + j) < t1k ? v : kNegInf;
        }
        float tmax = x[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, x[j]);
        tmax = group_max4(tmax);
        const float mnew = fmaxf(m[nt], tmax);
        const float muse = mnew == kNegInf ? 0.f : mnew;
        alpha[nt] = fast_exp2((m[nt] - muse) * sc);
        const float msc = muse * sc;
        float p[8], psum = 0.f;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          p[j] = fast_exp2(fmaf(x[j], sc, -msc));
          psum += p[j];
        }
        l[nt] = fmaf(l[nt], alpha[nt], psum);
        m[nt] = mnew;
        pf[nt] = __builtin_bit_cast(
            bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]),
                          pack_bf16x2(p[4], p[5]), pack_bf16x2(p[6], p[7])});
      }
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const bf16x8 vf = as_bf16x8(load16(vt + (16 * dt + r) * kMVRow + 8 * g));
#pragma unroll
        for (int nt = 0; nt < kMNT; ++nt) {
          acc[nt][dt] *= alpha[nt];
          acc[nt][dt] = mfma_bf16(vf, pf[nt], acc[nt][dt]);
        }
      }
    }
    if (ti + 1 < ntiles) {
      gload(t0 + kMTK);
      kstore(buf ^ 1);
    }
    __syncthreads();
    if (ti + 1 < ntiles) transpose(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds O[head][16 dt + 4g + i]
#pragma unroll
  for (int nt = 0; nt < kMNT; ++nt) {
    const float lrow = group_sum4(l[nt]);
    if (!row_ok[nt]) continue;
    const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
    const float lse = lrow > 0.f ? m[nt] * a.scale + __log2f(lrow) * kLn2 : kNegInf;
    const int64_t bh = (int64_t)b * a.Hq + head[nt];
    if (S == 1) {
      __bf16* op = (__bf16*)a.out + bh * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        *reinterpret_cast<u32x2*>(op + 16 * dt) =
            u32x2{pack_bf16x2(acc[nt][dt][0] * inv, acc[nt][dt][1] * inv),
                  pack_bf16x2(acc[nt][dt][2] * inv, acc[nt][dt][3] * inv)};
      if (g == 0 && a.lse) a.lse[bh] = lse;
    } else {
      float* op = a.part_o + (bh * S + s) * kDv + 4 * g;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        store16(op + 16 * dt, __builtin_bit_cast(u32x4, acc[nt][dt] * inv));
      if (g == 0) a.part_lse[bh * S + s] = lse;
    }
  }
}

}  // namespace

hipError_t launch_mla_split(const MlaArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.num_splits;
  if (blocks <= 0) return hipSuccess;
  const size_t lds = sizeof(MlaLds);
  hipError_t e = hipFuncSetAttribute((const void*)mla_split_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_split_kernel, dim3(blocks), dim3(kMlaThreads), lds, s, a);
  return hipGetLastError();
}

}  // namespace pa
