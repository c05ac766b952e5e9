// pa_mla.hip — absorbed multi-head latent attention decode on gfx950.
//
// All query heads of a request attend to one cached latent row per token;
// the row (576 columns) is the key and its first 512 columns are the value
// ("vLLM AMD ROCm Attention Backend Optimization", sections "AITER MLA
// backend" and "Hybrid processing strategy").  With 128 heads on one latent
// head the work per cached byte is high (about 240 flop per byte), so one
// workgroup takes all heads of one request and every latent tile is read
// from HBM exactly once.  The workgroup has 8 waves, two per SIMD; wave w
// owns heads 16 w .. 16 w + 15 on v_mfma_f32_16x16x32_bf16 (lane layouts in
// pa_device.h).  A wave's output tile (16 heads x 512 columns) is 128
// accumulator registers, so two waves fit on a SIMD and one runs its matrix
// products while the other waits on LDS or runs its softmax.
//
// Per 32-key tile:
//   * HBM -> LDS by direct-to-LDS copies (16 bytes per lane, no registers),
//     issued by waves 0-3, into a 2-stage ring with one barrier per tile,
//     each tile's copies issued one tile ahead.  The tile is stored
//     "chunk-group major": [9 groups of 8 sixteen-byte chunks][32 keys][8],
//     with the chunk index inside a group XOR-swizzled by the key, so that a
//     thread's 9 copies of a tile are 128 bytes apart in HBM (one address
//     register) and the operand reads hit distinct banks;
//   * S^T = K Q^T: M-row r of key block kb (0, 1) holds key 8 (r / 4) + 4 kb
//     + r % 4, so lane (r, g) ends with keys 8 g .. 8 g + 7 of head r — the
//     B operand (P^T) of the value product, in order;
//   * O^T = V^T P^T: one instruction per 16 columns; its V^T operand (8 keys
//     of one column per lane) is read from the row-major tile with two LDS
//     transpose reads (ds_read_b64_tr_b16);
//   * online softmax in base 2 with lazy rescaling: the running max of a head
//     only moves when a tile would push probabilities above 2^8.
// Every wave reads the whole key and value tile from LDS: the 8-wave loop
// reads twice the LDS bytes per key tile that a 4-wave loop of 32 heads per
// wave would, and the second wave per SIMD is worth more.
// The keys of a request are cut into page-aligned partitions, one workgroup
// each, combined by the log-sum-exp merge in a second launch.
#include <atomic>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kMlaThreads = 512;           // 8 waves, two per SIMD
constexpr int kMergeThreads = 256;
constexpr int kDqk = 576, kDv = 512;
constexpr int kMTK = 32;                   // keys per tile
constexpr int kRowChunks = kDqk / 8;       // 16-byte chunks per latent row (72)
constexpr int kGroups = kRowChunks / 8;    // chunk groups per row (9)
constexpr int kStages = 2;
constexpr int kStageBytes = kMTK * kDqk * 2;  // 36 KiB
constexpr float kLazyLog2 = 8.f;           // rescale when probabilities would exceed 2^8
constexpr int kKSteps = kDqk / 32;                       // 18 K-steps of 32 columns
// The query's trailing K-steps are kept in LDS: the 128 accumulator
// registers plus the whole query would not fit in a wave's half of the
// register file.
constexpr int kQRegSteps = 14;                           // query K-steps held in registers
constexpr int kQLdsSteps = kKSteps - kQRegSteps;         // the rest in LDS
constexpr int kQLdsStride = kQLdsSteps * 32 * 2 + 32;    // bytes per head row (padded: 288
                                                         // measured conflict-free, 272 2-way)
constexpr int kQLdsBytes = 128 * kQLdsStride;
constexpr size_t kMlaLds = (size_t)kStages * kStageBytes + kQLdsBytes;

typedef __attribute__((ext_vector_type(4))) short short4v;
typedef __attribute__((address_space(3))) short4v lds_short4;
typedef __attribute__((address_space(3))) const char lds_cchar;

// Swizzle of the chunk index inside its group of 8, by key.  Chosen by
// measurement (the LDS bank-conflict counter over every invertible linear
// map of key bits 1, 3 and 4 onto the 3 chunk bits) among those with no
// conflicts for both the key-operand reads and the transposing value reads:
// LDS bank selection on this part is not a plain function of the low
// address bits, so the choice is not derived here.
__device__ __forceinline__ int swz(int k) {
  const int k1 = (k >> 1) & 1, k3 = (k >> 3) & 1, k4 = (k >> 4) & 1;
  return k1 | ((k1 ^ k3) << 1) | ((k3 ^ k4) << 2);
}

// Byte offset of 16-byte chunk c (0..71) of key k (0..31) inside a stage.
__device__ __forceinline__ int chunk_off(int k, int c) {
  return (((c >> 3) * kMTK + k) * 8 + ((c & 7) ^ swz(k))) * 16;
}

// Keys [t0k, t1k) of request b for all its heads, by one workgroup.  The
// result rows go to the output (pbase < 0) or, normalised, to the partial
// rows part_o / part_lse at index pbase + head * pstride.  Every thread of
// the workgroup calls this together; LDS is free on entry and on return.
__device__ __forceinline__ void mla_keys(const MlaArgs& a, char* mla_smem, int tid, int b,
                                         int t0k, int t1k, int64_t pbase, int pstride) {
  constexpr int DT = kDv / 16;  // 32 column tiles of O^T
  const int wave = tid >> 6, lane = tid & 63;
  const int r = lane & 15, g = lane >> 4;
  const int P = a.P, lp = a.log2_page;
  const int ntiles = (t1k - t0k + kMTK - 1) / kMTK;

  // The block table is read-only for the whole call: reading it through the
  // constant address space lets the uniform reads become scalar loads (a
  // vector load would make the compiler wait for every copy in flight).  The
  // request's table row and the cache base are workgroup-uniform: kept in
  // scalar registers, nothing on the copy path is reloaded from spill slots.
  typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;
  const ConstI32Ptr bt =
      (ConstI32Ptr)uniform_ptr(a.block_table + (int64_t)__builtin_amdgcn_readfirstlane(b) * a.max_pages);
  const char* kv = uniform_ptr((const char*)a.kv);

  // DMA of tile ti into stage st by waves 0-3 (one per SIMD): thread t of
  // them copies key t / 8, chunk slot t % 8 of each of the 9 groups; one
  // wave instruction fills 64 consecutive chunk positions of a group.
  const int wave_s = __builtin_amdgcn_readfirstlane(wave);
  const bool copier = wave_s < 4;
  const uint32_t lds_wave = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_cchar*)mla_smem + (wave_s & 3) * 64 * 16);
  auto issue_tile = [&](int ti, int st) {
    // The thread's key and chunk are recomputed from the lane index at every
    // call (the empty asm keeps the compiler from hoisting them out of the
    // tile loop): kept live across the loop they get spilled, and their
    // reload would wait for the copies in flight.
    int lane_now = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    asm volatile("" : "+v"(lane_now));
    const int dt = (wave_s & 3) * 64 + lane_now;
    const int dkey = dt >> 3;
    const int dchunk = (dt & 7) ^ swz(dkey);
    const int lane_src = dkey * (kDqk * 2) + dchunk * 16;
    const int t0 = t0k + ti * kMTK;
    const char* src;
    if (P >= kMTK && t0 + kMTK <= t1k) {
      // all 32 keys real and in one page: a scalar page base plus a fixed
      // per-lane offset
      const int page = checked_page(bt[t0 >> lp], a.num_pages, a.dbg);
      src = kv + (((int64_t)page << lp) + (t0 & (P - 1))) * (kDqk * 2) + lane_src;
    } else {
      const int key = min(t0 + dkey, t1k - 1);  // clamped: real data, masked later
      const int last_pg = (t1k - 1) >> lp;
      const int pg0 = __builtin_amdgcn_readfirstlane(t0 >> lp);
      int page;
      if (P >= kMTK) {
        page = checked_page(bt[pg0], a.num_pages, a.dbg);
      } else {
        const int j = (key >> lp) - pg0;  // 0 .. 32 / P - 1
        const int p0 = checked_page(bt[pg0], a.num_pages, a.dbg);
        const int p1 = checked_page(bt[min(pg0 + 1, last_pg)], a.num_pages, a.dbg);
        const int p2 = checked_page(bt[min(pg0 + 2, last_pg)], a.num_pages, a.dbg);
        const int p3 = checked_page(bt[min(pg0 + 3, last_pg)], a.num_pages, a.dbg);
        page = j == 0 ? p0 : (j == 1 ? p1 : (j == 2 ? p2 : p3));
      }
      src = kv + (((int64_t)page << lp) + (key & (P - 1))) * (kDqk * 2) + dchunk * 16;
    }
    const uint32_t dst = lds_wave + st * kStageBytes;
    const void* gsrc[kGroups];
    uint32_t ldst[kGroups];
#pragma unroll
    for (int j = 0; j < kGroups; ++j) {
      gsrc[j] = src + 128 * j;
      ldst[j] = dst + j * kMTK * 8 * 16;
    }
    lds_dma16_m0_seq<kGroups>(gsrc, ldst);
  };

  // query: K-steps [0, kQRegSteps) in registers, the rest in LDS after the
  // ring (each wave writes and reads only its own heads' rows)
  const int head = 16 * wave + r;
  const bool row_ok = head < a.Hq;
  char* qlds = mla_smem + kStages * kStageBytes;
  lds_cchar* qlds3 = (lds_cchar*)mla_smem + kStages * kStageBytes;
  bf16x8 qf[kQRegSteps];  // B operand of S^T: Q[head][32 ks + 8 g .. +7]
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)b * a.Hq + head) * kDqk + 8 * g;
#pragma unroll
    for (int ks = 0; ks < kQRegSteps; ++ks)
      qf[ks] = row_ok ? as_bf16x8(load16(qp + 32 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
#pragma unroll
    for (int ks = kQRegSteps; ks < kKSteps; ++ks) {
      const u32x4 v = row_ok ? load16(qp + 32 * ks) : u32x4{0, 0, 0, 0};
      store16(qlds + head * kQLdsStride + (32 * (ks - kQRegSteps) + 8 * g) * 2, v);
    }
  }
  wait_vmcnt<0>();
  if (copier && ntiles > 0) issue_tile(0, 0);

  const float sc = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;  // l: this lane's share of the head's sum
  floatx4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // K operand offsets: K-step ks = 2 j + u reads chunk 4 ks + g = 8 j + 4 u + g
  int koff[2][2];  // [kb][u]; chunk group j adds 4 KiB
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int u = 0; u < 2; ++u)
      koff[kb][u] = chunk_off(8 * (r >> 2) + 4 * kb + (r & 3), 4 * u + g);
  // V^T operand: in 16-lane group g, source lane r of read hh addresses key
  // 8 g + 4 hh + r / 4, columns 16 dt + 4 (r % 4) .. +3 (chunk 2 dt + (r / 2)
  // % 2, half r % 2); lane r of the group receives column 16 dt + r
  int voff[2][4];  // [hh][dt % 4]; chunk group dt / 4 adds 4 KiB
#pragma unroll
  for (int hh = 0; hh < 2; ++hh)
#pragma unroll
    for (int d4 = 0; d4 < 4; ++d4)
      voff[hh][d4] = chunk_off(8 * g + 4 * hh + (r >> 2), 2 * d4 + ((r >> 1) & 1)) + 8 * (r & 1);

  for (int ti = 0; ti < ntiles; ++ti) {
    if (copier) wait_vmcnt<0>();
    __syncthreads();  // tile ti is in LDS; stage (ti + 1) % 2 is no longer read
    if (copier && ti + 1 < ntiles) issue_tile(ti + 1, (ti + 1) % kStages);
    const int t0 = t0k + ti * kMTK;
    lds_cchar* stage = (lds_cchar*)mla_smem + (ti % kStages) * kStageBytes;

    // S^T: instruction i = 2 ks + kb; operand reads kAhead instructions ahead
    constexpr int kAhead = 4;
    auto kread = [&](int i) {
      const int ks = i >> 1, kb = i & 1;
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          stage + koff[kb][ks & 1] + (ks >> 1) * (kMTK * 8 * 16));
      return as_bf16x8(v);
    };
    auto qread = [&](int ks) {
      const u32x4 v = *reinterpret_cast<const __attribute__((address_space(3))) u32x4*>(
          qlds3 + head * kQLdsStride + (32 * (ks - kQRegSteps) + 8 * g) * 2);
      return as_bf16x8(v);
    };
    floatx4 s0 = floatx4{0.f, 0.f, 0.f, 0.f}, s1 = floatx4{0.f, 0.f, 0.f, 0.f};
    bf16x8 kbuf[kAhead], qbuf[4];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) kbuf[i] = kread(i);
#pragma unroll
    for (int i = 0; i < 2 * kKSteps; ++i) {
      const int ks = i >> 1, kb = i & 1;
      // LDS query steps, two K-steps ahead of their use
      if (kb == 0 && ks + 2 >= kQRegSteps && ks + 2 < kKSteps) qbuf[(ks + 2) & 3] = qread(ks + 2);
      const bf16x8 qv = ks < kQRegSteps ? qf[ks < kQRegSteps ? ks : 0] : qbuf[ks & 3];
      if (kb == 0) s0 = mfma_bf16(kbuf[i % kAhead], qv, s0);
      else s1 = mfma_bf16(kbuf[i % kAhead], qv, s1);
      if (i + kAhead < 2 * kKSteps) kbuf[i % kAhead] = kread(i + kAhead);
      __builtin_amdgcn_sched_barrier(0);
    }
    // lane (r, g) holds S[head][t0 + 8 g + j] in x[j]
    float x[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      x[j] = s0[j];
      x[4 + j] = s1[j];
    }
    if (t0 + kMTK > t1k) {  // the last tile of the range: mask the keys past its end
#pragma unroll
      for (int j = 0; j < 8; ++j) x[j] = t0 + 8 * g + j < t1k ? x[j] : kNegInf;
    }
    float tm0 = fmaxf(x[0], x[1]), tm1 = fmaxf(x[4], x[5]);
    tm0 = fmaxf(tm0, fmaxf(x[2], x[3]));
    tm1 = fmaxf(tm1, fmaxf(x[6], x[7]));
    const float tmax = group_max4(fmaxf(tm0, tm1));
    const bool grow = (tmax - m) * sc > kLazyLog2;  // always true on the first tile
    if (__builtin_amdgcn_ballot_w64(grow)) {
      const float mnew = grow ? tmax : m;
      const float alpha = grow ? fast_exp2((m - mnew) * sc) : 1.f;  // 0 while m = -inf
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] *= alpha;
      m = mnew;
    }
    const float msc = (m == kNegInf ? 0.f : m) * sc;
    float p[8], ps0 = 0.f, ps1 = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(fmaf(x[j], sc, -msc));
      if (j & 1) ps1 += p[j];
      else ps0 += p[j];
    }
    l += ps0 + ps1;
    const bf16x8 pf = __builtin_bit_cast(
        bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])});

    // O^T += V^T P^T, operand reads kAheadV instructions ahead
    constexpr int kAheadV = 4;
    auto vread = [&](int dt) {
      const int goff = (dt >> 2) * (kMTK * 8 * 16);
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(stage + voff[0][dt & 3] + goff));
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_short4*)(stage + voff[1][dt & 3] + goff));
      const u32x2 lo2 = __builtin_bit_cast(u32x2, lo), hi2 = __builtin_bit_cast(u32x2, hi);
      return __builtin_bit_cast(bf16x8, u32x4{lo2[0], lo2[1], hi2[0], hi2[1]});
    };
    bf16x8 vbuf[kAheadV];
#pragma unroll
    for (int i = 0; i < kAheadV; ++i) vbuf[i] = vread(i);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] = mfma_bf16(vbuf[dt % kAheadV], pf, acc[dt]);
      if (dt + kAheadV < DT) vbuf[dt % kAheadV] = vread(dt + kAheadV);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  // every wave is done with the ring before a later segment's copies refill it
  __syncthreads();

  // epilogue: lane (r, g) holds O[head][16 dt + 4 g + v] in acc[dt][v]
  const float lrow = group_sum4(l);
  if (!row_ok) return;
  const float inv = lrow > 0.f ? 1.f / lrow : 0.f;
  const float lse = lrow > 0.f ? m * a.scale + __log2f(lrow) * kLn2 : kNegInf;
  const int64_t bh = (int64_t)b * a.Hq + head;
  if (pbase < 0) {
    __bf16* op = (__bf16*)a.out + bh * kDv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      *reinterpret_cast<u32x2*>(op + 16 * dt) =
          u32x2{pack_bf16x2(acc[dt][0] * inv, acc[dt][1] * inv),
                pack_bf16x2(acc[dt][2] * inv, acc[dt][3] * inv)};
    if (g == 0 && a.lse) a.lse[bh] = lse;
  } else {
    const int64_t pi = pbase + (int64_t)head * pstride;
    float* op = a.part_o + pi * kDv + 4 * g;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
      store16(op + 16 * dt, __builtin_bit_cast(u32x4, acc[dt] * inv));
    if (g == 0) a.part_lse[pi] = lse;
  }
}

// pa_decode_split-style partitions: workgroup (b, s) takes the s-th of
// num_splits page-aligned key ranges of request b.
__global__ __launch_bounds__(kMlaThreads) void mla_split_kernel(MlaArgs a) {
  extern __shared__ __align__(16) char mla_smem[];
  const int S = a.num_splits;
  const int s = blockIdx.x % S, b = blockIdx.x / S;
  const int L = a.seq_lens[b], P = a.P;
  const int pages = (L + P - 1) >> a.log2_page;
  const long long per = (long long)P * ((pages + S - 1) / S);
  const long long a0 = per * s, a1 = a0 + per;
  const int t0k = a0 < L ? (int)a0 : L, t1k = a1 < L ? (int)a1 : L;
  const int64_t pbase = S > 1 ? (int64_t)b * a.Hq * S + s : -1;
  mla_keys(a, mla_smem, threadIdx.x, b, t0k, t1k, pbase, S);
}

// Tiles a request contributes to the balanced schedule (an empty request
// still gets one, so that its zero output is written).
__device__ __forceinline__ int mla_tiles(int L) { return L > kMTK ? (L + kMTK - 1) / kMTK : 1; }

// Sum / maximum over the workgroup (every thread gets the result).
template <int NT>
__device__ __forceinline__ long long mla_block_sum(long long v, long long* red) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  __syncthreads();  // red is free
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += red[w];
  return t;
}

// Balanced schedule: the key tiles of all requests, taken in request order,
// form one sequence of T tiles, cut into gridDim.x (one workgroup per compute
// unit) contiguous ranges of ceil(T / gridDim.x) tiles.  Workgroup w walks its
// range request by request: a request wholly inside the range is written to
// the output, a request the range shares with a neighbour (cut) is written as
// partial rows that the merge kernel combines.  A range cuts at most its first
// and its last request, so workgroup w owns two partial slots: 2 w for its
// first segment, 2 w + 1 for a later one.  A cut request b whose first tile
// lies in range w0 and last tile in range w1 has its pieces in slots
// merge_info[2 b] (2 w0 or 2 w0 + 1), then 2 (w0 + 1), ..., 2 w1;
// merge_info[2 b + 1] is the piece count (1: not cut).  Every workgroup
// recomputes the (small) schedule from seq_lens.  The tile loop (mla_keys)
// runs once per segment on the same LDS ring; its LDS accesses stay LDS
// instructions (the ring is addressed through the kernel's own shared array).
__global__ __launch_bounds__(kMlaThreads) void mla_balanced_kernel(MlaArgs a) {
  constexpr int NT = kMlaThreads;
  extern __shared__ __align__(16) char mla_smem[];
  __shared__ long long s_red[NT / 64];
  __shared__ int s_b;
  __shared__ long long s_tb;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  long long T = 0;
  for (int b = tid; b < a.B; b += NT) T += mla_tiles(a.seq_lens[b]);
  T = mla_block_sum<NT>(T, s_red);
  const long long G = gridDim.x, w = blockIdx.x;
  const long long per = (T + G - 1) / G;
  const long long start = w * per, end = min(start + per, T);
  if (start >= end) return;  // uniform: no tile left for this workgroup
  // first request of the range: the one whose tiles [ex, ex + n) hold `start`
  if (tid == 0) s_b = -1;
  long long run = 0;
  for (int base = 0; base < a.B; base += NT) {
    const int b = base + tid;
    const long long n = b < a.B ? mla_tiles(a.seq_lens[b]) : 0;
    long long incl = n;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const long long y = __shfl_up(incl, o);
      if (lane >= o) incl += y;
    }
    __syncthreads();  // s_red is free
    if (lane == 63) s_red[wave] = incl;
    __syncthreads();
    long long before = run, tot = 0;
#pragma unroll
    for (int v = 0; v < NT / 64; ++v) {
      if (v < wave) before += s_red[v];
      tot += s_red[v];
    }
    const long long ex = before + incl - n;
    if (n > 0 && ex <= start && start < ex + n) {
      s_b = b;
      s_tb = ex;
    }
    run += tot;
    if (run > start) break;  // uniform
  }
  __syncthreads();
  int b = __builtin_amdgcn_readfirstlane(s_b);
  long long tb = s_tb;  // first tile of request b in the sequence
  for (int k = 0; b < a.B && tb < end; ++k, ++b) {
    const int L = __builtin_amdgcn_readfirstlane(a.seq_lens[b]);
    const long long n = mla_tiles(L);
    const long long s0 = max(start, tb) - tb, s1 = min(end, tb + n) - tb;
    const bool cut = s0 > 0 || s1 < n;
    const int slot = 2 * (int)w + (k > 0 ? 1 : 0);
    if (tid == 0 && s0 == 0) {  // the request's first tile is in this range
      a.merge_info[2 * b] = slot;
      a.merge_info[2 * b + 1] = cut ? (int)((tb + n - 1) / per - w + 1) : 1;
    }
    const long long k0 = s0 * kMTK, k1 = s1 * kMTK;
    const int t0k = k0 < L ? (int)k0 : L, t1k = k1 < L ? (int)k1 : L;
    const int64_t pbase = cut ? (int64_t)slot * a.Hq : -1;
    mla_keys(a, mla_smem, tid, b, t0k, t1k, pbase, 1);
    tb += n;
  }
}

// Rows of the requests the balanced schedule cut: workgroup (b, 16 heads),
// 16 lanes per row with 32 columns each, folding the pieces' partial rows
// (slots merge_info[2 b], then 2 (w0 + 1), 2 (w0 + 2), ... with w0 =
// merge_info[2 b] / 2) with a running log-sum-exp.
__global__ __launch_bounds__(kMergeThreads) void mla_balanced_merge_kernel(MlaArgs a) {
  const int hg_count = a.Hq / 16;
  const int b = blockIdx.x / hg_count, hg = blockIdx.x % hg_count;
  const int w0 = a.merge_info[2 * b], np = a.merge_info[2 * b + 1];
  if (np <= 1) return;  // written whole by one workgroup
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int head = 16 * hg + 4 * wave + (lane >> 4);
  const int c0 = (lane & 15) * 32;
  float m = kNegInf, wsum = 0.f;
  float o[32];
#pragma unroll
  for (int c = 0; c < 32; ++c) o[c] = 0.f;
  for (int i = 0; i < np; ++i) {
    const int slot = i == 0 ? w0 : 2 * ((w0 >> 1) + i);
    const int64_t pi = (int64_t)slot * a.Hq + head;
    const float ls = a.part_lse[pi];
    const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + pi * kDv + c0);
    floatx4 v[8];
#pragma unroll
    for (int c = 0; c < 8; ++c) v[c] = po[c];
    const float mn = fmaxf(m, ls);
    const float f = mn == kNegInf ? 1.f : __expf(m - mn);
    const float wt = ls == kNegInf ? 0.f : __expf(ls - mn);
    m = mn;
    wsum = fmaf(wsum, f, wt);
#pragma unroll
    for (int c = 0; c < 8; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) o[4 * c + e] = fmaf(wt, v[c][e], o[4 * c + e] * f);
  }
  const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
  const int64_t bh = (int64_t)b * a.Hq + head;
  __bf16* op = (__bf16*)a.out + bh * kDv + c0;
#pragma unroll
  for (int c = 0; c < 32; c += 8)
    store16(op + c, u32x4{pack_bf16x2(o[c] * inv, o[c + 1] * inv), pack_bf16x2(o[c + 2] * inv, o[c + 3] * inv),
                          pack_bf16x2(o[c + 4] * inv, o[c + 5] * inv), pack_bf16x2(o[c + 6] * inv, o[c + 7] * inv)});
  if ((lane & 15) == 0 && a.lse) a.lse[bh] = wsum > 0.f ? m + __logf(wsum) : kNegInf;
}

// Raises a kernel's dynamic-LDS limit once per device (a host-side runtime
// call that need not be repeated on every launch).
hipError_t allow_lds_once(const void* kernel, std::atomic<uint64_t>& done, size_t lds) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = 1ull << (dev & 63);
  if (done.load(std::memory_order_acquire) & bit) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e == hipSuccess) done.fetch_or(bit, std::memory_order_release);
  return e;
}

std::atomic<uint64_t> g_lds_balanced{0}, g_lds_split{0};


}  // namespace

hipError_t launch_mla_balanced(const MlaArgs& a, int grid, hipStream_t s) {
  if (a.B <= 0 || grid <= 0) return hipSuccess;
  hipError_t e = allow_lds_once((const void*)mla_balanced_kernel, g_lds_balanced, kMlaLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_balanced_kernel, dim3(grid), dim3(kMlaThreads), kMlaLds, s, a);
  return hipGetLastError();
}

hipError_t launch_mla_balanced_merge(const MlaArgs& a, hipStream_t s) {
  if (a.B <= 0) return hipSuccess;
  hipLaunchKernelGGL(mla_balanced_merge_kernel, dim3(a.B * (a.Hq / 16)), dim3(kMergeThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_mla_split(const MlaArgs& a, hipStream_t s) {
  const int64_t blocks = (int64_t)a.B * a.num_splits;
  if (blocks <= 0) return hipSuccess;
  hipError_t e = allow_lds_once((const void*)mla_split_kernel, g_lds_split, kMlaLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mla_split_kernel, dim3(blocks), dim3(kMlaThreads), kMlaLds, s, a);
  return hipGetLastError();
}

}  // namespace pa
