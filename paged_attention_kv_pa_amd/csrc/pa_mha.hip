// pa_mha.hip — bf16 paged attention on gfx950 matrix cores (MHA / GQA).
//
// Method (sources: "vLLM Triton Attention Backend Deep Dive" [TDD] and
// "vLLM AMD ROCm Attention Backend Optimization" [ROC]):
//   * paged attention: keys and values are fetched page by page through the
//     block table ([TDD] "Technical implementation of paged attention");
//   * Q-block: the rows of one work item are (new token x query head of one KV
//     head), so one KV load serves every query head of the group
//     ([TDD] "Q-block optimization");
//   * split KV + second-launch log-sum-exp merge for decode rows
//     ([TDD] "Parallel tiled softmax (3D kernel)"; [ROC] "Chunked context
//     processing");
//   * persistent kernel: a fixed grid pulls work items that a planner kernel
//     wrote to device memory, so the launch is graph-capturable
//     ([TDD] "Persistent kernels and CUDA graphs").
//
// Both matrix products run on v_mfma_f32_16x16x32_bf16 with fp32 accumulation
// and are formed transposed, S^T = K Q^T and O^T = V^T P^T, so that every row
// statistic of the online softmax stays inside one lane:
//   * lane l (group g = l / 16, r = l % 16) owns query row r of a 16-row tile;
//   * in S^T the A operand is K with its 16 M-rows permuted so that, for the two
//     16-key M-tiles of a 32-key step, lane group g receives keys 8g .. 8g+7 —
//     exactly the 8 contraction slots it must supply as the B operand (P^T) of
//     the value product;
//   * in O^T the A operand is V^T, read 16 bytes at a time straight from the
//     column-major value page ([dim][slot]); the lane's accumulator holds
//     O[r][16 dt + 4g + i].
// Softmax runs in base 2 on fp32 scores (scale * log2 e folded into one FMA);
// the probabilities are rounded to bf16 for the value product.
#include <algorithm>
#include <type_traits>

#include "pa_device.h"
#include "pa_internal.h"

namespace pa {

namespace {

constexpr int kTK = 64;  // keys per LDS tile in prefill mode

// Key that M-row m of M-tile mt (0, 1) of a 32-key step stands for.
__device__ __forceinline__ int kperm(int mt, int m) { return 8 * (m >> 2) + 4 * mt + (m & 3); }

// Where the rows of an item go.
// Partial row `row` of an item (output row out_row) goes to
// part_o[po_base + row po_row + out_row po_out ..] and
// part_lse[pl_base + row pl_row + out_row pl_out].
struct Dest {
  bool partial;
  float* po;                        // partial outputs and their log-sum-exps
  float* pl;
  int64_t po_base, po_row, po_out;  // partial output offsets (elements)
  int64_t pl_base, pl_row, pl_out;
};

template <int D, int NW>
struct alignas(16) LdsDecode {
  static constexpr int kOStride = D + 4;  // floats per row of the merge buffer
  float m[NW][16];
  float l[NW][16];
  float o[NW][16][kOStride];
};

// Write one finished row: o[] are this thread's `n` consecutive columns
// starting at column c0, already divided by the row sum.
template <int D, int N>
__device__ __forceinline__ void store_row_chunk(const MhaArgs& a, const Dest& dst, int row,
                                                int64_t out_row, int c0, const float* o) {
  static_assert(N == 2 || N == 4 || N == 8, "columns per store");
  if (dst.partial) {
    float* p = dst.po + dst.po_base + (int64_t)row * dst.po_row + out_row * dst.po_out + c0;
    if constexpr (N == 2) {
      *reinterpret_cast<u32x2*>(p) = u32x2{__float_as_uint(o[0]), __float_as_uint(o[1])};
    } else {
#pragma unroll
      for (int e = 0; e < N; e += 4)
        store16(p + e, __builtin_bit_cast(u32x4, floatx4{o[e], o[e + 1], o[e + 2], o[e + 3]}));
    }
  } else {
    __bf16* p = (__bf16*)a.out + out_row * D + c0;
    if constexpr (N == 8) {
      store16(p, u32x4{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]), pack_bf16x2(o[4], o[5]),
                       pack_bf16x2(o[6], o[7])});
    } else if constexpr (N == 4) {
      *reinterpret_cast<u32x2*>(p) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
    } else {
      *reinterpret_cast<uint32_t*>(p) = pack_bf16x2(o[0], o[1]);
    }
  }
}

__device__ __forceinline__ void store_lse(const MhaArgs& a, const Dest& dst, int row,
                                          int64_t out_row, float v) {
  if (dst.partial) {
    dst.pl[dst.pl_base + (int64_t)row * dst.pl_row + out_row * dst.pl_out] = v;
  } else if (a.lse) {
    a.lse[out_row] = v;
  }
}

// ---------------------------------------------------------------------------
// Decode mode: an item of at most 16 rows.  The 4 waves take interleaved
// 32-key steps of the item's key range straight from global memory into MFMA
// operands (no LDS staging: nothing is shared between waves), then merge their
// partial softmax states through LDS.
// ---------------------------------------------------------------------------
// `counter` (may be NULL): thread 0 takes the workgroup's next item index from
// it once the keys are done, so the round trip overlaps the epilogue; the
// index is returned in thread 0.
// ALIBI: subtract the ALiBi term (alibi_term) from every score.
template <int DK, int DV, int NW, bool ALIBI = false>
__device__ int run_decode_item(const MhaArgs& a, const WorkItem& it, const Dest& dst,
                               LdsDecode<DV, NW>& sm, int32_t* counter) {
  constexpr int KS = DK / 32, DT = DV / 16;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, g = lane >> 4, r = lane & 15;
  const int b = it.seq, kvh = it.kvh, G = a.G, P = a.P;
  const int kv_end = __builtin_amdgcn_readfirstlane(it.kv_end);

  // this lane's query row
  const bool row_ok = r < it.nrows;
  const int ridx = it.row0 + r;
  const int tok = ridx / G;
  const int head = kvh * G + (ridx - tok * G);
  const int pfx = a.mask == kMaskPrefix ? a.prefix_lens[b] : 0;
  const int lim = row_ok ? min(visible_end(a.mask, it.ctx, tok, pfx), kv_end) : it.kv_begin;
  // ALiBi: the row's slope in raw-score units and its query position
  float alibi_m = 0.f;
  if constexpr (ALIBI) alibi_m = row_ok ? a.alibi[head] / a.scale : 0.f;
  const int qpos = it.ctx + tok;
  const int alibi_sqrt = ALIBI ? __builtin_amdgcn_readfirstlane(a.alibi_sqrt) : 0;

  bf16x8 qf[KS];
  {
    const __bf16* qp = (const __bf16*)a.q + ((int64_t)(it.q0 + tok) * a.Hq + head) * DK + 8 * g;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = row_ok ? as_bf16x8(load16(qp + 32 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }

  const float sc = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;
  floatx4 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  // The request's block-table row, read by scalar loads: a vector load of a
  // table entry would be counted behind the K / V loads already in flight,
  // and waiting for it would wait for all of them (one step of look-ahead
  // instead of two).
  typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;
  const ConstI32Ptr bt = (ConstI32Ptr)uniform_ptr(
      a.block_table + (int64_t)__builtin_amdgcn_readfirstlane(b) * a.max_pages);
  const int64_t kpage_elems = (int64_t)a.Hkv * P * DK, vpage_elems = (int64_t)a.Hkv * DV * P;
  const __bf16* kbase = (const __bf16*)a.k_cache + (int64_t)kvh * P * DK + 8 * g;
  const __bf16* vbase = (const __bf16*)a.v_cache + (int64_t)kvh * DV * P + (int64_t)r * P;
  const int last8 = (kv_end - 1) & ~7;
  const int last_pg = __builtin_amdgcn_readfirstlane((kv_end - 1) / P);

  // One 32-key step of this wave: load K / V^T operands, then update the
  // online softmax and the accumulator.  Steps are software-pipelined: the
  // next step's loads are in flight while the current one computes.
  struct Step {
    bf16x8 kf[2][KS];
    bf16x8 vf[DT];
  };
  auto load_step = [&](int t0, Step& st) {
    // Pages of the step's four 8-key groups (P is a multiple of 8, so a group
    // lies in one page); groups past the end take the last page, where their
    // clamped keys are.
    const int ts = __builtin_amdgcn_readfirstlane(t0);
    int pidx = ts / P, off = ts - pidx * P;
    auto next_group = [&]() {
      off += 8;
      if (off >= P) {
        off -= P;
        ++pidx;
      }
      return min(pidx, last_pg);
    };
    const int i0 = min(pidx, last_pg), i1 = next_group(), i2 = next_group(), i3 = next_group();
    const int pg0 = checked_page(bt[i0], a.num_pages, a.dbg);
    const int pg1 = checked_page(bt[i1], a.num_pages, a.dbg);
    const int pg2 = checked_page(bt[i2], a.num_pages, a.dbg);
    const int pg3 = checked_page(bt[i3], a.num_pages, a.dbg);
    // per-lane selects of the four scalars (written out: an indexed array
    // would live in scratch memory)
    auto pick = [](int j, int v0, int v1, int v2, int v3) {
      int x = v0;
      x = j == 1 ? v1 : x;
      x = j == 2 ? v2 : x;
      x = j == 3 ? v3 : x;
      return x;
    };
    {
      // K rows (group r / 4), clamped into the valid range (masked below)
      const int page = pick(r >> 2, pg0, pg1, pg2, pg3);
      const int kb = pick(r >> 2, i0, i1, i2, i3) * P;
#pragma unroll
      for (int mt = 0; mt < 2; ++mt) {
        const int key = min(t0 + kperm(mt, r), kv_end - 1);
        const __bf16* kp = kbase + (int64_t)page * kpage_elems + (key - kb) * DK;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) st.kf[mt][ks] = as_bf16x8(load16(kp + 32 * ks));
      }
    }
    // V^T operand: keys t0+8g .. t0+8g+7 of column 16dt + r
    const int key8 = min(t0 + 8 * g, last8);
    const int page = pick(g, pg0, pg1, pg2, pg3);
    const __bf16* vp = vbase + (int64_t)page * vpage_elems + (key8 - pick(g, i0, i1, i2, i3) * P);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) st.vf[dt] = as_bf16x8(load16(vp + (int64_t)16 * dt * P));
  };
  auto compute_step = [&](int t0, Step& st) {
    if (t0 + 32 > kv_end) {  // keys past the end may be NaN poison: zero their values
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
        st.vf[dt] = as_bf16x8(zero_tail8(as_u32x4(st.vf[dt]), t0 + 8 * g, kv_end));
    }
    floatx4 s[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s[0] = mfma_bf16(st.kf[0][ks], qf[ks], s[0]);
      s[1] = mfma_bf16(st.kf[1][ks], qf[ks], s[1]);
    }
    // online softmax on keys t0 + 8g + j, j = 0..7
    float x[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int key = t0 + 8 * g + j;
      const float v = s[j >> 2][j & 3];
      float vb = v;
      if constexpr (ALIBI) vb -= alibi_term(alibi_m, alibi_sqrt, qpos - key);
      x[j] = key < lim ? vb : kNegInf;
    }
    float tmax = x[0];
#pragma unroll
    for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, x[j]);
    tmax = group_max4(tmax);
    const float mnew = fmaxf(m, tmax);
    const float muse = mnew == kNegInf ? 0.f : mnew;
    const float alpha = fast_exp2((m - muse) * sc);
    const float msc = muse * sc;
    float p[8], psum = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      p[j] = fast_exp2(fmaf(x[j], sc, -msc));
      psum += p[j];
    }
    l = fmaf(l, alpha, psum);
    m = mnew;
    const bf16x8 pf = __builtin_bit_cast(
        bf16x8, u32x4{pack_bf16x2(p[0], p[1]), pack_bf16x2(p[2], p[3]), pack_bf16x2(p[4], p[5]),
                      pack_bf16x2(p[6], p[7])});
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      acc[dt] *= alpha;
      acc[dt] = mfma_bf16(st.vf[dt], pf, acc[dt]);
    }
  };

  {
    // The step bounds are wave-uniform (scalar branches), and the next step's
    // loads are issued unconditionally (past the end they re-read the clamped
    // last key, a cache hit): with a conditional issue the compiler cannot
    // count the loads in flight and waits for all of them before every step
    // (one step of look-ahead instead of two).  Every clamped key is a real
    // key of the item (the wave's range is not empty).
    constexpr int kStride = 32 * NW;  // NW waves x 32 keys
    const int kv_begin = __builtin_amdgcn_readfirstlane(it.kv_begin);
    int t0 = kv_begin + 32 * __builtin_amdgcn_readfirstlane(wave);
    Step sa, sb;
    if (t0 < kv_end) {
      load_step(t0, sa);
      // Two steps per pass and a single exit test at the bottom (an exit
      // between the two steps is merged by the compiler into a flow block
      // whose fall-through path makes it wait for every load at the loop
      // head).  The second step of the last pass may lie wholly past the
      // end: its keys are masked and its values zeroed, so it adds nothing.
      do {
        load_step(t0 + kStride, sb);
        compute_step(t0, sa);
        load_step(t0 + 2 * kStride, sa);
        compute_step(t0 + kStride, sb);
        t0 += 2 * kStride;
      } while (t0 < kv_end);
    }
    // Drain the last look-ahead here, with a wait the compiler sees, so that
    // no load is counted as in flight when the next item's loop starts.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
  }

  int claim = 0;
  if (counter && tid == 0) claim = atomicAdd(counter, 1);

  // merge the NW waves' states
  const float lrow = group_sum4(l);
  if (g == 0) {
    sm.m[wave][r] = m;
    sm.l[wave][r] = lrow;
  }
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
    store16(&sm.o[wave][r][16 * dt + 4 * g], __builtin_bit_cast(u32x4, acc[dt]));
  __syncthreads();
  {
    constexpr int TPR = 4 * NW;   // threads per row
    constexpr int NC = DV / TPR;  // columns per thread
    const int row = tid / TPR, c0 = (tid % TPR) * NC;
    float M = kNegInf;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, sm.m[w][row]);
    float o[NC];
#pragma unroll
    for (int e = 0; e < NC; ++e) o[e] = 0.f;
    float wsum = 0.f;
    if (M != kNegInf) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float f = fast_exp2((sm.m[w][row] - M) * sc);
        wsum = fmaf(f, sm.l[w][row], wsum);
#pragma unroll
        for (int e = 0; e < NC; ++e) o[e] = fmaf(f, sm.o[w][row][c0 + e], o[e]);
      }
    }
    if (row < it.nrows) {
      const int rid = it.row0 + row;
      const int t = rid / G;
      const int head = kvh * G + (rid - t * G);
      const int64_t out_row = (int64_t)(it.q0 + t) * a.Hq + head;
      float lse = wsum > 0.f ? M * a.scale + __log2f(wsum) * kLn2 : kNegInf;
      float f = wsum > 0.f ? 1.f / wsum : 0.f;
      // a sink enters finished rows only (split rows get it in their merge)
      if (a.sinks && !dst.partial) f *= fold_sink(a.sinks[head], &lse);
#pragma unroll
      for (int e = 0; e < NC; ++e) o[e] *= f;
      store_row_chunk<DV, NC>(a, dst, row, out_row, c0, o);
      if (tid % TPR == 0) store_lse(a, dst, row, out_row, lse);
    }
  }
  __syncthreads();
  return claim;
}

// ---------------------------------------------------------------------------
// Prefill mode: an item of up to 256 rows; wave w (of 8) owns rows
// [32 w, 32 w + 32), two waves per SIMD.
// Both products run on v_mfma_f32_32x32x16_bf16, again transposed:
//   * S^T = K Q^T per 32-key block: lane l (n = l % 32, h = l / 32) supplies
//     K row kperm32(n) of the block, columns 16 ks + 8 h .. +7 (A operand) and
//     Q row n, the same columns (B operand, kept in registers); element v of
//     the result is the score of row n and key 16 (v / 8) + 8 h + v % 8;
//   * O^T = V^T P^T per 16-key step: the lane's probabilities for keys
//     16 kc + 8 h .. +7 are exactly its B operand, and V^T[32 dt + n][16 kc +
//     8 h ..] its A operand, so P never leaves the lane.
// 64-key tiles are copied HBM -> LDS by global_load_lds_dwordx4 into a
// four-stage ring shared by the 8 waves: one 64-key tile feeds 256 rows, so
// the L2 -> LDS traffic is 32 KiB per 8.4 MFLOP.  The two waves of a SIMD
// work in ping-pong: while one runs its matrix products, the other runs its
// softmax (see the schedule in run_prefill_item).  LDS layouts (16-byte chunks):
//   K   [16-key group][4-chunk column group][key % 16][chunk % 4 ^ swizzle]
//       — one copy instruction moves 4 column chunks of 16 keys, four
//       consecutive lanes reading 64 contiguous bytes of a key row; the
//       swizzle puts the 16 lanes of a read phase on 16 distinct bank groups;
//   V^T [16-key group][column][8-key half] — one copy instruction moves 32
//       columns of a 16-key group, a lane pair reading the 32 contiguous
//       bytes of one column; operand reads are consecutive.
// The online softmax rescales the accumulator only when a row maximum grows by
// more than 2^8 (exact either way: numerator and denominator share the stale
// maximum).
// ---------------------------------------------------------------------------

// Key held by M-row m (0..31) of the K operand of a 32-key block.
__device__ __forceinline__ int kperm32(int m) {
  const int q = m >> 3, h = (m >> 2) & 1, w = m & 3;
  return 16 * (q >> 1) + 8 * h + 4 * (q & 1) + w;
}

// Scheduling hint for a block of N LDS operand reads each feeding one MFMA:
// keep 4 reads in flight ahead of the matrix instructions instead of waiting
// for each operand right before its use.
template <int N>
__device__ __forceinline__ void pipeline_reads_and_mfma() {
  constexpr int kAhead = N < 4 ? N : 4;
  __builtin_amdgcn_sched_group_barrier(0x100, kAhead, 0);  // LDS reads
#pragma unroll
  for (int i = 0; i < N - kAhead; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
  }
  __builtin_amdgcn_sched_group_barrier(0x008, kAhead, 0);
}

// The K and V^T tiles live in two rings: K of tile t is read in step t only,
// V^T of tile t in step t + 1 (see the schedule in run_prefill_item), and the
// copy of tile t + 2 starts at the beginning of step t.  So the K ring needs
// the 3 stages of tiles t .. t + 2 and the V^T ring the 4 of tiles t - 1 ..
// t + 2 (for DK = 192 one 4-stage ring of both would not fit in LDS).
template <int DK, int DV>
struct PrefillLayout {
  static constexpr int kKStages = 3, kVStages = 4;
  static constexpr int kChunks = DK / 8;                 // 16-byte chunks per key row
  static constexpr int kKBytes = kTK * DK * 2;           // K tile
  static constexpr int kVBytes = kTK * DV * 2;           // V^T tile
  static constexpr int kRingBytes = kKStages * kKBytes + kVStages * kVBytes;
  static constexpr int kKCopies = kChunks / 4;           // K copies per wave per tile
  static constexpr int kVCopies = DV / 32;               // V copies per wave per tile
  static constexpr int kCopies = kKCopies + kVCopies;    // copy instructions per thread per tile
  static_assert(kChunks % 8 == 0 && DV % 32 == 0, "head dims");
  // byte offsets of tile t's K and V^T stages in the ring
  __device__ static __forceinline__ int kstage(int t) { return (t % kKStages) * kKBytes; }
  __device__ static __forceinline__ int vstage(int t) {
    return kKStages * kKBytes + (t % kVStages) * kVBytes;
  }
  // byte offset of column chunk c of tile key k in the K tile: blocks of
  // 16 keys x 4 chunks (1 KiB, one copy instruction), key-major inside, the
  // chunk position XOR-swizzled by key bits 2..3
  __device__ static __forceinline__ int koff(int k, int c) {
    return (((((k >> 4) * (kChunks / 4) + (c >> 2)) * 16 + (k & 15)) * 4) +
            ((c & 3) ^ ((k >> 2) & 3))) * 16;
  }
  // byte offset of key chunk c (keys 8c .. 8c + 7), column d in the V^T tile:
  // per 16-key group, column-major, the group's two 8-key chunks of a column
  // side by side (the 32 bytes one column of a 16-key page row holds)
  __device__ static __forceinline__ int voff(int c, int d) {
    return (((c >> 1) * DV + d) * 2 + (c & 1)) * 16;
  }
};

template <int DK, int DV>
struct alignas(16) LdsPrefill {
  char ring[PrefillLayout<DK, DV>::kRingBytes];
  float alibi_tab[kPrefillWaves][128];  // per wave: sqrt of the tile's distances (ALiBi-sqrt)
};

// ALIBI: subtract the ALiBi term (alibi_term) from every score.
template <int DK, int DV, bool ALIBI = false>
__device__ void run_prefill_item(const MhaArgs& a, const WorkItem& it, const Dest& dst,
                                 LdsPrefill<DK, DV>& sm) {
  using LY = PrefillLayout<DK, DV>;
  constexpr int KS = DK / 16, DT = DV / 32;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 31, h = lane >> 5;
  const int G = __builtin_amdgcn_readfirstlane(a.G), P = __builtin_amdgcn_readfirstlane(a.P);
  // item fields are workgroup-uniform: keep them in scalar registers so that
  // block-table reads become scalar loads
  const int b = __builtin_amdgcn_readfirstlane(it.seq);
  const int kvh = __builtin_amdgcn_readfirstlane(it.kvh);
  const int kv_begin = __builtin_amdgcn_readfirstlane(it.kv_begin);
  const int kv_end = __builtin_amdgcn_readfirstlane(it.kv_end);
  const int nrows = __builtin_amdgcn_readfirstlane(it.nrows);
  const int row0 = __builtin_amdgcn_readfirstlane(it.row0);
  const int ctx = __builtin_amdgcn_readfirstlane(it.ctx);
  const int q0 = __builtin_amdgcn_readfirstlane(it.q0);
  const int mask = __builtin_amdgcn_readfirstlane(a.mask);
  const int pfx = mask == kMaskPrefix ? __builtin_amdgcn_readfirstlane(a.prefix_lens[b]) : 0;

  // this lane's row
  const int row = 32 * wave + n;
  const bool row_ok = row < nrows;
  int64_t out_row;
  int lim;
  float alibi_m = 0.f;  // ALiBi: the row's slope in raw-score units
  int qpos;             // the row's query position
  bf16x8 qf[KS];  // B operand of S^T: Q[row][16 ks + 8 h .. +7]
  {
    const int rid = row0 + row;
    const int t = rid / G;
    const int head = kvh * G + (rid - t * G);
    out_row = (int64_t)(q0 + t) * a.Hq + head;
    lim = row_ok ? min(visible_end(mask, ctx, t, pfx), kv_end) : kv_begin;
    qpos = ctx + t;
    if constexpr (ALIBI) alibi_m = row_ok ? a.alibi[head] / a.scale : 0.f;
  }
  // ALiBi-sqrt: the wave's 32 rows cover at most 32 consecutive query
  // positions from qmin (lane 0's), so with the 64 keys of a tile they span
  // at most 95 distances; the tile's square roots are taken once per wave into
  // a table (two per lane) instead of once per score.  Entry i of the table is
  // for distance qmin - t0 - 63 + i; the lane's entries start at tab_lb.
  const int qmin = __builtin_amdgcn_readfirstlane(qpos);
  const int tab_lb = qpos - qmin + 8 - 8 * h;  // (qpos - qmin) + 63 - 8 h - 55, >= 0
  {
    const __bf16* qp = (const __bf16*)a.q + out_row * DK + 8 * h;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[ks] = row_ok ? as_bf16x8(load16(qp + 16 * ks)) : as_bf16x8(u32x4{0, 0, 0, 0});
  }
  // key limits of the wave's valid rows (rows ascend with the token, so the
  // first row has the smallest limit and the last the largest)
  int wave_lim = kv_begin, wave_min = kv_begin;
  {
    const int first = 32 * wave, last = min(32 * wave + 32, nrows) - 1;
    if (last >= first) {
      wave_min = min(visible_end(mask, ctx, (row0 + first) / G, pfx), kv_end);
      wave_lim = min(visible_end(mask, ctx, (row0 + last) / G, pfx), kv_end);
    }
  }
  // q must be in registers before the copies start counting; tying the
  // fragments to an empty asm makes the compiler wait for them here and not
  // at their first use inside the key loop (where the wait would also drain
  // the copies in flight)
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) asm volatile("" : "+v"(qf[ks]));
  wait_vmcnt<0>();

  // (the arguments may live in vector registers here: the kernel also makes
  // a real call with them; make the bases visibly uniform)
  const int32_t* bt = uniform_ptr(a.block_table + (int64_t)b * a.max_pages);
  const int64_t kpage_elems = (int64_t)__builtin_amdgcn_readfirstlane(a.Hkv * P * DK);
  const int64_t vpage_elems = (int64_t)__builtin_amdgcn_readfirstlane(a.Hkv * DV * P);
  const char* kbase = uniform_ptr((const char*)((const __bf16*)a.k_cache + (int64_t)kvh * P * DK));
  const char* vbase = uniform_ptr((const char*)((const __bf16*)a.v_cache + (int64_t)kvh * DV * P));

  // The copies are issued by the four waves of group A (waves 0-3, which
  // start every step with their matrix products, see the schedule below):
  // wave w copies, of each 64-key tile, all column chunks of K for the 16
  // keys of group w and V^T of the 8-key chunks 2w and 2w + 1.  Issued by
  // all eight waves they cost the softmax group time on its critical path
  // (measured 4.6% slower for the Qwen3 prefill + extend batch).  The keys
  // of group w lie in two 8-key groups, one page each; keys
  // at or past kv_end are clamped to kv_end - 1 (real data, masked or zeroed
  // later).  The block table is read-only for the whole call: reading it
  // through the constant address space lets these uniform reads become
  // scalar loads.
  typedef const __attribute__((address_space(4))) int32_t* ConstI32Ptr;
  const ConstI32Ptr cbt = (ConstI32Ptr)bt;
  // Copy addressing is wave-uniform wherever it can be (scalar registers and
  // scalar arithmetic): the per-lane part is one 32-bit offset per copy.
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  const bool copier = wave_u < kPrefillWaves / 2;  // group A
  const int kgroup = wave_u & (kPrefillWaves / 2 - 1);
  const uint32_t lds_ring = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)sm.ring);
  struct TilePages {
    int pg0, first0;  // physical page and its first key, keys 16 kgroup + 0 .. 7
    int pg1, first1;  // the same for keys 16 kgroup + 8 .. 15
  };
  auto load_pages = [&](int t0) {
    TilePages tp;
    const int ts = __builtin_amdgcn_readfirstlane(t0);
    const int i0 = min(ts + 16 * kgroup, kv_end - 1) / P;
    const int i1 = min(ts + 16 * kgroup + 8, kv_end - 1) / P;
    tp.pg0 = checked_page(cbt[i0], a.num_pages, a.dbg);
    tp.pg1 = checked_page(cbt[i1], a.num_pages, a.dbg);
    tp.first0 = i0 * P;
    tp.first1 = i1 * P;
    return tp;
  };
  auto issue_tile = [&](int t0, int tile, const TilePages& tp) {
    if (!copier) return;
    const uint32_t kst = lds_ring + LY::kstage(tile), vst = lds_ring + LY::vstage(tile);
    const int ts = __builtin_amdgcn_readfirstlane(t0);
#pragma unroll
    for (int half = 0; half < 2; ++half) {  // the two 8-key halves of the group
      // four consecutive lanes copy 64 contiguous bytes of one key row (in
      // swizzled order), so a copy instruction reads 16 whole 64-byte pieces
      const int k16 = lane >> 2;
      const int cl = (lane & 3) ^ ((k16 >> 2) & 3);
      const bool hi = k16 >= 8;
      const int key = min(ts + 16 * kgroup + k16, kv_end - 1);
      const int c0 = half * (LY::kChunks / 2);  // first column chunk of this half
      const char* page0 = kbase + (int64_t)tp.pg0 * kpage_elems * 2;
      const char* page1 = kbase + (int64_t)tp.pg1 * kpage_elems * 2;
      const int off = ((key - (hi ? tp.first1 : tp.first0)) * DK + 8 * (c0 + cl)) * 2;
      const char* src = (hi ? page1 : page0) + off;
      // (each half's copies back to back, m0 saved once for them)
      const void* gsrc[LY::kKCopies / 2];
      uint32_t ldst[LY::kKCopies / 2];
#pragma unroll
      for (int j = 0; j < LY::kKCopies / 2; ++j) {
        gsrc[j] = src + 64 * j;
        ldst[j] = kst + LY::koff(16 * kgroup, c0 + 4 * j);
      }
      lds_dma16_m0_seq<LY::kKCopies / 2>(gsrc, ldst);
    }
    {
      // V^T: lanes 2j and 2j + 1 copy the two 8-key chunks of column 32 i + j
      // for the group's 16 keys; where one page holds all 16 (P >= 16) the
      // pair reads 32 contiguous bytes, and at P = 16 a copy instruction
      // reads 1 KiB in one piece
      const int hv = lane & 1;
      const int cs = min(ts + 8 * (2 * kgroup + hv), (kv_end - 1) & ~7);
      const int pg = hv ? tp.pg1 : tp.pg0;
      const int slot = cs - (hv ? tp.first1 : tp.first0);
      const char* vsrc = vbase + ((int64_t)pg * vpage_elems + (int64_t)(lane >> 1) * P + slot) * 2;
#pragma unroll
      for (int i = 0; i < LY::kVCopies; i += 2) {
        lds_dma16_m0_x2(vsrc + (int64_t)(32 * i) * P * 2, vsrc + (int64_t)(32 * i + 32) * P * 2,
                        vst + LY::voff(2 * kgroup, 32 * i), vst + LY::voff(2 * kgroup, 32 * i + 32));
      }
    }
  };

  const float sc = a.scale * kLog2e;
  float m = kNegInf, l = 0.f;  // m in scaled base-2 units
  floatx16 acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[dt][v] = 0.f;

  const int krow = kperm32(n);
  const int ntiles = (kv_end - kv_begin + kTK - 1) / kTK;
  // tiles this wave computes on: those starting below its largest key limit
  const int wave_tiles = min(ntiles, (wave_lim - kv_begin + kTK - 1) / kTK);

  floatx16 s[2];  // S^T of the tile between its GEMM phase and its softmax phase
  bf16x8 pf[4];   // P^T of the tile between its softmax phase and the next GEMM phase

  // GEMM phase of step t: S^T of tile t, then O^T += V^T P^T of tile t - 1
  // The operand reads are software-pipelined by hand, kAhead reads ahead of
  // the matrix instruction that consumes them; scheduling barriers keep that
  // order (left to itself the scheduler sinks each read next to its use).
  constexpr int kAhead = 4;
  auto gemm_phase = [&](int t) {
    if (t < wave_tiles) {
      const char* stage = sm.ring + LY::kstage(t);
      auto kread = [&](int i) {  // operand i = (ks, kb) = (i / 2, i % 2)
        return as_bf16x8(*reinterpret_cast<const u32x4*>(
            stage + LY::koff(32 * (i & 1) + krow, 2 * (i >> 1) + h)));
      };
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v) s[kb][v] = 0.f;
      bf16x8 buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) buf[i] = kread(i);
#pragma unroll
      for (int i = 0; i < 2 * KS; ++i) {
        s[i & 1] = mfma32_bf16(buf[i % kAhead], qf[i >> 1], s[i & 1]);
        if (i + kAhead < 2 * KS) buf[i % kAhead] = kread(i + kAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (t >= 1 && t - 1 < wave_tiles) {
      const char* stage = sm.ring + LY::vstage(t - 1);
      auto vread = [&](int i) {  // operand i = (kc, dt) = (i / DT, i % DT)
        return as_bf16x8(*reinterpret_cast<const u32x4*>(
            stage + LY::voff(2 * (i / DT) + h, 32 * (i % DT) + n)));
      };
      bf16x8 buf[kAhead];
#pragma unroll
      for (int i = 0; i < kAhead; ++i) buf[i] = vread(i);
#pragma unroll
      for (int i = 0; i < 4 * DT; ++i) {
        acc[i % DT] = mfma32_bf16(buf[i % kAhead], pf[i / DT], acc[i % DT]);
        if (i + kAhead < 4 * DT) buf[i % kAhead] = vread(i + kAhead);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  };

  // softmax phase of tile t: masks, running maximum, lazy rescale of the
  // accumulator (which already holds tiles < t), probabilities.  Works in
  // place on the scores; element (kb, v) is key t0 + 32 kb + 16 (v / 8) + 8 h
  // + v % 8.
  auto softmax_phase = [&](int t) {
    if (t < 0 || t >= wave_tiles) return;
    const int t0 = kv_begin + t * kTK;
    if constexpr (ALIBI) {
      const int alibi_sqrt = __builtin_amdgcn_readfirstlane(a.alibi_sqrt);
      if (alibi_sqrt) {
        float* tab = sm.alibi_tab[wave];
        const int dbase = qmin - t0 - 63;
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          const int d = dbase + lane + 64 * i;
          tab[lane + 64 * i] = __builtin_amdgcn_sqrtf((float)(d < 0 ? -d : d));
        }
        // the key at offset o = 8 h + 32 kb + 16 (v / 8) + v % 8 from t0 is at
        // distance qpos - t0 - o, entry tab_lb + 55 - (o - 8 h)
        const float* tp = tab + tab_lb;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[kb][v] -= alibi_m * tp[55 - (32 * kb + 16 * (v >> 3) + (v & 7))];
      } else {
        const int d0 = qpos - t0 - 8 * h;  // distance to the key at offset 0 from t0 + 8 h
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int v = 0; v < 16; ++v)
            s[kb][v] -= alibi_term(alibi_m, 0, d0 - (32 * kb + 16 * (v >> 3) + (v & 7)));
      }
    }
    if (t0 + kTK > wave_min) {  // only tiles that reach past the smallest limit need masks
      const int rel = lim - t0 - 8 * h;  // visible iff the key's offset from t0 + 8 h is < rel
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (32 * kb + 16 * (v >> 3) + (v & 7) >= rel) s[kb][v] = kNegInf;
    }
    // row maximum: two independent chains (one per 32-key half), then the
    // lane holding the row's other keys (lane ^ 32)
    float tm0 = fmaxf(s[0][0], s[0][1]), tm1 = fmaxf(s[1][0], s[1][1]);
#pragma unroll
    for (int v = 2; v < 16; ++v) {
      tm0 = fmaxf(tm0, s[0][v]);
      tm1 = fmaxf(tm1, s[1][v]);
    }
    const float tmax = xor32_max(fmaxf(tm0, tm1)) * sc;  // scale > 0
    // lazy rescale: move the reference maximum only when it grew by > 2^8
    const bool grow = tmax > m + 8.f;
    if (__any(grow)) {
      const float mnew = grow ? tmax : m;
      const float alpha = grow ? fast_exp2(m - mnew) : 1.f;  // m = -inf gives 0
      l *= alpha;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[dt][v] *= alpha;
      m = mnew;
    }
    const float nmuse = m == kNegInf ? 0.f : -m;
    float ps[4] = {0.f, 0.f, 0.f, 0.f};  // four partial sums: short dependency chains
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        s[kb][v] = fast_exp2(fmaf(s[kb][v], sc, nmuse));
        ps[v & 3] += s[kb][v];
      }
    l += (ps[0] + ps[1]) + (ps[2] + ps[3]);
    // bf16 probabilities: the B operand of O^T
#pragma unroll
    for (int kc = 0; kc < 4; ++kc) {
      const int kb = kc >> 1, v0 = 8 * (kc & 1);
      pf[kc] = __builtin_bit_cast(
          bf16x8, u32x4{pack_bf16x2(s[kb][v0 + 0], s[kb][v0 + 1]), pack_bf16x2(s[kb][v0 + 2], s[kb][v0 + 3]),
                        pack_bf16x2(s[kb][v0 + 4], s[kb][v0 + 5]), pack_bf16x2(s[kb][v0 + 6], s[kb][v0 + 7])});
    }
  };

  // Ping-pong schedule.  Waves 0-3 (group A, one per SIMD) and 4-7 (group B)
  // alternate between a GEMM phase and a softmax phase, B one phase behind A,
  // so each SIMD always has one wave on the matrix core and one on the
  // vector ALU.  Every step ends with a workgroup barrier.  Step t:
  //   even phase: A gemm(t)       B softmax(t - 1)   (copy of tile t + 2 starts)
  //   odd phase:  A softmax(t)    B gemm(t)          (copy of tile t + 1 waited)
  // K of tile t is read in step t and its V^T in step t + 1; tile t + 2 lands
  // in the stages of tiles t - 1 (K) and t - 2 (V^T), last read in step t - 1.
  static_assert(LY::kKStages == 3 && LY::kVStages == 4, "two tiles in flight ahead");
  const bool group_b = wave >= kPrefillWaves / 2;
  if (ntiles > 0) issue_tile(kv_begin, 0, load_pages(kv_begin));
  if (ntiles > 1) {
    issue_tile(kv_begin + kTK, 1, load_pages(kv_begin + kTK));
    if (copier) wait_vmcnt<LY::kCopies>();
  } else {
    wait_vmcnt<0>();
  }
  __syncthreads();
  TilePages next_pages;
  if (ntiles > 2) next_pages = load_pages(kv_begin + 2 * kTK);
  for (int t = 0; t <= ntiles; ++t) {
    if (t + 2 < ntiles) issue_tile(kv_begin + (t + 2) * kTK, t + 2, next_pages);
    if (group_b) softmax_phase(t - 1);
    else gemm_phase(t);
    // (no barrier between the two phases: they share no LDS data; the groups
    // settle into the ping-pong through the barrier at the end of the step,
    // which measured 2% faster than a barrier per phase)
    if (t + 3 < ntiles) next_pages = load_pages(kv_begin + (t + 3) * kTK);
    if (t == ntiles - 1 && kv_begin + (t + 1) * kTK > kv_end) {
      // last tile: zero the values of keys >= kv_end before their first use
      // in the next step (their slots may hold anything, and 0 * NaN would
      // reach the output)
      char* stage = sm.ring + LY::vstage(t);
      const int t0 = kv_begin + t * kTK;
      for (int e = tid; e < 8 * DV; e += kPrefillThreads) {
        const int c = e / DV, d = e - c * DV;
        const int k0 = t0 + 8 * c;
        if (k0 + 8 > kv_end) {
          u32x4* pz = reinterpret_cast<u32x4*>(stage + LY::voff(c, d));
          *pz = zero_tail8(*pz, k0, kv_end);
        }
      }
    }
    if (group_b) gemm_phase(t);
    else softmax_phase(t);
    // this thread's part of tile t + 1 is in LDS (tile t + 2 may stay in flight)
    if (t + 2 < ntiles) {
      if (copier) wait_vmcnt<LY::kCopies>();
    } else {
      wait_vmcnt<0>();
    }
    __syncthreads();
  }
  __syncthreads();  // every wave is done with the ring before the next item

  // epilogue: element v of acc[dt] is O[row][32 dt + 8 (v / 4) + 4 h + v % 4]
  const float lrow = xor32_sum(l);
  if (!row_ok) return;
  float lse = lrow > 0.f ? (m + __log2f(lrow)) * kLn2 : kNegInf;
  float inv = lrow > 0.f ? 1.f / lrow : 0.f;
  // a sink enters finished rows only (partial rows get it in their merge)
  if (a.sinks && !dst.partial) inv *= fold_sink(a.sinks[out_row % a.Hq], &lse);
#pragma unroll
  for (int dt = 0; dt < DT; ++dt)
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float o[4] = {acc[dt][4 * q] * inv, acc[dt][4 * q + 1] * inv,
                          acc[dt][4 * q + 2] * inv, acc[dt][4 * q + 3] * inv};
      store_row_chunk<DV, 4>(a, dst, row, out_row, 32 * dt + 8 * q + 4 * h, o);
    }
  if (h == 0) store_lse(a, dst, row, out_row, lse);
}

template <int DK, int DV, bool DECODE_ONLY>
struct FwdLds {
  union U {
    LdsDecode<DV, kPrefillWaves> dec;
    LdsPrefill<DK, DV> pre;
  };
  typedef typename std::conditional<DECODE_ONLY, LdsDecode<DV, 4>, U>::type type;
};

// Largest b in [0, B) with off[b] <= idx (off is non-decreasing, off[0] = 0):
// the request whose item range [off[b], off[b + 1]) holds idx.  Called by a
// whole wave with a wave-uniform idx: the 64 lanes probe 64 evenly spaced
// entries at once, so B <= 64 takes one round of loads and B <= 4096 two
// (a one-lane binary search would take log2 B dependent loads).
__device__ __forceinline__ int find_request(const int32_t* off, int B, int idx) {
  const int lane = threadIdx.x & 63;
  int lo = 0, n = B;  // the answer lies in [lo, lo + n)
  while (n > 1) {
    const int step = (n + 63) / 64;
    const int k = lane * step;
    const bool ok = k < n && off[lo + k] <= idx;
    const int c = __popcll(__ballot(ok));  // >= 1: off[lo] <= idx
    lo += (c - 1) * step;
    n = min(step, n - (c - 1) * step);
  }
  return lo;
}

static_assert(sizeof(WorkItem) == kItemInts * sizeof(int32_t), "work item size");

// Prefill-mode work item `idx` of pa_forward, decoded from the planner's
// per-request offsets: (KV head, key chunk, row block) in that order, so that
// consecutive items read the same keys; the heaviest row block of a
// (KV head, chunk) comes first.  A request the planner cut into key chunks
// (long contexts, "vLLM AMD ROCm Attention Backend Optimization", bullet
// "Chunked context processing") gets one item per chunk, over the chunk's
// keys below the block's last key limit (possibly none: the item then writes
// empty partials), writing partial rows that the chunk merge combines.
__device__ WorkItem make_prefill_item(const MhaArgs& a, int idx) {
  WorkItem it;
  const int G = a.G;
  const int b = find_request(a.pre_off, a.num_seqs, idx);
  const ReqPlan rp = a.req[b];
  int local = idx - a.pre_off[b];
  const int blk = rp.nblk - 1 - local % rp.nblk;
  local /= rp.nblk;
  const int chunk = local % rp.nchunk;
  const int kvh = local / rp.nchunk;
  const int rows = rp.nq * G;
  it.seq = b;
  it.kvh = kvh;
  it.row0 = blk * kPrefillRows;
  it.nrows = min(kPrefillRows, rows - it.row0);
  it.ctx = rp.L - rp.nq;
  const int pfx = a.mask == kMaskPrefix ? a.prefix_lens[b] : 0;
  const int lim = min(rp.L, visible_end(a.mask, it.ctx, (it.row0 + it.nrows - 1) / G, pfx));
  if (rp.nchunk > 1) {
    const int c0 = chunk * a.chunk_keys;
    it.kv_begin = c0;
    it.kv_end = max(c0, min(lim, c0 + a.chunk_keys));
    it.part = rp.pbase;
    it.nchunk = rp.nchunk;
    it.chunk = chunk;
  } else {
    it.kv_begin = 0;
    it.kv_end = lim;
    it.part = -1;
    it.nchunk = it.chunk = 0;
  }
  it.q0 = rp.q0;
  it.pad = 0;
  return it;
}

// The decode item as a real call, for the kernel that also runs prefill
// items: this keeps the decode code's register allocation out of the prefill
// loop (a call costs little next to a decode item's key loads).
template <int DK, int DV, bool ALIBI>
__device__ __noinline__ int run_decode_item_outlined(const MhaArgs& a, const WorkItem& it,
                                                     const Dest& dst,
                                                     LdsDecode<DV, kPrefillWaves>& sm,
                                                     int32_t* counter) {
  return run_decode_item<DK, DV, kPrefillWaves, ALIBI>(a, it, dst, sm, counter);
}

// ---------------------------------------------------------------------------
// Work planning rules shared by the planner kernel and the persistent
// kernel's own planning (decode-only calls of up to kFusedPlanMax requests).
// ---------------------------------------------------------------------------
// New-token count, key count and first query row of request b.  Requests
// whose lengths are inconsistent (seq_len < q_len, or no key) get no work;
// seq_len is capped at the block-table capacity so no item can index past a
// table row.
__device__ __forceinline__ void shape_of(const int32_t* qsl, const int32_t* seq_lens,
                                         int max_pages, int P, int b, int* nq, int* L, int* q0) {
  *q0 = qsl[b];
  int q = qsl[b + 1] - *q0;
  int l = seq_lens[b];
  const long long cap = (long long)max_pages * P;
  if (l > cap) l = (int)cap;
  if (q < 0 || l < q || l < 1) q = 0;
  *nq = q;
  *L = l;
}

// Smallest decode partition of a call with dec_reqs decode-mode requests.
// When the (request, KV head) pairs are many next to the items aimed at
// (pairs x 2 x kItemsPerWorkgroup >= target_items: at least one pair per two
// workgroups at the usual target, one per four at the wide one), cutting short
// requests only adds partial rows and a merge: the floor is then
// kMinChunkWide.  Fewer pairs need the cuts for parallelism: kMinChunk.
__device__ __forceinline__ long long decode_min_chunk(int dec_reqs, int Hkv, int target_items) {
  const long long pairs = (long long)dec_reqs * Hkv;
  return pairs * 2 * kItemsPerWorkgroup >= target_items ? kMinChunkWide : kMinChunk;
}

// Keys per decode partition: the decode work (keys x KV heads) spread over
// about target_items items, at least minc keys, a multiple of 64.
__device__ __forceinline__ long long decode_chunk(unsigned long long dec_keys, int Hkv,
                                                  int target_items, long long minc) {
  const unsigned long long work = dec_keys * (unsigned long long)Hkv;
  long long chunk = (long long)((work + target_items - 1) / (unsigned long long)target_items);
  chunk = chunk < minc ? minc : chunk;
  return (chunk + 63) & ~63LL;
}

// Partitions of a decode-mode request of L keys.  Items are handed out in
// request order, so the last requests' items run last: cutting those finer
// shortens the tail where workgroups finish at different times (the extra
// partial rows stay few).
__device__ __forceinline__ void decode_split(int L, long long chunk, long long minc, bool tail,
                                             int* per, int* nsplit) {
  long long ck = chunk;
  if (tail) {
    ck = (chunk / kTailDivisor + 63) & ~63LL;
    ck = ck < minc ? minc : ck;
  }
  long long sp = (L + ck - 1) / ck;
  sp = sp < 1 ? 1 : (sp > kMaxFwdSplits ? kMaxFwdSplits : sp);
  *per = 64 * (int)(((L + 63) / 64 + sp - 1) / sp);
  *nsplit = (L + *per - 1) / *per;
}

__device__ __forceinline__ bool is_tail_request(int b, int B) { return b >= B - B / kTailFraction; }

__device__ __forceinline__ int4 wave_inclusive_scan4(int4 v) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int4 u = int4{__shfl_up(v.x, o), __shfl_up(v.y, o), __shfl_up(v.z, o), __shfl_up(v.w, o)};
    if (lane >= o) v = int4{v.x + u.x, v.y + u.y, v.z + u.z, v.w + u.w};
  }
  return v;
}

// Exclusive scan over a workgroup of NT threads; *total gets the sum.
template <int NT>
__device__ int4 block_exclusive_scan4(int4 v, int4* wsum, int4* total) {
  static_assert(NT % 64 == 0 && NT / 64 <= 64, "block size");
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int4 incl = wave_inclusive_scan4(v);
  if (lane == 63) wsum[w] = incl;
  __syncthreads();
  if (w == 0) {
    int4 t = lane < NT / 64 ? wsum[lane] : int4{0, 0, 0, 0};
    t = wave_inclusive_scan4(t);
    if (lane < NT / 64) wsum[lane] = t;  // inclusive prefix of wave totals
  }
  __syncthreads();
  const int4 before = w > 0 ? wsum[w - 1] : int4{0, 0, 0, 0};
  *total = wsum[NT / 64 - 1];
  __syncthreads();
  return int4{before.x + incl.x - v.x, before.y + incl.y - v.y, before.z + incl.z - v.z,
              before.w + incl.w - v.w};
}

// The persistent kernel's own plan of a decode-only call (every workgroup
// computes it; workgroup 0 also writes the merge entries and their count):
// per request its first item and first partial slot.
struct FusedPlan {
  int doff[kFusedPlanMax + 1];  // first decode item of each request; [B] = item count
  int soff[kFusedPlanMax + 1];  // first partial slot
  int nq[kFusedPlanMax];        // each request's shape (shape_of), loaded once
  int L[kFusedPlanMax];
  int q0[kFusedPlanMax];
  int4 wsum[kThreads / 64];
  unsigned long long keys;
  int reqs;       // decode-mode requests
  long long minc;  // smallest partition (decode_min_chunk)
};

__device__ long long fused_plan(const MhaArgs& a, FusedPlan& fp) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    fp.keys = 0;
    fp.reqs = 0;
  }
  __syncthreads();
  unsigned long long my_keys = 0;
  int my_reqs = 0;
  for (int b = tid; b < a.num_seqs; b += kThreads) {
    int nq, L, q0;
    shape_of(a.qsl, a.seq_lens, a.max_pages, a.P, b, &nq, &L, &q0);
    fp.nq[b] = nq;  // read after the barrier below, by the second pass and fused_item
    fp.L[b] = L;
    fp.q0[b] = q0;
    if (nq > 0) {
      my_keys += (unsigned long long)L;
      ++my_reqs;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    my_keys += __shfl_xor(my_keys, o);
    my_reqs += __shfl_xor(my_reqs, o);
  }
  if ((tid & 63) == 0 && my_keys) atomicAdd(&fp.keys, my_keys);
  if ((tid & 63) == 0 && my_reqs) atomicAdd(&fp.reqs, my_reqs);
  __syncthreads();
  const long long minc = decode_min_chunk(fp.reqs, a.Hkv, a.target_items);
  const long long chunk = decode_chunk(fp.keys, a.Hkv, a.target_items, minc);
  if (tid == 0) fp.minc = minc;  // read after the barrier at the end
  int4 run = int4{0, 0, 0, 0};  // decode items, partial slots, merge entries
  for (int base = 0; base < a.num_seqs; base += kThreads) {
    const int b = base + tid;
    int4 cnt = int4{0, 0, 0, 0};
    int nq = 0, L = 0, q0 = 0, per = 0, nsplit = 0;
    if (b < a.num_seqs) {
      nq = fp.nq[b];
      L = fp.L[b];
      q0 = fp.q0[b];
      if (nq > 0) {
        decode_split(L, chunk, minc, is_tail_request(b, a.num_seqs), &per, &nsplit);
        cnt.x = a.Hkv * nsplit;
        if (nsplit > 1) {
          cnt.y = a.Hkv * nsplit;
          cnt.z = a.Hkv;
        }
      }
    }
    int4 tot;
    const int4 ex = block_exclusive_scan4<kThreads>(cnt, fp.wsum, &tot);
    if (b < a.num_seqs) {
      fp.doff[b] = run.x + ex.x;
      fp.soff[b] = run.y + ex.y;
      if (blockIdx.x == 0) {
        // one merge entry per (request, KV head) pair, split or not
        int4* me = reinterpret_cast<int4*>(a.merges) + (int64_t)b * a.Hkv;
        const int slot0 = run.y + ex.y;
        for (int kvh = 0; kvh < a.Hkv; ++kvh)
          me[kvh] = nsplit > 1 ? int4{slot0 + kvh * nsplit, nsplit | (nq * a.G) << 16, q0, kvh}
                               : int4{0, 0, 0, kvh};
      }
    }
    run = int4{run.x + tot.x, run.y + tot.y, run.z + tot.z, 0};
  }
  if (tid == 0) fp.doff[a.num_seqs] = run.x;
  __syncthreads();
  return chunk;
}

// Decode item j of the kernel's own plan (the planner kernel's item layout).
__device__ WorkItem fused_item(const MhaArgs& a, const FusedPlan& fp, long long chunk, int j) {
  const int b = find_request(fp.doff, a.num_seqs, j);
  int per, nsplit;
  const int nq = fp.nq[b], L = fp.L[b], q0 = fp.q0[b];
  decode_split(L, chunk, fp.minc, is_tail_request(b, a.num_seqs), &per, &nsplit);
  const int local = j - fp.doff[b];
  const int kvh = local / nsplit, sp = local - kvh * nsplit;
  WorkItem it;
  it.seq = b;
  it.kvh = kvh;
  it.row0 = 0;
  it.nrows = nq * a.G;
  it.kv_begin = sp * per;
  it.kv_end = min(L, sp * per + per);
  it.part = nsplit > 1 ? fp.soff[b] + kvh * nsplit + sp : -1;
  it.q0 = q0;
  it.ctx = L - nq;
  it.nchunk = it.chunk = it.pad = 0;
  return it;
}

// Item j of a single-pass call: request j / Hkv, KV head j % Hkv, all its
// keys (an empty request gets an empty key range and writes nothing).
__device__ WorkItem pair_item(const MhaArgs& a, int j) {
  const int b = j / a.Hkv;
  int nq, L, q0;
  shape_of(a.qsl, a.seq_lens, a.max_pages, a.P, b, &nq, &L, &q0);
  WorkItem it;
  it.seq = b;
  it.kvh = j - b * a.Hkv;
  it.row0 = 0;
  it.nrows = nq * a.G;
  it.kv_begin = 0;
  it.kv_end = nq > 0 ? L : 0;
  it.part = -1;
  it.q0 = q0;
  it.ctx = L - nq;
  it.nchunk = it.chunk = it.pad = 0;
  return it;
}

// Persistent forward kernel: a fixed grid; each workgroup takes items from
// device counters until the planner's item count is reached.
//
// Prefill-mode items (indices below n_pre) are dealt to 8 queues in runs of
// kXcdRun consecutive indices (run r goes to queue r % 8).  Consecutive
// indices are row blocks of one (request, KV head), which read the same keys;
// workgroup w serves queue w % 8 first, and workgroups are placed on the 8
// chiplets (XCDs, each with its own L2) round-robin by index, so the row
// blocks that share keys run side by side on one chiplet and share its L2.
// A workgroup whose queue is empty takes from the next queues, then from the
// decode-mode items.  The item order only affects speed: every index is
// handed out exactly once.
//
// A workgroup runs one loop over prefill-mode items and then one over
// decode-mode items; the two loops keep the register allocation of the two
// item kinds apart.
//
// FUSED (decode-only calls of at most kFusedPlanMax requests): no planner
// kernel runs before this one; every workgroup computes the plan itself
// (fused_plan) and builds its items from it, and the only preceding launch
// resets the queue counter.
// (Decode-only grids run two workgroups per compute unit, except with 192-wide
// keys: their decode item's two steps of key operands in flight need more
// registers than a half share of the register file.)
template <int DK, int DV, bool DECODE_ONLY, bool FUSED = false, bool ALIBI = false>
__global__ __launch_bounds__(DECODE_ONLY ? kThreads : kPrefillThreads,
                             (DECODE_ONLY && DK <= 128) ? 2 : 1)
void mha_forward_kernel(MhaArgs a) {
  static_assert(!FUSED || DECODE_ONLY, "the kernel plans only decode-only calls");
  __shared__ typename FwdLds<DK, DV, DECODE_ONLY>::type sm;
  __shared__ WorkItem s_item;
  __shared__ int s_idx;
  __shared__ typename std::conditional<FUSED, FusedPlan, int>::type fp;
  long long chunk = 0;
  int n_items, n_pre;
  if constexpr (FUSED) {
    n_pre = 0;
    if (a.single_pass) {
      n_items = a.num_seqs * a.Hkv;  // no plan: item j is (request, KV head) pair j
    } else {
      chunk = fused_plan(a, fp);
      n_items = __builtin_amdgcn_readfirstlane(fp.doff[a.num_seqs]);
    }
  } else {
    n_items = a.ctrl->n_items;
    n_pre = a.ctrl->n_pre;
  }
  const int n_dec = n_items - n_pre;
  // A decode-only grid starts workgroup w on decode-mode item w, so the queue
  // hands out the items after the first gridDim.x.
  const int dec_base = DECODE_ONLY ? (int)gridDim.x : 0;
  // The planner zeroes the counter; a call that plans itself finds it zeroed
  // by the previous call's merge kernel, or else takes a fixed item sequence
  // (see Control).  `ready` is not written while this kernel runs, so every
  // workgroup reads the same value.
  // A decode-only call with no more items than workgroups has nothing to
  // hand out: its workgroups skip the claim (an atomic round trip on the
  // path of the call's last item).
  const bool queue = (!DECODE_ONLY || n_dec > (int)gridDim.x) &&
                     (!FUSED || __builtin_amdgcn_readfirstlane(a.ctrl->ready) == kQueueReady);
  int32_t* const counter = queue ? &a.ctrl->work_counter : nullptr;
  int idx;
  WorkItem it;
  const int home = blockIdx.x & 7;
  int drained = 0;  // queues found empty (thread 0)
  // wave 0: decode-mode item j into s_item, lane k copying word k
  auto fetch_decode = [&](int j) {
    const int lane = threadIdx.x;
    if constexpr (FUSED) {
      if (j < n_dec) {
        const WorkItem w = a.single_pass ? pair_item(a, j) : fused_item(a, fp, chunk, j);
        if (lane == 0) s_item = w;
      }
    } else {
      if (j < n_dec && lane < kItemInts)
        reinterpret_cast<int32_t*>(&s_item)[lane] = a.dec_items[(int64_t)j * kItemInts + lane];
    }
    if (lane == 0) s_idx = n_pre + j;
  };
  // Every thread reads the published item; the reads are made visibly
  // uniform (scalar registers), so the item loop and the key loops inside an
  // item compile to scalar branches.
  auto publish = [&]() {
    __syncthreads();
    idx = __builtin_amdgcn_readfirstlane(s_idx);
#pragma unroll
    for (int k = 0; k < kItemInts; ++k)
      reinterpret_cast<int32_t*>(&it)[k] =
          __builtin_amdgcn_readfirstlane(reinterpret_cast<const int32_t*>(&s_item)[k]);
    __syncthreads();
  };
  // wave 0 takes the next index (lane 0's atomics, broadcast to the wave):
  // the prefill-mode queues first, then the decode-mode queue
  auto next = [&]() {
    if (threadIdx.x < 64) {
      int i = -1;
      if constexpr (!DECODE_ONLY) {
        for (int q = 0; q < 8 && i < 0; ++q) {
          const int qx = (home + q) & 7;
          if ((drained >> qx) & 1) continue;
          int j = 0;
          if (threadIdx.x == 0) j = atomicAdd(&a.ctrl->xcd_counter[qx], 1);
          j = __shfl(j, 0);
          const int cand = (8 * (j / kXcdRun) + qx) * kXcdRun + j % kXcdRun;
          if (cand < n_pre) i = cand;
          else drained |= 1 << qx;
        }
      }
      if (i >= 0) {
        const WorkItem w = make_prefill_item(a, i);
        if (threadIdx.x == 0) {
          s_idx = i;
          s_item = w;
        }
      } else {
        int j = 0;
        if (threadIdx.x == 0) j = atomicAdd(counter, 1);
        fetch_decode(__shfl(j, 0) + dec_base);
      }
    }
    publish();
  };
  auto dest = [&]() {
    Dest dst;
    dst.partial = it.part >= 0;
    if (it.nchunk > 1) {
      // chunk partials of a cut request, row-major [token, head, chunk]:
      // partial row pbase + (out_row - q0 Hq) nchunk + chunk
      dst.po = a.cpart_o;
      dst.pl = a.cpart_lse;
      const int64_t r0 = (int64_t)it.part - (int64_t)it.q0 * a.Hq * it.nchunk + it.chunk;
      dst.po_base = r0 * DV;
      dst.po_row = 0;
      dst.po_out = (int64_t)it.nchunk * DV;
      dst.pl_base = r0;
      dst.pl_row = 0;
      dst.pl_out = it.nchunk;
    } else {
      dst.po = a.part_o;
      dst.pl = a.part_lse;
      dst.po_base = (int64_t)it.part * kDecodeRows * DV;
      dst.po_row = DV;
      dst.po_out = 0;
      dst.pl_base = (int64_t)it.part * kDecodeRows;
      dst.pl_row = 1;
      dst.pl_out = 0;
    }
    return dst;
  };
  if constexpr (DECODE_ONLY) {
    if (threadIdx.x < 64) fetch_decode(blockIdx.x);
    publish();
  } else {
    next();
    for (; idx < n_pre && idx < n_items; next())
      run_prefill_item<DK, DV, ALIBI>(a, it, dest(), sm.pre);
  }
  // decode-mode items: each one claims its successor while its epilogue runs
  // (without the queue: the item gridDim.x further on)
  while (idx < n_items) {
    int j;
    if constexpr (DECODE_ONLY) j = run_decode_item<DK, DV, 4, ALIBI>(a, it, dest(), sm, counter);
    else j = run_decode_item_outlined<DK, DV, ALIBI>(a, it, dest(), sm.dec, counter);
    if (threadIdx.x < 64)
      fetch_decode(queue ? __shfl(j, 0) + dec_base : idx - n_pre + (int)gridDim.x);
    publish();
  }
}

// pa_decode_split: one workgroup per (request, KV head, partition).
template <int DK, int DV, bool DEC>
__global__ __launch_bounds__(DEC ? kThreads : kPrefillThreads, DEC ? 2 : 1)
void mha_split_kernel(MhaArgs a) {
  constexpr int D = DV;
  __shared__ typename std::conditional<DEC, LdsDecode<DV, 4>, LdsPrefill<DK, DV>>::type sm;
  const int S = a.num_splits;
  const int s = blockIdx.x % S;
  const int bk = blockIdx.x / S;
  const int kvh = bk % a.Hkv, b = bk / a.Hkv;
  const int L = a.seq_lens[b];
  const int pages = (L + a.P - 1) / a.P;
  const int per = a.P * ((pages + S - 1) / S);
  const long long a0 = (long long)s * per, a1 = a0 + per;
  const int t0 = a0 < L ? (int)a0 : L, t1 = a1 < L ? (int)a1 : L;
  Dest dst;
  dst.partial = true;
  dst.po = a.part_o;
  dst.pl = a.part_lse;
  dst.po_base = ((int64_t)(b * a.Hq + kvh * a.G) * S + s) * D;
  dst.po_row = (int64_t)S * D;
  dst.po_out = 0;
  dst.pl_base = (int64_t)(b * a.Hq + kvh * a.G) * S + s;
  dst.pl_row = S;
  dst.pl_out = 0;
  if (t1 <= t0) {  // empty partition: zeros and -inf
    for (int i = threadIdx.x; i < a.G * D; i += blockDim.x)
      a.part_o[dst.po_base + (int64_t)(i / D) * dst.po_row + (i % D)] = 0.f;
    for (int i = threadIdx.x; i < a.G; i += blockDim.x)
      a.part_lse[dst.pl_base + (int64_t)i * dst.pl_row] = kNegInf;
    return;
  }
  WorkItem it;
  it.seq = b;
  it.kvh = kvh;
  it.row0 = 0;
  it.nrows = a.G;
  it.kv_begin = t0;
  it.kv_end = t1;
  it.part = 0;
  it.q0 = b;
  it.ctx = L - 1;
  it.nchunk = it.chunk = it.pad = 0;
  if constexpr (DEC) run_decode_item<DK, DV, 4>(a, it, dst, sm, nullptr);
  else run_prefill_item<DK, DV>(a, it, dst, sm);
}

// pa_forward_chunked: chunked-context processing ("vLLM AMD ROCm Attention
// Backend Optimization", bullet "Chunked context processing").  Workgroup
// (request b, KV head, row block, chunk s) runs the prefill-mode item of the
// block's rows (up to 256: query tokens x the G heads of the KV head) over
// the keys of chunk s, [s C, (s + 1) C), cut at the key limit of the
// block's last row (causal for pa_forward_chunked; pa_forward's chunked route
// passes its mask).  Its partials are indexed by output row:
// part_o[(out_row S + s) D ..] and part_lse[out_row S + s].  A row that sees
// no key of the chunk gets zeros and -inf: inside the item when another row
// of the block sees the chunk, here when none does.  Requests with no work
// (no new token, or inconsistent lengths) write nothing.
template <int DK, int DV>
__global__ __launch_bounds__(kPrefillThreads, 1) void mha_chunked_kernel(MhaArgs a) {
  constexpr int D = DV;
  __shared__ LdsPrefill<DK, DV> sm;
  const int S = a.num_splits, nblk = a.row_blocks;
  // Workgroups go to the 8 chiplets (XCDs, each with its own L2) round-robin
  // by index.  The index is remapped so that consecutive logical indices sit
  // on one XCD and are dispatched together, and the row blocks of one
  // (request, KV head, chunk), which read the same keys, are consecutive.
  const int n = gridDim.x, q8 = n >> 3, r8 = n & 7;
  const int x = blockIdx.x & 7, p = blockIdx.x >> 3;
  int idx = x * q8 + min(x, r8) + p;
  const int blk = idx % nblk;
  idx /= nblk;
  const int s = idx % S;
  idx /= S;
  const int kvh = idx % a.Hkv, b = idx / a.Hkv;
  int nq, L, q0;
  shape_of(a.qsl, a.seq_lens, a.max_pages, a.P, b, &nq, &L, &q0);
  const int G = a.G, rows = nq * G, row0 = blk * kPrefillRows;
  if (row0 >= rows) return;
  const int nrows = min(kPrefillRows, rows - row0);
  const int ctx = L - nq;
  const long long t0 = (long long)s * a.chunk_keys;
  const int pfx = a.mask == kMaskPrefix ? a.prefix_lens[b] : 0;
  const long long last_lim = min(L, visible_end(a.mask, ctx, (row0 + nrows - 1) / G, pfx));
  const long long t1 = min(last_lim, t0 + a.chunk_keys);
  if (t1 <= t0) {
    constexpr int C4 = D / 4;
    for (int i = threadIdx.x; i < nrows * C4; i += kPrefillThreads) {
      const int r = i / C4, c = 4 * (i - r * C4);
      const int rid = row0 + r, t = rid / G;
      const int64_t out_row = (int64_t)(q0 + t) * a.Hq + kvh * G + (rid - t * G);
      store16(a.part_o + (out_row * S + s) * D + c, u32x4{0, 0, 0, 0});
      if (c == 0) a.part_lse[out_row * S + s] = kNegInf;
    }
    return;
  }
  Dest dst;
  dst.partial = true;
  dst.po = a.part_o;
  dst.pl = a.part_lse;
  dst.po_base = (int64_t)s * D;
  dst.po_row = 0;
  dst.po_out = (int64_t)S * D;
  dst.pl_base = s;
  dst.pl_row = 0;
  dst.pl_out = S;
  WorkItem it;
  it.seq = b;
  it.kvh = kvh;
  it.row0 = row0;
  it.nrows = nrows;
  it.kv_begin = (int)t0;
  it.kv_end = (int)t1;
  it.part = 0;
  it.q0 = q0;
  it.ctx = ctx;
  it.nchunk = it.chunk = it.pad = 0;
  run_prefill_item<DK, DV>(a, it, dst, sm);
}

// Planner: one workgroup of 1024 threads turns (seq_lens, query_start_loc)
// into per-request plans and item / merge offsets; the persistent kernel and
// the merge kernel decode their units from these on the fly.
constexpr int kPlanThreads = 1024;

// Exclusive scan of one int4 per thread over the 1024-thread block: wave-level
// scans with shuffles, then one wave scans the 16 wave totals.
__device__ __forceinline__ void request_shape(const PlanArgs& a, int b, int* nq, int* L, int* q0) {
  shape_of(a.qsl, a.seq_lens, a.max_pages, a.P, b, nq, L, q0);
}

__global__ __launch_bounds__(kPlanThreads) void plan_kernel(PlanArgs a) {
  __shared__ int4 sh[kPlanThreads / 64];
  __shared__ unsigned long long s_dec_keys;
  __shared__ int s_dec_reqs;
  __shared__ int s_doff[kPlanThreads + 1];
  __shared__ ReqPlan s_plan[kPlanThreads];
  const int tid = threadIdx.x;
  const int G = a.G, Hkv = a.Hkv;
  if (tid == 0) {
    s_dec_keys = 0;
    s_dec_reqs = 0;
  }
  __syncthreads();
  // pass 1: total decode-mode keys and requests, which set the partition size
  unsigned long long my_keys = 0;
  int my_reqs = 0;
  int nq_first = 0, L_first = 0, q0_first = 0;  // request tid, reused by pass 2
  for (int b = tid; b < a.B; b += kPlanThreads) {
    int nq, L, q0;
    request_shape(a, b, &nq, &L, &q0);
    if (b == tid) {
      nq_first = nq;
      L_first = L;
      q0_first = q0;
    }
    if (nq > 0 && nq * G <= kDecodeRows) {
      my_keys += (unsigned long long)L;
      ++my_reqs;
    }
  }
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) {
    my_keys += __shfl_xor(my_keys, o);
    my_reqs += __shfl_xor(my_reqs, o);
  }
  if ((tid & 63) == 0 && my_keys) atomicAdd(&s_dec_keys, my_keys);
  if ((tid & 63) == 0 && my_reqs) atomicAdd(&s_dec_reqs, my_reqs);
  __syncthreads();
  const long long minc = decode_min_chunk(s_dec_reqs, Hkv, a.target_items);
  const long long chunk = decode_chunk(s_dec_keys, Hkv, a.target_items, minc);

  // pass 2: per-request counts, exclusive scans, plans
  int4 run = int4{0, 0, 0, 0};  // prefill items, decode items, partial slots, merge entries
  // requests cut into key chunks: candidate partial rows, then chunked
  // requests, their output rows and partial rows
  long long run_cand = 0;
  int4 run_c = int4{0, 0, 0, 0};
  const int Hq = G * Hkv;
  for (int base = 0; base < a.B; base += kPlanThreads) {
    const int b = base + tid;
    ReqPlan rp = {0, 0, 0, 0, 0, 0, 0, 1, 0, {0, 0, 0}};
    int4 cnt = int4{0, 0, 0, 0};
    if (b < a.B) {
      if (base == 0) {
        rp.nq = nq_first;
        rp.L = L_first;
        rp.q0 = q0_first;
      } else {
        request_shape(a, b, &rp.nq, &rp.L, &rp.q0);
      }
    }
    // A prefill-mode request of at least long_keys keys is cut into chunks of
    // chunk_keys keys, in request order while the partial rows fit the budget.
    int nchunk = 1;
    if (b < a.B && a.long_keys > 0 && rp.nq > 0 && rp.nq * G > kDecodeRows &&
        rp.L >= a.long_keys) {
      const int n = (rp.L + a.chunk_keys - 1) / a.chunk_keys;
      if (n > 1 && n <= kMaxSplits) nchunk = n;
    }
    const long long cand = nchunk > 1 ? (long long)rp.nq * Hq * nchunk : 0;
    {
      int4 tot_a;
      // (capped at budget + 1: a capped prefix exceeds the budget exactly when
      // the true one does, and 1024 capped values cannot overflow the scan)
      const int cand_i = (int)min(cand, (long long)a.crow_budget + 1);
      const int4 ex_a = block_exclusive_scan4<kPlanThreads>(int4{cand_i, 0, 0, 0}, sh, &tot_a);
      if (nchunk > 1 && run_cand + ex_a.x + cand_i > a.crow_budget) nchunk = 1;
      run_cand = min(run_cand + tot_a.x, (long long)a.crow_budget + 1);
    }
    rp.nchunk = nchunk;
    {
      int4 tot_c;
      const int4 cc = nchunk > 1 ? int4{1, rp.nq * Hq, rp.nq * Hq * nchunk, 0} : int4{0, 0, 0, 0};
      const int4 ex_c = block_exclusive_scan4<kPlanThreads>(cc, sh, &tot_c);
      if (nchunk > 1) {
        rp.pbase = run_c.z + ex_c.z;
        reinterpret_cast<int4*>(a.cmerge)[run_c.x + ex_c.x] =
            int4{b, run_c.y + ex_c.y, nchunk, rp.pbase};
      }
      run_c = int4{run_c.x + tot_c.x, run_c.y + tot_c.y, run_c.z + tot_c.z, 0};
    }
    if (b < a.B) {
      const int rows = rp.nq * G;
      if (rp.nq > 0 && rows <= kDecodeRows) {
        decode_split(rp.L, chunk, minc, is_tail_request(b, a.B), &rp.per, &rp.nsplit);
        cnt.y = Hkv * rp.nsplit;
        if (rp.nsplit > 1) {
          cnt.z = Hkv * rp.nsplit;
          cnt.w = Hkv;
        }
      } else if (rp.nq > 0) {
        rp.nblk = (rows + kPrefillRows - 1) / kPrefillRows;
        cnt.x = Hkv * rp.nblk * rp.nchunk;
      }
    }
    int4 tot;
    const int4 ex = block_exclusive_scan4<kPlanThreads>(cnt, sh, &tot);
    if (b < a.B) {
      rp.slot0 = run.z + ex.z;
      a.req[b] = rp;
      a.pre_off[b] = run.x + ex.x;
      // one merge entry per (request, KV head) pair; S <= 1: nothing to merge
      int4* me = reinterpret_cast<int4*>(a.merges) + (int64_t)b * Hkv;
      for (int kvh = 0; kvh < Hkv; ++kvh)
        me[kvh] = rp.nsplit > 1 ? int4{rp.slot0 + kvh * rp.nsplit, rp.nsplit | (rp.nq * G) << 16,
                                       rp.q0, kvh}
                                : int4{0, 0, 0, kvh};
    }
    // Decode-mode items of this chunk of requests, written by all threads:
    // item i of the chunk belongs to the last request whose first item is at
    // or before i; a request's items are KV head major, then partition.
    s_doff[tid] = ex.y;
    s_plan[tid] = rp;
    if (tid == kPlanThreads - 1) s_doff[kPlanThreads] = tot.y;
    __syncthreads();
    for (int i = tid; i < tot.y; i += kPlanThreads) {
      int lo = 0;  // largest k with s_doff[k] <= i; empty requests share offsets
      for (int step = kPlanThreads / 2; step >= 1; step >>= 1)
        if (s_doff[lo + step] <= i) lo += step;
      const ReqPlan q = s_plan[lo];
      const int local = i - s_doff[lo];
      const int kvh = local / q.nsplit, sp = local - kvh * q.nsplit;
      const int kb = sp * q.per;
      int4* d4 = reinterpret_cast<int4*>(a.dec_items + (int64_t)(run.y + i) * kItemInts);
      // seq, kvh, row0, nrows | kv_begin, kv_end, part, q0 | ctx, pad
      d4[0] = int4{base + lo, kvh, 0, q.nq * G};
      d4[1] = int4{kb, min(q.L, kb + q.per), q.nsplit > 1 ? q.slot0 + kvh * q.nsplit + sp : -1, q.q0};
      d4[2] = int4{q.L - q.nq, 0, 0, 0};
    }
    __syncthreads();
    run = int4{run.x + tot.x, run.y + tot.y, run.z + tot.z, run.w + tot.w};
  }
  if (tid == 0) {
    a.pre_off[a.B] = run.x;
    a.ctrl->n_pre = run.x;
    a.ctrl->n_items = run.x + run.y;
    a.ctrl->n_cmerge = run_c.x;
    a.ctrl->n_crows = run_c.y;
    a.ctrl->work_counter = 0;
#pragma unroll
    for (int x = 0; x < 8; ++x) a.ctrl->xcd_counter[x] = 0;
  }
}

// Merge of pa_forward's split decode rows.  One wave takes 4 rows of a
// (request, KV head) pair (unit e = pair x merge_groups + row group; a pair
// has at most merge_groups x 4 <= 16 rows, fixed on the host from
// max_q_len); the pair's entry, indexed by the pair itself so that no count
// has to be read first, says whether its rows were split: 16 lanes per row, each with
// D / 16 consecutive columns, folding the partitions in one pass with a
// running log-sum-exp (max, rescaled weight sum, rescaled sum); the loads of
// several partitions are in flight together.
template <int D>
__global__ __launch_bounds__(kThreads) void mha_forward_merge_kernel(MhaArgs a) {
  constexpr int NC = D / 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int rsub = lane >> 4, c0 = (lane & 15) * NC;
  // The attention kernel of this call is done with the queue counters: zero
  // them for the next call and mark them so (see Control).
  if (blockIdx.x == 0 && threadIdx.x < 64) {
    if (threadIdx.x == 0) a.ctrl->work_counter = 0;
    if (threadIdx.x < 8) a.ctrl->xcd_counter[threadIdx.x] = 0;
    if (threadIdx.x == 0) a.ctrl->ready = kQueueReady;  // seen with the zeros by the next kernel
  }
  const int groups = a.merge_groups;
  const int stride = gridDim.x * (kThreads / 64);
  const int64_t units = (int64_t)a.num_seqs * a.Hkv * groups;
  for (int64_t e = blockIdx.x * (kThreads / 64) + wv; e < units; e += stride) {
    const int4 me = reinterpret_cast<const int4*>(a.merges)[e / groups];
    const int slot0 = me.x, S = me.y & 0xffff, nrows = me.y >> 16, q0 = me.z, kvh = me.w;
    if (S <= 1) continue;  // the pair's rows were written whole
    {
      const int row = 4 * (e % groups) + rsub;
      if (row >= nrows) continue;
      float m = kNegInf, wsum = 0.f;
      float o[NC];
#pragma unroll
      for (int c = 0; c < NC; ++c) o[c] = 0.f;
#pragma unroll 8
      for (int sp = 0; sp < S; ++sp) {
        const int64_t slot = slot0 + sp;
        const float ls = a.part_lse[slot * kDecodeRows + row];
        const floatx4* po = reinterpret_cast<const floatx4*>(a.part_o + (slot * kDecodeRows + row) * D + c0);
        floatx4 v[NC / 4];
#pragma unroll
        for (int c = 0; c < NC / 4; ++c) v[c] = po[c];  // finite for every written partition
        const float mn = fmaxf(m, ls);
        const float f = mn == kNegInf ? 1.f : __expf(m - mn);   // rescale of the running sums
        const float w = ls == kNegInf ? 0.f : __expf(ls - mn);  // weight of this partition
        m = mn;
        wsum = fmaf(wsum, f, w);
#pragma unroll
        for (int c = 0; c < NC / 4; ++c) {
          o[4 * c] = fmaf(w, v[c][0], o[4 * c] * f);
          o[4 * c + 1] = fmaf(w, v[c][1], o[4 * c + 1] * f);
          o[4 * c + 2] = fmaf(w, v[c][2], o[4 * c + 2] * f);
          o[4 * c + 3] = fmaf(w, v[c][3], o[4 * c + 3] * f);
        }
      }
      float inv = wsum > 0.f ? 1.f / wsum : 0.f;
      float lse = wsum > 0.f ? m + __logf(wsum) : kNegInf;
      const int t = row / a.G;
      const int head = kvh * a.G + (row - t * a.G);
      const int64_t out_row = (int64_t)(q0 + t) * a.Hq + head;
      if (a.sinks) inv *= fold_sink(a.sinks[head], &lse);
      __bf16* op = (__bf16*)a.out + out_row * D + c0;
#pragma unroll
      for (int c = 0; c < NC; c += 4)
        *reinterpret_cast<u32x2*>(op + c) =
            u32x2{pack_bf16x2(o[c] * inv, o[c + 1] * inv), pack_bf16x2(o[c + 2] * inv, o[c + 3] * inv)};
      if ((lane & 15) == 0 && a.lse) a.lse[out_row] = lse;
    }
  }
}

// Merge of the key chunks of the requests the planner cut: one wave per 4
// output rows of the concatenated rows of those requests (16 lanes per row,
// D / 16 consecutive columns each), folding the request's nchunk partial rows
// with a running log-sum-exp, then the sink logit if any.
template <int D>
__global__ __launch_bounds__(kThreads) void mha_chunk_merge_kernel(MhaArgs a) {
  constexpr int NC = D / 16;
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int c0 = (lane & 15) * NC;
  const int n_cm = a.ctrl->n_cmerge, n_rows = a.ctrl->n_crows;
  const int4* cm = reinterpret_cast<const int4*>(a.cmerge);
  const int stride = gridDim.x * (kThreads / 64);
  for (int u = blockIdx.x * (kThreads / 64) + wv; 4 * u < n_rows; u += stride) {
    const int r = 4 * u + (lane >> 4);
    if (r >= n_rows) continue;
    int lo = 0, hi = n_cm - 1;  // last entry whose first row is <= r
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (cm[mid].y <= r) lo = mid; else hi = mid - 1;
    }
    const int4 e = cm[lo];
    const int lr = r - e.y, nchunk = e.z;
    const int j = lr / a.Hq, head = lr - j * a.Hq;
    const int64_t out_row = (int64_t)(a.req[e.x].q0 + j) * a.Hq + head;
    const int64_t p0 = (int64_t)e.w + (int64_t)lr * nchunk;
    float m = kNegInf, wsum = 0.f;
    float o[NC];
#pragma unroll
    for (int c = 0; c < NC; ++c) o[c] = 0.f;
#pragma unroll 4
    for (int sp = 0; sp < nchunk; ++sp) {
      const float ls = a.cpart_lse[p0 + sp];
      const floatx4* po = reinterpret_cast<const floatx4*>(a.cpart_o + (p0 + sp) * D + c0);
      floatx4 v[NC / 4];
#pragma unroll
      for (int c = 0; c < NC / 4; ++c) v[c] = po[c];
      const float mn = fmaxf(m, ls);
      const float f = mn == kNegInf ? 1.f : __expf(m - mn);
      const float w = ls == kNegInf ? 0.f : __expf(ls - mn);
      m = mn;
      wsum = fmaf(wsum, f, w);
#pragma unroll
      for (int c = 0; c < NC / 4; ++c)
#pragma unroll
        for (int k = 0; k < 4; ++k) o[4 * c + k] = fmaf(w, v[c][k], o[4 * c + k] * f);
    }
    float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    float lse = wsum > 0.f ? m + __logf(wsum) : kNegInf;
    if (a.sinks) inv *= fold_sink(a.sinks[head], &lse);
    __bf16* op = (__bf16*)a.out + out_row * D + c0;
#pragma unroll
    for (int c = 0; c < NC; c += 4)
      *reinterpret_cast<u32x2*>(op + c) =
          u32x2{pack_bf16x2(o[c] * inv, o[c + 1] * inv), pack_bf16x2(o[c + 2] * inv, o[c + 3] * inv)};
    if ((lane & 15) == 0 && a.lse) a.lse[out_row] = lse;
  }
}

}  // namespace

hipError_t launch_mha_chunk_merge(const MhaArgs& a, int Dv, int grid, hipStream_t s) {
  if (Dv == 128) hipLaunchKernelGGL(mha_chunk_merge_kernel<128>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (Dv == 64) hipLaunchKernelGGL(mha_chunk_merge_kernel<64>, dim3(grid), dim3(kThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_plan(const PlanArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(plan_kernel, dim3(1), dim3(kPlanThreads), 0, s, a);
  return hipGetLastError();
}

// The bf16 head-dim pairs (Dqk, Dv) the MHA kernels are built for, by variant
// index (see mha_variant).
template <typename F>
hipError_t with_dims(int variant, F&& f) {
  switch (variant) {
    case 0: return f(std::integral_constant<int, 64>(), std::integral_constant<int, 64>());
    case 1: return f(std::integral_constant<int, 128>(), std::integral_constant<int, 128>());
    case 2: return f(std::integral_constant<int, 192>(), std::integral_constant<int, 128>());
  }
  return hipErrorInvalidValue;
}

int mha_variant(int dk, int dv) {
  if (dk == 64 && dv == 64) return 0;
  if (dk == 128 && dv == 128) return 1;
  if (dk == 192 && dv == 128) return 2;
  return -1;
}

hipError_t mha_occupancy(int variant, bool decode_only, int* blocks_per_cu) {
  return with_dims(variant, [&](auto dk, auto dv) {
    constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
    const void* f = decode_only ? (const void*)mha_forward_kernel<DK, DV, true>
                                : (const void*)mha_forward_kernel<DK, DV, false>;
    return hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks_per_cu, f,
                                                        decode_only ? kThreads : kPrefillThreads, 0);
  });
}

hipError_t launch_mha_forward(const MhaArgs& a, int variant, bool decode_only, bool alibi,
                              int grid, hipStream_t s) {
  return with_dims(variant, [&](auto dk, auto dv) {
    constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
    if (alibi) {
      if constexpr (DK <= 128) {  // ALiBi kernels are built for head dims 64 and 128
        if (decode_only)
          hipLaunchKernelGGL((mha_forward_kernel<DK, DV, true, false, true>), dim3(grid),
                             dim3(kThreads), 0, s, a);
        else
          hipLaunchKernelGGL((mha_forward_kernel<DK, DV, false, false, true>), dim3(grid),
                             dim3(kPrefillThreads), 0, s, a);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    if (decode_only)
      hipLaunchKernelGGL((mha_forward_kernel<DK, DV, true>), dim3(grid), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((mha_forward_kernel<DK, DV, false>), dim3(grid), dim3(kPrefillThreads), 0,
                         s, a);
    return hipGetLastError();
  });
}

hipError_t launch_mha_forward_fused(const MhaArgs& a, int variant, bool alibi, int grid,
                                    hipStream_t s) {
  return with_dims(variant, [&](auto dk, auto dv) {
    constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
    if (alibi) {
      if constexpr (DK <= 128) {
        hipLaunchKernelGGL((mha_forward_kernel<DK, DV, true, true, true>), dim3(grid),
                           dim3(kThreads), 0, s, a);
        return hipGetLastError();
      }
      return hipErrorInvalidValue;
    }
    hipLaunchKernelGGL((mha_forward_kernel<DK, DV, true, true>), dim3(grid), dim3(kThreads), 0, s,
                       a);
    return hipGetLastError();
  });
}

hipError_t launch_mha_forward_merge(const MhaArgs& a, int Dv, int grid, hipStream_t s) {
  if (Dv == 128) hipLaunchKernelGGL(mha_forward_merge_kernel<128>, dim3(grid), dim3(kThreads), 0, s, a);
  else if (Dv == 64) hipLaunchKernelGGL(mha_forward_merge_kernel<64>, dim3(grid), dim3(kThreads), 0, s, a);
  else return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_mha_split(const MhaArgs& a, int variant, hipStream_t s) {
  const int64_t blocks = (int64_t)a.num_seqs * a.Hkv * a.num_splits;
  if (blocks <= 0) return hipSuccess;
  const bool dec = a.G <= kDecodeRows;
  return with_dims(variant, [&](auto dk, auto dv) {
    constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
    if (dec)
      hipLaunchKernelGGL((mha_split_kernel<DK, DV, true>), dim3(blocks), dim3(kThreads), 0, s, a);
    else
      hipLaunchKernelGGL((mha_split_kernel<DK, DV, false>), dim3(blocks), dim3(kPrefillThreads), 0,
                         s, a);
    return hipGetLastError();
  });
}

hipError_t launch_mha_chunked(const MhaArgs& a, int variant, hipStream_t s) {
  const int64_t blocks = (int64_t)a.num_seqs * a.Hkv * a.row_blocks * a.num_splits;
  if (blocks <= 0) return hipSuccess;
  return with_dims(variant, [&](auto dk, auto dv) {
    constexpr int DK = decltype(dk)::value, DV = decltype(dv)::value;
    hipLaunchKernelGGL((mha_chunked_kernel<DK, DV>), dim3(blocks), dim3(kPrefillThreads), 0, s, a);
    return hipGetLastError();
  });
}

FwdWorkspace fwd_workspace_layout(int B, int Hkv, int D, int target_items, int64_t long_rows) {
  FwdWorkspace w;
  auto align = [](size_t x) { return (x + 255) & ~(size_t)255; };
  // Decode-mode items (and so partial slots) of one call: a (request, KV head)
  // pair of L keys gets at most ceil(L / ck) <= L / ck + 1 partitions, with
  // ck >= chunk / 2 (the tail rule) and chunk >= the call's decode keys x Hkv
  // / target_items; summed over the pairs, at most 2 target_items + B Hkv.
  w.cap_slots = std::min<int64_t>((int64_t)Hkv * B * kMaxFwdSplits,
                                  2 * (int64_t)target_items + (int64_t)Hkv * B);
  size_t off = 0;
  w.ctrl_off = off;
  off = align(off + sizeof(Control));
  w.req_off = off;
  off = align(off + (size_t)B * sizeof(ReqPlan));
  w.pre_off = off;
  off = align(off + (size_t)(B + 1) * sizeof(int32_t));
  w.items_off = off;
  off = align(off + (size_t)w.cap_slots * kItemInts * sizeof(int32_t));
  w.merges_off = off;
  off = align(off + (size_t)B * Hkv * 4 * sizeof(int32_t));
  w.plse_off = off;
  off = align(off + (size_t)w.cap_slots * kDecodeRows * sizeof(float));
  w.po_off = off;
  off = align(off + (size_t)w.cap_slots * kDecodeRows * D * sizeof(float));
  w.crow_budget = (int32_t)std::min<int64_t>(std::max<int64_t>(long_rows, 0), INT32_MAX / 4);
  w.cmerge_off = off;
  off = align(off + (w.crow_budget > 0 ? (size_t)B * 4 * sizeof(int32_t) : 0));
  w.cpl_off = off;
  off = align(off + (size_t)w.crow_budget * sizeof(float));
  w.cpo_off = off;
  off = align(off + (size_t)w.crow_budget * D * sizeof(float));
  w.total = off;
  return w;
}

}  // namespace pa
