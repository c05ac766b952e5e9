// pa_device.h — device-side building blocks shared by the gfx950 kernels:
// vector types, the bf16 MFMA, 16-byte loads, bf16 packing, wave reductions.
//
// Lane layout of v_mfma_f32_16x16x32_bf16 (64 lanes, lane l, group g = l / 16,
// r = l % 16):  A[m][k] (16 x 32): lane holds A[r][8g .. 8g+7];
//               B[k][n] (32 x 16): lane holds B[8g .. 8g+7][r];
//               D[m][n] (16 x 16): lane holds D[4g .. 4g+3][r].
// The contraction index only has to be laid out the same way in A and B, so
// the kernels are free to permute which key / column a K-slot stands for.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) float floatx4;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;
typedef __attribute__((ext_vector_type(16))) float floatx16;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

__device__ __forceinline__ floatx4 mfma_bf16(const bf16x8& a, const bf16x8& b,
                                             const floatx4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_32x32x16_bf16: A[m][k] (32 x 16): lane holds A[l % 32][8 (l / 32) ..];
// B[k][n]: lane holds B[8 (l / 32) ..][l % 32]; D[m][n]: lane holds, in element
// v, D[8 (v / 4) + 4 (l / 32) + v % 4][l % 32].
__device__ __forceinline__ floatx16 mfma32_bf16(const bf16x8& a, const bf16x8& b,
                                                const floatx16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Direct HBM -> LDS copy of 16 bytes per lane (global_load_lds_dwordx4): lane
// L's bytes land at lds_wave_base + 16 L; lds_wave_base must be the same for
// the whole wave.  Issued through inline assembly so that the compiler neither
// waits for these copies at every barrier nor counts them: the caller waits
// with wait_vmcnt<N>() and must not expect compiler-inserted waits for them.
//
// The instruction takes its LDS address from m0, a register the compiler
// reserves (a clobber of m0 is ignored).  So the statement saves m0 in a
// scalar register of its own, writes the address, waits the one wait state an
// SALU write of m0 needs before an LDS-DMA instruction reads it, issues the
// copy and puts the saved value back: whatever the compiler keeps in m0
// survives.
__device__ __forceinline__ void lds_dma16_m0(const void* gsrc, uint32_t lds_wave_base) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(lds_wave_base), "v"(gsrc)
      : "memory");
}

// N copies as lds_dma16_m0, issued back to back with m0 saved once before
// them and restored once after them (two scalar instructions per copy fewer
// than N single calls).  gsrc[i] goes to lds_wave_base[i].
__device__ __forceinline__ void lds_dma16_m0_x2(const void* g0, const void* g1, uint32_t l0,
                                                uint32_t l1) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %4\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g0), "v"(g1), "s"(l0), "s"(l1)
      : "memory");
}
__device__ __forceinline__ void lds_dma16_m0_x4(const void* g0, const void* g1, const void* g2,
                                                const void* g3, uint32_t l0, uint32_t l1,
                                                uint32_t l2, uint32_t l3) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %5\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, off\n\t"
      "s_mov_b32 m0, %6\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %7\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %3, off\n\t"
      "s_mov_b32 m0, %8\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %4, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(g0), "v"(g1), "v"(g2), "v"(g3), "s"(l0), "s"(l1), "s"(l2), "s"(l3)
      : "memory");
}
// The N copies gsrc[0..N) -> lds_wave_base[0..N) in groups of 4, 2 and 1.
template <int N>
__device__ __forceinline__ void lds_dma16_m0_seq(const void* const* g, const uint32_t* l) {
  if constexpr (N >= 4) {
    lds_dma16_m0_x4(g[0], g[1], g[2], g[3], l[0], l[1], l[2], l[3]);
    lds_dma16_m0_seq<N - 4>(g + 4, l + 4);
  } else if constexpr (N >= 2) {
    lds_dma16_m0_x2(g[0], g[1], l[0], l[1]);
    lds_dma16_m0_seq<N - 2>(g + 2, l + 2);
  } else if constexpr (N == 1) {
    lds_dma16_m0(g[0], l[0]);
  }
}

// A pointer every lane holds the same value of, made visibly uniform (scalar
// registers): loads through it with uniform indices become scalar loads,
// which the copy waits do not count.
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (T*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

// s_waitcnt immediate for "no vector-memory operation in flight" (gfx9
// encoding: vmcnt bits [3:0] and [15:14] zero, expcnt [6:4] and lgkmcnt [11:8]
// at their maxima, i.e. not waited for).  Passed to __builtin_amdgcn_s_waitcnt,
// which the compiler's own wait insertion takes into account.
constexpr int kWaitVmcnt0 = 0x0F70;

// Wait until at most N vector-memory operations of this wave are in flight.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt immediate");
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

__device__ __forceinline__ u32x4 load16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}

__device__ __forceinline__ void store16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

__device__ __forceinline__ bf16x8 as_bf16x8(const u32x4& v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ u32x4 as_u32x4(const bf16x8& v) {
  return __builtin_bit_cast(u32x4, v);
}

// bf16 (raw 16-bit pattern) -> float, exact.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Lane exchanges within the VALU (v_permlane32_swap / v_permlane16_swap: no
// LDS round trip, unlike a generic shuffle).  xor32_pair returns the values
// of lanes l and l ^ 32 in a fixed order (lower half's first), so that both
// lanes of a pair combine them into the same bits.
struct LanePair {
  float lo, hi;
};
__device__ __forceinline__ LanePair xor32_pair(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
// The same for lanes l and l ^ 16 (16-lane rows 0 / 1 and 2 / 3 paired).
__device__ __forceinline__ LanePair xor16_pair(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return LanePair{__uint_as_float(r[0]), __uint_as_float(r[1])};
}
__device__ __forceinline__ float xor32_max(float v) {
  const LanePair p = xor32_pair(v);
  return fmaxf(p.lo, p.hi);
}
__device__ __forceinline__ float xor32_sum(float v) {
  const LanePair p = xor32_pair(v);
  return p.lo + p.hi;
}

// Butterfly reductions across the 4 lane groups (lanes l, l^16, l^32, l^48)
// that hold the same MFMA row.
__device__ __forceinline__ float group_max4(float v) {
  const LanePair p = xor16_pair(v);
  return xor32_max(fmaxf(p.lo, p.hi));
}
__device__ __forceinline__ float group_sum4(float v) {
  const LanePair p = xor16_pair(v);
  return xor32_sum(p.lo + p.hi);
}

// Full 64-lane reductions.
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// Zero the bf16 elements i (0..7) of a 16-byte group whose key index
// key0 + i is >= limit.
__device__ __forceinline__ u32x4 zero_tail8(u32x4 v, int key0, int limit) {
  int n = limit - key0;  // number of valid leading elements
  if (n >= 8) return v;
  uint32_t w[4] = {v[0], v[1], v[2], v[3]};
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t m = 0;
    if (2 * j < n) m |= 0x0000ffffu;
    if (2 * j + 1 < n) m |= 0xffff0000u;
    w[j] &= m;
  }
  return u32x4{w[0], w[1], w[2], w[3]};
}

// One unit of work of the MHA kernels: rows = (new token x query head of one
// KV head) of one request over the key range [kv_begin, kv_end).
struct WorkItem {
  int32_t seq;       // request
  int32_t kvh;       // KV head
  int32_t row0;      // first row; row index = token_in_request * G + head_in_group
  int32_t nrows;     // rows in the item
  int32_t kv_begin;  // first key (multiple of 8)
  int32_t kv_end;    // one past the last key any row of the item may see
  int32_t part;      // < 0: write the final output; >= 0: partial slot, or for a
                     // chunked prefill-mode item its request's first partial row
  int32_t q0;        // row of the request's first new token in q / out
  int32_t ctx;       // cached keys before the new tokens (seq_len - q_len)
  int32_t nchunk;    // prefill-mode item of a request cut into key chunks: their
                     // number (0 otherwise)
  int32_t chunk;     // ... and this item's chunk
  int32_t pad;
};

// Per-request plan written by the planner kernel of pa_forward.
struct ReqPlan {
  int32_t nq;      // new tokens (0: the request gets no work)
  int32_t L;       // keys
  int32_t q0;      // first query row
  int32_t nblk;    // prefill-mode row blocks per KV head (0 for decode-mode requests)
  int32_t nsplit;  // decode-mode key partitions per KV head (0 for prefill-mode requests)
  int32_t per;     // keys per partition
  int32_t slot0;   // first partial slot (requests with nsplit > 1)
  int32_t nchunk;  // prefill-mode key chunks (1: not cut)
  int32_t pbase;   // first chunk-partial row (requests with nchunk > 1)
  int32_t pad[3];
};

// Control block at the start of the pa_forward workspace.
//
// The queue counters are zero when a call starts: the planner kernel zeroes
// them, and the merge kernel that ends every call zeroes them again for the
// next call and then writes kQueueReady into `ready`.  A decode-only call,
// which runs no planner, claims items from the counter only when it finds
// that marker (a workspace the library has not used yet holds anything);
// without it every workgroup takes the fixed sequence of items w, w + grid,
// w + 2 grid ... instead, which needs no counter.
constexpr uint32_t kQueueReady = 0x51a9e7c3u;
struct Control {
  int32_t n_pre;            // prefill-mode items; item indices [0, n_pre)
  int32_t n_items;          // all items; decode-mode items are [n_pre, n_items)
  int32_t unused0;          // (free; keeps the layout)
  int32_t work_counter;     // decode-mode items claimed from the queue
  int32_t xcd_counter[8];   // next entry of each prefill-mode item queue
  uint32_t ready;           // kQueueReady: the counters above are zero
  int32_t n_cmerge;         // prefill-mode requests cut into key chunks
  int32_t n_crows;          // their output rows (new tokens x query heads)
  int32_t pad[49];
};

}  // namespace pa
