// Device helpers shared by the attention kernels (bf16 and FP8): LDS DMA and waits, LDS
// addressing, cross-lane reductions, the online-softmax state and the key-block sequences.
#pragma once

#include "common.h"

namespace recap {

typedef const __attribute__((address_space(4))) int32_t* cptr_i32;
typedef const __attribute__((address_space(4))) uint8_t* cptr_u8;
typedef const __attribute__((address_space(4))) uint32_t* cptr_u32;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) void*)p;
}
// 16 bytes per lane global -> LDS (global_load_lds_dwordx4, SGPR base + 32-bit lane offset);
// lane i lands at lds_dst + 16 * i. Written as asm with no output register so the compiler does
// not insert a full vmcnt wait before every later LDS read; completion is tracked by hand with
// wait_vmem<> in issue order. M0 (the LDS base operand, read at issue) is restored afterwards.
__device__ __forceinline__ void load_lds16(const void* base_uniform, uint32_t voff,
                                           uint32_t lds_dst_uniform) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      // readfirstlane: a no-op for a value the compiler keeps in a scalar register, and a
      // move back to one where it has merged uniform values into a vector register
      : "s"(__builtin_amdgcn_readfirstlane(lds_dst_uniform)), "v"(voff), "s"(base_uniform)
      : "memory");
}
// 16-byte LDS read at a byte address
__device__ __forceinline__ bf16x8 lds_read16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) bf16x8*>((size_t)addr);
}
// Uniform LDS byte address of a __shared__ buffer (scalar register)
__device__ __forceinline__ uint32_t lds_base(const void* p) {
  return __builtin_amdgcn_readfirstlane(lds_offset(p));
}

// Hide a value from the optimiser so precomputed per-lane offsets are used as they are
// (otherwise the address arithmetic gets re-derived per tile with 64-bit vector multiplies).
__device__ __forceinline__ uint32_t opaque(uint32_t x) {
  asm volatile("" : "+v"(x));
  return x;
}
__device__ __forceinline__ float opaque_f(float x) {
  asm volatile("" : "+v"(x));
  return x;
}

// ------------------------------------------------------------------------------------------
// Block sequences walked by one attention phase. first()/next() return a key-block index or
// -1 when the sequence is exhausted. All values are uniform across the work-group.
// ------------------------------------------------------------------------------------------
struct ListSeq {  // kept blocks, in list order
  const int32_t* lst;
  int n, c, M;
  __device__ int at(int i) const { return min(max(((cptr_i32)lst)[i], 0), M - 1); }
  __device__ int first() { c = 0; return n > 0 ? at(0) : -1; }
  __device__ int next() { ++c; return c < n ? at(c) : -1; }
};
struct AllSeq {  // every block once, starting at `start` and wrapping around
  int c, M, start;
  __device__ int first() { c = 0; return M > 0 ? start : -1; }
  __device__ int next() {
    ++c;
    if (c >= M) return -1;
    const int j = start + c;
    return j >= M ? j - M : j;
  }
};

struct UnionSeq {  // blocks set in either of two LDS bitmaps, ascending
  const uint32_t* a;
  const uint32_t* b;
  int M, j;
  __device__ int scan(int from) {
    const int nw = (M + 31) >> 5;
    for (int w = from >> 5; w < nw; ++w) {
      uint32_t m = a[w] | b[w];
      if (w == (from >> 5)) m &= ~0u << (from & 31);
      if (m != 0u) return w * 32 + __builtin_ctz(m);
    }
    return -1;
  }
  __device__ int first() { j = scan(0); return j; }
  __device__ int next() { j = j + 1 < M ? scan(j + 1) : -1; return j; }
};

struct SoftmaxState {
  float m, l;  // running max (log2 units, may lag the true max by < kLazy) and per-lane sum
};

// Rescale the running state only when some lane's max grows by more than kLazy (log2 units):
// the probabilities of a row are exp2(x - m) for a per-row m that may lag its true max by up
// to kLazy, so they stay below 2^kLazy (exact in fp32 / bf16 range); the final O / l is the
// same quantity for any m.
constexpr float kLazy = 8.0f;

// max(a, b, c) in one instruction (fmaxf on matrix-core results would first canonicalise
// every input against signalling NaNs, tripling the instruction count). The compiler inserts
// no wait states before inline asm: a matrix-core result must first be read by a compiler-
// generated instruction (which gets the wait states a vector read of that result needs), so a
// chain over a product's result starts with fmaxf and continues with max3.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

__device__ __forceinline__ float cross_half_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float cross_half_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Position in a block sequence: key block j (< 0: none) and its 64-key sub-tile st.
struct TileCur {
  int j, st;
};
template <class Seq>
__device__ __forceinline__ TileCur advance(TileCur c, Seq& seq, int block, int N) {
  if (c.j < 0) return c;
  const int st = c.st + 1;
  if (st * kKeyTile >= min(block, N - c.j * block)) return TileCur{seq.next(), 0};
  return TileCur{c.j, st};
}

}  // namespace recap
