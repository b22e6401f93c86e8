// Block-sparse and dense attention on gfx950 (bf16 MFMA, fp32 online softmax).
//
// RECAP (paperpeel.com/paper/2610.26244) Sec. 4.1 computes the selected block interactions
// with a block-sparse kernel and dense refreshes with a dense one; Sec. 3.2 adds the cached
// dense refinement to the fresh sparse estimate. This file holds one kernel template for
// three modes:
//   kSparse   walk the compacted kept-block list; optional fused O += c_h * R epilogue;
//   kDense    walk every key block;
//   kCapture  walk the kept list, snapshot the normalised sparse output, continue over the
//             remaining blocks, then write O_dense and R = O_dense - O_sparse.
//
// Layout of the work (one work-group per query block of `block` rows, one wavefront per 32
// query rows, 64-key tiles):
//   S^T = K Q^T  with v_mfma_f32_32x32x16_bf16: A = K tile from LDS (row = key), B = Q^T held
//                in registers for the whole kernel (column = query). Lane (n, half) of the
//                result owns query n and 16 keys of each 32-key tile, so the row max needs a
//                single cross-half exchange and the row sum stays per lane until the end.
//   O^T += V^T P^T  A = V^T tile from LDS (row = head dim), B = P^T taken straight from the
//                S^T registers after bf16 rounding. The 16-key contraction step pairs lane
//                half 0 with keys {0-3, 8-11} and half 1 with {4-7, 12-15}, which is what
//                the S^T accumulator already holds; V^T is packed with the same key order so
//                each A fragment is one 16-byte LDS read.
// K and V^T tiles go global -> LDS directly (global_load_lds, 16 bytes per lane) into two
// separate buffers: the load of the next K tile overlaps softmax + PV of the current tile,
// the load of the next V^T tile overlaps the next QK^T.
#include "common.h"

namespace recap {

typedef const __attribute__((address_space(1))) void* gptr_t;
typedef __attribute__((address_space(3))) void* lptr_t;
typedef const __attribute__((address_space(4))) int32_t* cptr_i32;

__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}
template <int N>
__device__ __forceinline__ void wait_vmem() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
__device__ __forceinline__ void load_lds16(const void* src, void* lds_dst_uniform) {
  __builtin_amdgcn_global_load_lds((gptr_t)src, (lptr_t)lds_dst_uniform, 16, 0, 0);
}

// Key order inside each 16-key group of packed V^T: position pos holds key swap23(pos).
__device__ __forceinline__ int swap23(int p) { return (p & 3) | ((p & 4) << 1) | ((p & 8) >> 1); }

// ------------------------------------------------------------------------------------------
// V -> packed V^T [B*H][D][npad] (npad = M * block, zero past N), keys permuted inside each
// 16-key group as described above. One work-group per (b*h, 64-key tile), staged through LDS.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pack_vt_kernel(const bf16_t* __restrict__ v, Strides st,
                                                      int H, int N, int npad,
                                                      bf16_t* __restrict__ vt) {
  constexpr int CH = D / 8;
  __shared__ bf16_t tile[64][D + 2];
  const int ntile = npad / 64;
  const int bh = blockIdx.x / ntile, kt = blockIdx.x - bh * ntile;
  const int b = bh / H, h = bh - b * H;
  const bf16_t* src = v + b * st.b + h * st.h;
  const int key0 = kt * 64;
  for (int s = threadIdx.x; s < 64 * CH; s += 256) {
    const int key = s / CH, c = s - key * CH;
    bf16x8 x = {};
    if (key0 + key < N) x = *reinterpret_cast<const bf16x8*>(src + (int64_t)(key0 + key) * st.n + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[key][c * 8 + e] = x[e];
  }
  __syncthreads();
  bf16_t* dst = vt + (int64_t)bh * D * npad + key0;
  for (int s = threadIdx.x; s < D * 8; s += 256) {
    const int d = s >> 3, c = s & 7;
    bf16x8 y;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = c * 8 + e;
      y[e] = tile[(pos & ~15) | swap23(pos & 15)][d];
    }
    *reinterpret_cast<bf16x8*>(dst + (int64_t)d * npad + c * 8) = y;
  }
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
struct AllSeq {  // every block, ascending
  int c, M;
  __device__ int first() { c = 0; return M > 0 ? 0 : -1; }
  __device__ int next() { ++c; return c < M ? c : -1; }
};
struct ComplementSeq {  // blocks whose bit is clear, ascending
  const uint32_t* bits;
  int c, M;
  __device__ int scan(int j) {
    while (j < M && ((bits[j >> 5] >> (j & 31)) & 1u)) ++j;
    return j < M ? j : -1;
  }
  __device__ int first() { c = scan(0); return c; }
  __device__ int next() { c = scan(c + 1); return c; }
};

template <int D, int NW>
struct Tiles {
  static constexpr int CH = D / 8;        // 16-byte chunks in a K row
  static constexpr int LD = CH / NW;      // global->LDS instructions per wave per tensor tile
  static constexpr int TILE_BYTES = 64 * D * 2;
};

template <int D, int NW>
__device__ __forceinline__ void issue_k(unsigned char* kbuf, const bf16_t* kp, int64_t sn, int N,
                                        int key0, int wave, int lane) {
  constexpr int CH = Tiles<D, NW>::CH, LD = Tiles<D, NW>::LD;
#pragma unroll
  for (int it = 0; it < LD; ++it) {
    const int slot0 = (wave * LD + it) * 64;
    const int slot = slot0 + lane;
    const int key = slot / CH;
    const int c = (slot % CH) ^ (key & (CH - 1));
    const bf16_t* src = kp + (int64_t)min(key0 + key, N - 1) * sn + c * 8;
    load_lds16(src, kbuf + slot0 * 16);
  }
}

template <int D, int NW>
__device__ __forceinline__ void issue_v(unsigned char* vbuf, const bf16_t* vtp, int npad,
                                        int key0, int wave, int lane) {
  constexpr int LD = Tiles<D, NW>::LD;
#pragma unroll
  for (int it = 0; it < LD; ++it) {
    const int slot0 = (wave * LD + it) * 64;
    const int slot = slot0 + lane;
    const int d = slot >> 3;
    const int c = (slot & 7) ^ ((d >> 1) & 7);
    const bf16_t* src = vtp + (int64_t)d * npad + key0 + c * 8;
    load_lds16(src, vbuf + slot0 * 16);
  }
}

struct SoftmaxState {
  float m, l;
};

// One attention phase over a block sequence, continuing the online-softmax state (m, l, o).
template <int D, int NW, class Seq>
__device__ __forceinline__ void attend_phase(Seq& seq, unsigned char* kbuf, unsigned char* vbuf,
                                             const bf16_t* kp, const bf16_t* vtp, int64_t sn,
                                             int N, int block, int npad, float scale_log2,
                                             const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                             SoftmaxState& sm, int wave, int lane) {
  constexpr int CH = Tiles<D, NW>::CH, LD = Tiles<D, NW>::LD;
  const int n = lane & 31, half = lane >> 5;
  int j = seq.first();
  if (j < 0) return;
  int st = 0;
  issue_k<D, NW>(kbuf, kp, sn, N, j * block, wave, lane);
  issue_v<D, NW>(vbuf, vtp, npad, j * block, wave, lane);
  while (true) {
    const int key0 = j * block + st * kKeyTile;
    int jn = j, stn = st + 1;
    if (stn * kKeyTile >= min(block, N - j * block)) {
      jn = seq.next();
      stn = 0;
    }
    const bool has_next = jn >= 0;

    // ---- S^T = K Q^T ----
    wait_vmem<LD>();  // this wave's K(t) landed (V(t) may still be in flight)
    lds_barrier();    // ... and every other wave's
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int c = ks * 2 + half;
      const int key_a = n, key_b = 32 + n;
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kbuf + (key_a * CH + (c ^ (key_a & (CH - 1)))) * 16);
      const bf16x8 kb = *reinterpret_cast<const bf16x8*>(kbuf + (key_b * CH + (c ^ (key_b & (CH - 1)))) * 16);
      s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s0, 0, 0, 0);
      s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb, qf[ks], s1, 0, 0, 0);
    }
    lds_barrier();  // K buffer free
    if (has_next) issue_k<D, NW>(kbuf, kp, sn, N, jn * block + stn * kKeyTile, wave, lane);

    // ---- online softmax (base-2 domain) ----
    float x[32];
    float mx = -INFINITY;
    const bool tail = key0 + kKeyTile > N;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = s0[r] * scale_log2;
      x[16 + r] = s1[r] * scale_log2;
    }
    if (tail) {
#pragma unroll
      for (int r = 0; r < 32; ++r) {
        const int key = key0 + (r >> 4) * 32 + ((r & 15) >> 2) * 8 + half * 4 + (r & 3);
        if (key >= N) x[r] = -INFINITY;
      }
    }
#pragma unroll
    for (int r = 0; r < 32; ++r) mx = fmaxf(mx, x[r]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mn = fmaxf(sm.m, mx);
    const float alpha = __builtin_amdgcn_exp2f(sm.m - mn);
    sm.m = mn;
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    bf16x8 pf[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const bf16_t pb = (bf16_t)__builtin_amdgcn_exp2f(x[ks * 8 + e] - mn);
        pf[ks][e] = pb;
        sm.l += (float)pb;
      }
    }

    // ---- O^T += V^T P^T ----
    if (has_next) wait_vmem<LD>(); else wait_vmem<0>();  // V(t) landed
    lds_barrier();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int c = ks * 2 + half;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const int d = dt * 32 + n;
        const bf16x8 va = *reinterpret_cast<const bf16x8*>(vbuf + (d * 8 + (c ^ ((d >> 1) & 7))) * 16);
        o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pf[ks], o[dt], 0, 0, 0);
      }
    }
    lds_barrier();  // V buffer free
    if (!has_next) break;
    issue_v<D, NW>(vbuf, vtp, npad, jn * block + stn * kKeyTile, wave, lane);
    j = jn;
    st = stn;
  }
}

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) void attn_kernel(AttnParams p) {
  __shared__ __align__(16) unsigned char kbuf[Tiles<D, NW>::TILE_BYTES];
  __shared__ __align__(16) unsigned char vbuf[Tiles<D, NW>::TILE_BYTES];
  __shared__ uint32_t bits[MODE == kCapture ? 8192 / 32 : 1];

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);  // = (b*H + h) * M + query block
  const int bh = tile / p.M, qi = tile - bh * p.M;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t base = b * p.st.b + h * p.st.h;
  const bf16_t* kp = p.k + base;
  const bf16_t* vtp = p.vt + (int64_t)bh * D * p.npad;
  const int qrow = qi * p.block + wave * 32 + n;

  bf16x8 qf[D / 16];
  {
    const bf16_t* src = p.q + base + (int64_t)min(qrow, p.N - 1) * p.st.n + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  SoftmaxState sm{-INFINITY, 0.f};

  const int32_t* lst = p.idx + (int64_t)tile * p.M;
  const int nlist = MODE == kDense ? 0 : min(max(((cptr_i32)p.count)[tile], 0), p.M);

  if (MODE == kDense) {
    AllSeq seq{0, p.M};
    attend_phase<D, NW>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad, p.scale_log2, qf,
                        o, sm, wave, lane);
  } else {
    if (MODE == kCapture) {
      for (int w = threadIdx.x; w < (p.M + 31) / 32; w += NW * 64) bits[w] = 0u;
      __syncthreads();
      for (int c = threadIdx.x; c < nlist; c += NW * 64) {
        const int j = min(max(lst[c], 0), p.M - 1);
        atomicOr(&bits[j >> 5], 1u << (j & 31));
      }
      __syncthreads();
    }
    ListSeq seq{lst, nlist, 0, p.M};
    attend_phase<D, NW>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad, p.scale_log2, qf,
                        o, sm, wave, lane);
  }

  float lt = sm.l + __shfl_xor(sm.l, 32);
  float inv = lt > 0.f ? 1.0f / lt : 0.f;

  if (MODE == kCapture) {
    // snapshot of the normalised sparse output, fp32, same lane reads it back below
    float* ws = p.os_ws + ((int64_t)bh * p.npad + qrow) * D;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        f32x4 v;
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][g * 4 + e] * inv;
        *reinterpret_cast<f32x4*>(ws + dt * 32 + g * 8 + half * 4) = v;
      }
    }
    ComplementSeq seq{bits, 0, p.M};
    attend_phase<D, NW>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad, p.scale_log2, qf,
                        o, sm, wave, lane);
    lt = sm.l + __shfl_xor(sm.l, 32);
    inv = lt > 0.f ? 1.0f / lt : 0.f;
    if (qrow < p.N) {
      // no FMA contraction of o * inv into the subtraction below: with every block kept the
      // snapshot and the final state are identical and R must come out exactly zero
#pragma clang fp contract(off)
      bf16_t* dst = p.out + base + (int64_t)qrow * p.st.n;
      bf16_t* rdst = p.res_out + base + (int64_t)qrow * p.st.n;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int d0 = dt * 32 + g * 8 + half * 4;
          const f32x4 os = *reinterpret_cast<const f32x4*>(ws + d0);
          bf16x4 wo, wr;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float od = o[dt][g * 4 + e] * inv;
            wo[e] = (bf16_t)od;
            wr[e] = (bf16_t)(od - os[e]);
          }
          *reinterpret_cast<bf16x4*>(dst + d0) = wo;
          *reinterpret_cast<bf16x4*>(rdst + d0) = wr;
        }
      }
    }
    return;
  }

  if (qrow < p.N) {
    bf16_t* dst = p.out + base + (int64_t)qrow * p.st.n;
    const bool has_res = MODE == kSparse && p.res != nullptr;
    const bf16_t* rsrc = has_res ? p.res + base + (int64_t)qrow * p.st.n : nullptr;
    const float c = p.res_scale.v[h];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + g * 8 + half * 4;
        float v[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] = o[dt][g * 4 + e] * inv;
        if (has_res) {
          const bf16x4 r4 = *reinterpret_cast<const bf16x4*>(rsrc + d0);
#pragma unroll
          for (int e = 0; e < 4; ++e) v[e] += c * (float)r4[e];
        }
        bf16x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = (bf16_t)v[e];
        *reinterpret_cast<bf16x4*>(dst + d0) = w;
      }
    }
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_pack_vt(const bf16_t* v, Strides st, int B, int H, int N, int D, int npad,
                          bf16_t* vt, hipStream_t stream) {
  const int grid = B * H * (npad / 64);
  if (D == 128)
    pack_vt_kernel<128><<<grid, 256, 0, stream>>>(v, st, H, N, npad, vt);
  else
    pack_vt_kernel<64><<<grid, 256, 0, stream>>>(v, st, H, N, npad, vt);
  return hipGetLastError();
}

template <int D, int NW>
static void launch_mode(const AttnParams& p, int grid, AttnMode mode, hipStream_t stream) {
  switch (mode) {
    case kSparse: attn_kernel<D, NW, kSparse><<<grid, NW * 64, 0, stream>>>(p); break;
    case kDense: attn_kernel<D, NW, kDense><<<grid, NW * 64, 0, stream>>>(p); break;
    case kCapture: attn_kernel<D, NW, kCapture><<<grid, NW * 64, 0, stream>>>(p); break;
  }
}

hipError_t launch_attention(const AttnParams& p, int B, int D, AttnMode mode, hipStream_t stream) {
  const int grid = B * p.H * p.M;
  if (D == 128) {
    if (p.block == 64) launch_mode<128, 2>(p, grid, mode, stream);
    else launch_mode<128, 4>(p, grid, mode, stream);
  } else {
    if (p.block == 64) launch_mode<64, 2>(p, grid, mode, stream);
    else launch_mode<64, 4>(p, grid, mode, stream);
  }
  return hipGetLastError();
}

}  // namespace recap
