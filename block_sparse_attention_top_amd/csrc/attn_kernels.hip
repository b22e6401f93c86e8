// Block-sparse and dense attention on gfx950 (bf16 MFMA, fp32 online softmax).
//
// RECAP (paperpeel.com/paper/2610.26244) Sec. 4.1 computes the selected block interactions
// with a block-sparse kernel and dense refreshes with a dense one; Sec. 3.2 adds the cached
// dense refinement to the fresh sparse estimate. This file holds one kernel template for
// five modes:
//   kSparse        walk the compacted kept-block list (two 64-row query blocks per work-group
//                  over the union of their lists); optional fused O += c_h * R epilogue;
//   kDense         walk every key block (128 query rows per work-group);
//   kDenseCapture  as kDense, with a second accumulator over the kept key blocks that shares
//                  the dense running maximum, so one pass writes O_dense and
//                  R = O_dense - O_sparse; a query block whose kept weights underflow against
//                  that maximum is flagged, and its fp32 dense output goes to a workspace;
//   kCaptureR      for flagged query blocks only: recompute the sparse output over the kept
//                  list with its own maximum and write R from the saved dense output;
//   kDenseTail     as kDenseCapture, and also the exact attention over the keys outside the
//                  kept set (the dense sums minus the kept sums), for RECAP's tail
//                  reconstruction (an instantiation of its own, so the capture kernel carries
//                  none of its code).
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
#include "attn_device.h"

// Build-time pipeline choices (defaults are the measured best on MI355X):
//   RECAP_STAGES4   LDS stages of the 4-wavefront (128-row) work-groups: 1 or 2
//   RECAP_PAIR      sparse calls with 64-row blocks run two query blocks per work-group
//   RECAP_PRIO      raise the wavefront priority around MFMA bursts
//   RECAP_WPE       wavefronts per SIMD targeted by register allocation
#ifndef RECAP_STAGES4
#define RECAP_STAGES4 2
#endif
#ifndef RECAP_PAIR
#define RECAP_PAIR 1
#endif
#ifndef RECAP_PRIO
#define RECAP_PRIO 0
#endif
#ifndef RECAP_WPE  // wavefronts per SIMD the register allocation targets
#define RECAP_WPE 2
#endif

namespace recap {

__device__ __forceinline__ void mfma_prio_hi() {
#if RECAP_PRIO
  __builtin_amdgcn_s_setprio(1);
#endif
}
__device__ __forceinline__ void mfma_prio_lo() {
#if RECAP_PRIO
  __builtin_amdgcn_s_setprio(0);
#endif
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

template <int D, int NW>
struct Tiles {
  static constexpr int CH = D / 8;       // 16-byte chunks in a K row
  static constexpr int ROWB = D * 2;     // bytes of a K row in LDS
  static constexpr int LD = CH / NW;     // global->LDS instructions per wave per tensor tile
  static constexpr int KROWS = 64 / CH;  // K rows written by one instruction
  static constexpr int TILE_BYTES = 64 * D * 2;
};

// Per-lane constants of the inner loop, computed once per work-group.
//  K tile in LDS: row `key` (0..63) holds its 16-byte chunks XOR-swizzled, chunk c stored at
//  position c ^ (key & (CH-1)). V^T tile: row d (0..D-1) of 64 keys, chunk c stored at
//  c ^ ((d >> 1) & 7). Both make the 16-byte MFMA-fragment reads bank-conflict free, and
//  both reduce to "lane base XOR (ks << 5)" plus an immediate offset per 32-row tile.
template <int D, int NW>
struct LaneConsts {
  static constexpr int LD = Tiles<D, NW>::LD;
  // K offsets repeat with the instruction index mod 4, V^T offsets mod 2. With enough
  // instructions per wavefront that index is a compile-time constant; otherwise the
  // wavefront's own instructions are folded in at init (never a run-time register index).
  static constexpr int KP = LD >= 4 ? 4 : LD;
  static constexpr int VP = LD >= 2 ? 2 : LD;
  uint32_t k_rd, v_rd;   // LDS read offsets (bytes) within a tile buffer
  uint32_t k_voff[KP];   // K DMA source offsets (bytes)
  uint32_t v_voff[VP];   // V^T DMA source offsets (bytes)
  __device__ void init(int lane, int wave, int64_t sn, int npad) {
    constexpr int CH = Tiles<D, NW>::CH, ROWB = Tiles<D, NW>::ROWB, KROWS = Tiles<D, NW>::KROWS;
    const int n = lane & 31, half = lane >> 5;
    k_rd = opaque(n * ROWB + ((half ^ (n & (CH - 1))) << 4));
    v_rd = opaque(n * 128 + ((half ^ ((n >> 1) & 7)) << 4));
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      const int x = LD >= 4 ? r : wave * LD + r;
      const int key = x * KROWS + lane / CH;  // row inside the tile (swizzle period 4 in x)
      const int c = (lane % CH) ^ (key & (CH - 1));
      k_voff[r] = opaque((uint32_t)((lane / CH) * sn * 2 + c * 16));
    }
#pragma unroll
    for (int r = 0; r < VP; ++r) {
      const int x = LD >= 2 ? r : wave * LD + r;
      const int c = (lane & 7) ^ ((x * 4 + (lane >> 4)) & 7);
      v_voff[r] = opaque((uint32_t)((lane >> 3) * npad * 2 + c * 16));
    }
  }
  __device__ uint32_t kv(int x, int it) const { return k_voff[LD >= 4 ? (x & 3) : it]; }
  __device__ uint32_t vv(int x, int it) const { return v_voff[LD >= 2 ? (x & 1) : it]; }
};

// Issue the global -> LDS loads of one 64-key K tile: rows [key0, key0 + 64) of this head.
// Addresses are a uniform 64-bit base (first row of the tile) plus a 32-bit lane offset, so
// the per-load cost is one 32-bit add.
template <int D, int NW>
__device__ __forceinline__ void issue_k(uint32_t kbuf, const bf16_t* kp, int64_t sn, int N,
                                        int key0, int wave, int lane,
                                        const LaneConsts<D, NW>& lc) {
  constexpr int CH = Tiles<D, NW>::CH, LD = Tiles<D, NW>::LD, KROWS = Tiles<D, NW>::KROWS;
  const char* tile_base = (const char*)(kp + (int64_t)key0 * sn);
  const uint32_t row_bytes = (uint32_t)(sn * 2);
  if (key0 + 64 <= N) {
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int x = wave * LD + it;
      load_lds16(tile_base, (uint32_t)(x * KROWS * row_bytes + lc.kv(x, it)), kbuf + x * 1024);
    }
  } else {
    // last, partial block: rows past N are clamped to row N-1 (their scores are masked). The
    // lane index is re-read opaquely so this rare path's address math is not hoisted out of
    // the tile loop (where it would hold registers for the whole loop).
    asm volatile("" ::: "memory");
    const int last = N - 1 - key0;
    const int ln = (int)opaque((uint32_t)lane);
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int slot0 = (wave * LD + it) * 64;
      const int slot = slot0 + ln;
      const int key = slot / CH;
      const int c = (slot % CH) ^ (key & (CH - 1));
      load_lds16(tile_base, (uint32_t)(min(key, last) * row_bytes + c * 16), kbuf + slot0 * 16);
    }
  }
}

template <int D, int NW>
__device__ __forceinline__ void issue_v(uint32_t vbuf, const bf16_t* vtp, int npad,
                                        int key0, int wave, const LaneConsts<D, NW>& lc) {
  constexpr int LD = Tiles<D, NW>::LD;
  const char* tile_base = (const char*)(vtp + key0);
  const uint32_t row_bytes = (uint32_t)npad * 2;
#pragma unroll
  for (int it = 0; it < LD; ++it) {
    const int x = wave * LD + it;
    load_lds16(tile_base, (uint32_t)(x * 8 * row_bytes + lc.vv(x, it)), vbuf + x * 1024);
  }
}

// Residual-capture side state: a second accumulator that sees only the kept key blocks of this
// wavefront's query block (bitmap in LDS). It shares the running max and the probabilities of
// the dense accumulator, so it costs only the extra PV products of kept tiles.
template <int D>
struct KeptAcc {
  f32x16 o[D / 32];
  float l;
  const uint32_t* bits;
};

// ---- per-tile math, shared by the pipeline drivers below ----

// S^T = K Q^T for one 64-key tile in LDS (raw dot products); ACC adds to s0, s1 instead.
// LDS buffers are 256-byte aligned, so base + (lane offset XOR (ks << 5)) equals
// (base + lane offset) XOR (ks << 5): one opaque base per tile, one XOR per fragment.
template <int D, int NW, bool ACC = false>
__device__ __forceinline__ void tile_qk(uint32_t kb, const bf16x8 (&qf)[D / 16],
                                        const LaneConsts<D, NW>& lc, f32x16& s0, f32x16& s1) {
  constexpr int ROWB = Tiles<D, NW>::ROWB;
  if (!ACC) {
    s0 = f32x16{};
    s1 = f32x16{};
  }
  const uint32_t base = opaque(kb + lc.k_rd);
  mfma_prio_hi();
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint32_t a = base ^ (uint32_t)(ks << 5);
    const bf16x8 ka = lds_read16(a);
    const bf16x8 kb2 = lds_read16(a + 32 * ROWB);
    s0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], s0, 0, 0, 0);
    s1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb2, qf[ks], s1, 0, 0, 0);
  }
  mfma_prio_lo();
}

// Keys past N in the last, partial tile get score -inf (a rare, uniform branch).
__device__ __forceinline__ void mask_tail(f32x16& s0, f32x16& s1, int key0, int N, int half) {
  if (key0 + kKeyTile > N) {
    asm volatile("" ::: "memory");  // keep the rare tail tile a real (uniform) branch
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = ((r >> 2) << 3) + half * 4 + (r & 3);
      if (key0 + kr >= N) s0[r] = -INFINITY;
      if (key0 + 32 + kr >= N) s1[r] = -INFINITY;
    }
  }
}

// Row maximum of one tile's scores in log2 units.
__device__ __forceinline__ float tile_rowmax(const f32x16& s0, const f32x16& s1, float scale_log2) {
  float mx = fmaxf(s0[0], s1[0]);  // compiler-generated first read of both products
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = max3(mx, s0[r], s1[r]);
  return cross_half_max(mx) * scale_log2;
}

// Lazy rescale: raise the running max to the tile max mt only when some lane's max grows by
// more than kLazy, rescaling the accumulators (and the kept-block ones under capture).
template <int D, bool CAP>
__device__ __forceinline__ void raise_max(float mt, SoftmaxState& sm, f32x16 (&o)[D / 32],
                                          KeptAcc<D>& ka) {
  if (__builtin_amdgcn_ballot_w64(mt > sm.m + kLazy) != 0) {
    const float mn = fmaxf(sm.m, mt);
    const float alpha = __builtin_amdgcn_exp2f(sm.m - mn);
    sm.m = mn;
    sm.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    if (CAP) {
      ka.l *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) ka.o[dt] *= alpha;
    }
  }
}

// Weights of one tile, p = exp2(s * scale - m) rounded to bf16 (the P^T operands of the PV
// product), and the per-lane sum of exactly those rounded weights.
__device__ __forceinline__ float tile_exp(const f32x16& s0, const f32x16& s1, float scale_log2,
                                          float m, bf16x8 (&pf)[4]) {
  const float neg_m = -m;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = (ks < 2) ? s0[(ks & 1) * 8 + e] : s1[(ks & 1) * 8 + e];
      pf[ks][e] = (bf16_t)__builtin_amdgcn_exp2f(__builtin_fmaf(x, scale_log2, neg_m));
    }
  }
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const bf16x2 one = {(bf16_t)1.0f, (bf16_t)1.0f};
  float acc = 0.f;
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      const bf16x2 pr = {pf[ks][e], pf[ks][e + 1]};
      acc = __builtin_amdgcn_fdot2_f32_bf16(pr, one, acc, false);
    }
  }
  return acc;
}

// Online softmax of one tile in the base-2 domain with lazy rescale; returns the bf16 P^T
// operands and whether the tile also feeds the kept-block accumulator.
template <int D, bool CAP>
__device__ __forceinline__ bool tile_softmax(f32x16& s0, f32x16& s1, int j, int key0, int N,
                                             float scale_log2, int half, f32x16 (&o)[D / 32],
                                             SoftmaxState& sm, KeptAcc<D>& ka, bf16x8 (&pf)[4]) {
  mask_tail(s0, s1, key0, N, half);  // finite max: a tile has a valid key
  raise_max<D, CAP>(tile_rowmax(s0, s1, scale_log2), sm, o, ka);
  const float acc = tile_exp(s0, s1, scale_log2, sm.m, pf);
  sm.l += acc;
  const bool kept = CAP && ((ka.bits[j >> 5] >> (j & 31)) & 1u);  // uniform per wavefront
  if (kept) ka.l += acc;
  return kept;
}

// O^T += V^T P^T for one tile (and the kept-block accumulator when `kept`). The kept-block
// products form their own sequence behind one wavefront-uniform branch per tile (re-reading
// their V^T operands from LDS), so that no branch splits the main product sequence and its
// operand reads can be issued ahead of the products, as in the dense pass.
template <int D, int NW>
__device__ __forceinline__ void tile_pv(uint32_t vb, const bf16x8 (&pf)[4],
                                        const LaneConsts<D, NW>& lc, f32x16 (&o)[D / 32],
                                        KeptAcc<D>& ka, bool kept) {
  const uint32_t base = opaque(vb + lc.v_rd);
  mfma_prio_hi();
#pragma unroll
  for (int ks = 0; ks < 4; ++ks) {
    const uint32_t a = base ^ (uint32_t)(ks << 5);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(a + dt * 4096), pf[ks], o[dt],
                                                      0, 0, 0);
  }
  if (kept) {
    const uint32_t kbase = opaque(vb + lc.v_rd);  // fresh reads, not values held from above
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const uint32_t a = kbase ^ (uint32_t)(ks << 5);
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        ka.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(lds_read16(a + dt * 4096), pf[ks],
                                                           ka.o[dt], 0, 0, 0);
    }
  }
  mfma_prio_lo();
}

// One attention phase over a block sequence, continuing the online-softmax state (m, l, o).
// STAGES = 1: one K and one V^T buffer; K(t+1) loads during softmax + PV of tile t and
//             V^T(t+1) during the QK^T of tile t+1 (four barriers per tile).
// STAGES = 2: two buffers each; tile t+2 loads into the buffers tile t has just released, so
//             every tile has a full tile of compute to land (two barriers per tile).
// SKIP: the work-group streams the union of two query blocks' kept sets; each wavefront
//       computes only the tiles of its own block's kept set (bitmap `own`).
template <int D, int NW, int STAGES, bool CAP, bool SKIP = false, class Seq>
__device__ __forceinline__ void attend_phase(Seq& seq, unsigned char* kbuf, unsigned char* vbuf,
                                             const bf16_t* kp, const bf16_t* vtp, int64_t sn,
                                             int N, int block, int npad, float scale_log2,
                                             const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                             SoftmaxState& sm, int wave, int lane,
                                             const LaneConsts<D, NW>& lc, KeptAcc<D>& ka,
                                             const uint32_t* own = nullptr) {
  constexpr int LD = Tiles<D, NW>::LD, TB = Tiles<D, NW>::TILE_BYTES;
  const int half = lane >> 5;
  TileCur cur{seq.first(), 0};
  if (cur.j < 0) return;
  const uint32_t kb0 = lds_base(kbuf), vb0 = lds_base(vbuf);
  auto issue_both = [&](TileCur t, int buf) {
    const int key0 = t.j * block + t.st * kKeyTile;
    issue_k<D, NW>(kb0 + buf * TB, kp, sn, N, key0, wave, lane, lc);
    issue_v<D, NW>(vb0 + buf * TB, vtp, npad, key0, wave, lc);
  };
  auto active_for = [&](int j) { return !SKIP || ((own[j >> 5] >> (j & 31)) & 1u); };

  if constexpr (STAGES == 2) {
    TileCur nxt = advance(cur, seq, block, N);
    issue_both(cur, 0);
    if (nxt.j >= 0) issue_both(nxt, 1);
    int b = 0;
    while (true) {
      const bool has1 = nxt.j >= 0;
      const TileCur nxt2 = advance(nxt, seq, block, N);
      // in flight, oldest first: K(t), V(t) [, K(t+1), V(t+1)]
      if (has1) wait_vmem<2 * LD>(); else wait_vmem<0>();
      lds_barrier();
      const int key0 = cur.j * block + cur.st * kKeyTile;
      if (active_for(cur.j)) {
        f32x16 s0, s1;
        tile_qk<D, NW>(kb0 + b * TB, qf, lc, s0, s1);
        bf16x8 pf[4];
        const bool kept = tile_softmax<D, CAP>(s0, s1, cur.j, key0, N, scale_log2, half, o, sm, ka, pf);
        tile_pv<D, NW>(vb0 + b * TB, pf, lc, o, ka, kept);
      }
      lds_barrier();  // every wave is done with buffers b
      if (!has1) break;
      if (nxt2.j >= 0) issue_both(nxt2, b);
      cur = nxt;
      nxt = nxt2;
      b ^= 1;
    }
  } else {
    issue_both(cur, 0);
    while (true) {
      const TileCur nxt = advance(cur, seq, block, N);
      const bool has_next = nxt.j >= 0;
      const int key0 = cur.j * block + cur.st * kKeyTile;
      const bool active = active_for(cur.j);
      wait_vmem<LD>();  // this wave's K(t) landed (V^T(t), issued after it, may be in flight)
      lds_barrier();    // ... and every other wave's
      f32x16 s0, s1;
      if (active) tile_qk<D, NW>(kb0, qf, lc, s0, s1);
      lds_barrier();  // every wave is done reading the K buffer
      if (has_next)
        issue_k<D, NW>(kb0, kp, sn, N, nxt.j * block + nxt.st * kKeyTile, wave, lane, lc);
      bf16x8 pf[4];
      bool kept = false;
      if (active) kept = tile_softmax<D, CAP>(s0, s1, cur.j, key0, N, scale_log2, half, o, sm, ka, pf);
      if (has_next) wait_vmem<LD>(); else wait_vmem<0>();  // V^T(t) landed (K(t+1) may not)
      lds_barrier();
      if (active) tile_pv<D, NW>(vb0, pf, lc, o, ka, kept);
      lds_barrier();  // every wave is done reading the V buffer
      if (!has_next) break;
      issue_v<D, NW>(vb0, vtp, npad, nxt.j * block + nxt.st * kKeyTile, wave, lc);
      cur = nxt;
    }
  }
}

template <int D, int NW, int MODE>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(RECAP_WPE, RECAP_WPE))) void attn_kernel(AttnParams p) {
  constexpr int STAGES = NW == 4 ? RECAP_STAGES4 : 1;
  __shared__ __align__(256) unsigned char kbuf[STAGES * Tiles<D, NW>::TILE_BYTES];
  __shared__ __align__(256) unsigned char vbuf[STAGES * Tiles<D, NW>::TILE_BYTES];
  constexpr int QROWS = NW * 32;  // query rows of one work-group

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // uniform per wavefront
  const int n = lane & 31, half = lane >> 5;
  // tile = (b*H + h) * mq + query tile; in the list modes a query tile is one query block
  // runs of 64 tiles per XCD (all XCDs on one head) rather than one range per XCD: 3% faster
  // dense capture and sparse calls at 720p
  const int tile = xcd_runs<64>(blockIdx.x, gridDim.x);
  const int bh = tile / p.mq, qi = tile - bh * p.mq;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t base = b * p.st.b + h * p.st.h;
  const bf16_t* kp = p.k + base;
  const bf16_t* vtp = p.vt + (int64_t)bh * D * p.npad;
  const int qrow = qi * QROWS + wave * 32 + n;
  LaneConsts<D, NW> lc;
  lc.init(lane, wave, p.st.n, p.npad);

  bf16x8 qf[D / 16];
  {
    const bf16_t* src = p.q + base + (int64_t)min(qrow, p.N - 1) * p.st.n + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
    // consume the fragments here, so the compiler's waits for these loads sit before the loop
    // (the tile loads in the loop are invisible to its wait-count bookkeeping)
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  SoftmaxState sm{-INFINITY, 0.f};

  constexpr bool TAIL = MODE == kDenseTail;
  constexpr bool CAP = MODE == kDenseCapture || TAIL;
  // sparse with 4 wavefronts and 64-row blocks: a pair of query blocks per work-group
  constexpr bool PAIRABLE = MODE == kSparse && NW == 4;
  constexpr bool BITS = CAP || PAIRABLE;
  constexpr int BLKS = BITS ? (QROWS / 64) : 1;  // query blocks of this work-group (block 64: 2)
  __shared__ uint32_t kept_bits[BITS ? BLKS : 1][BITS ? kMaxBlocks / 32 : 1];
  __shared__ int blk_flag[BLKS];
  KeptAcc<D> ka;
  int qb = 0;  // this wavefront's query block (capture mode)
  const bool pair = PAIRABLE && p.block == 64;
  if (CAP || pair) {
    // kept-block bitmaps of the query blocks covered by this work-group
    const int nb = QROWS / p.block;  // 2 for block 64, 1 for block 128
    qb = (qi * QROWS + wave * 32) / p.block;
    for (int w = threadIdx.x; w < nb * ((p.M + 31) / 32); w += NW * 64)
      kept_bits[w / ((p.M + 31) / 32)][w % ((p.M + 31) / 32)] = 0u;
    if (threadIdx.x < BLKS) blk_flag[threadIdx.x] = 0;
    __syncthreads();
    for (int lb = 0; lb < nb; ++lb) {
      const int blk = (qi * QROWS) / p.block + lb;
      if (blk >= p.M) break;
      const int64_t row = (int64_t)bh * p.M + blk;
      const int cnt = min(max(p.count[row], 0), p.M);
      for (int c = threadIdx.x; c < cnt; c += NW * 64) {
        const int jj = min(max(p.idx[row * p.M + c], 0), p.M - 1);
        atomicOr(&kept_bits[lb][jj >> 5], 1u << (jj & 31));
      }
    }
    __syncthreads();
    ka.bits = kept_bits[(wave * 32) / p.block];
    ka.l = 0.f;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) ka.o[dt] = f32x16{};
  }

  int nlist = 0;
  if (PAIRABLE && pair) {
    UnionSeq seq{kept_bits[0], kept_bits[1], p.M, 0};
    attend_phase<D, NW, STAGES, false, true>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad,
                                     p.scale_log2, qf, o, sm, wave, lane, lc, ka,
                                     kept_bits[(wave * 32) / p.block]);
  } else if (MODE == kDense || CAP) {
    // staggered start at the diagonal: neighbouring work-groups stream the same K/V tiles at
    // nearly the same time, which keeps them in L2
    AllSeq seq{0, p.M, min((qi * QROWS) / p.block, p.M - 1)};
    attend_phase<D, NW, STAGES, CAP>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad,
                             p.scale_log2, qf, o, sm, wave, lane, lc, ka);
  } else {
    const int32_t* lst = p.idx + (int64_t)tile * p.M;  // one query block per work-group here
    nlist = min(max(((cptr_i32)p.count)[tile], 0), p.M);
    if (MODE == kCaptureR && ((cptr_u8)p.flags)[tile] == 0) return;  // done in the dense pass
    ListSeq seq{lst, nlist, 0, p.M};
    attend_phase<D, NW, STAGES, false>(seq, kbuf, vbuf, kp, vtp, p.st.n, p.N, p.block, p.npad,
                               p.scale_log2, qf, o, sm, wave, lane, lc, ka);
  }

  const float lt = cross_half_sum(sm.l);
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;

  if (CAP) {
    // The kept accumulator shares the dense running max; if its weights sum to less than
    // 2^-64 against that maximum (too few significant bits left after bf16 rounding of the
    // weights), the block is left to the residual pass, which recomputes the sparse output
    // with its own maximum.
    const float ls = cross_half_sum(ka.l);
    const bool want_r = p.res_out != nullptr;  // the same for the whole grid
    bool flagged = false;
    if (want_r) {
      const bool bad = qrow < p.N && !(ls >= 0x1p-64f);
      if (__builtin_amdgcn_ballot_w64(bad) != 0 && lane == 0)
        atomicOr(&blk_flag[(wave * 32) / p.block], 1);
      __syncthreads();
      flagged = blk_flag[(wave * 32) / p.block] != 0;
      if (qb < p.M && lane == 0 && (wave * 32) % p.block == 0)
        p.flags[(int64_t)bh * p.M + qb] = flagged ? 1 : 0;
    }
    if (qrow >= p.N) return;
    if (half == 0) {
      const int64_t srow = (int64_t)bh * p.N + qrow;
      if (p.lse_out != nullptr) p.lse_out[srow] = (sm.m + log2f(lt)) * kLn2;
      if (p.kmass_out != nullptr) p.kmass_out[srow] = ls / lt;
    }
    if (TAIL) {
      // the keys outside the kept set: the dense sums minus the kept ones (same running max)
      const float ltail = cross_half_sum(sm.l - ka.l);
      if (half == 0)
        p.tail_lse[(int64_t)bh * p.N + qrow] =
            ltail > 0.f ? (sm.m + log2f(ltail)) * kLn2 : -INFINITY;
      const float invt = ltail > 0.f ? 1.0f / ltail : 0.f;
      float* to = p.tail_o + ((int64_t)bh * p.N + qrow) * D;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          f32x4 x;
#pragma unroll
          for (int e = 0; e < 4; ++e) x[e] = (o[dt][g * 4 + e] - ka.o[dt][g * 4 + e]) * invt;
          *reinterpret_cast<f32x4*>(to + dt * 32 + g * 8 + half * 4) = x;
        }
      }
    }
    const int64_t orow = base + (int64_t)qrow * p.st.n;
    const float invs = ls > 0.f ? 1.0f / ls : 0.f;
    const int64_t odrow = ((int64_t)bh * p.npad + qrow) * D;  // od_ws is NULL without residual
    {
#pragma clang fp contract(off)
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + g * 8 + half * 4;
        f32x4 vd;
        bf16x4 wo, wr;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          vd[e] = o[dt][g * 4 + e] * inv;
          const float vs = ka.o[dt][g * 4 + e] * invs;
          wo[e] = (bf16_t)vd[e];
          wr[e] = (bf16_t)(vd[e] - vs);
        }
        *reinterpret_cast<bf16x4*>(p.out + orow + d0) = wo;
        if (flagged) *reinterpret_cast<f32x4*>(p.od_ws + odrow + d0) = vd;
        else if (want_r) *reinterpret_cast<bf16x4*>(p.res_out + orow + d0) = wr;
      }
    }
    }
    return;
  }

  if (qrow >= p.N) return;
  const int64_t orow = base + (int64_t)qrow * p.st.n;
  if (MODE != kCaptureR && p.lse_out != nullptr && half == 0)
    p.lse_out[(int64_t)bh * p.N + qrow] = lt > 0.f ? (sm.m + log2f(lt)) * kLn2 : -INFINITY;

  if (MODE == kCaptureR) {
    // R = O_dense - O_sparse from the fp32 dense output of the same inputs; exactly zero when
    // the kept list covers every key block (then both are the same attention)
#pragma clang fp contract(off)
    const float* od = p.od_ws + ((int64_t)bh * p.npad + qrow) * D;
    const bool all_kept = nlist == p.M;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d0 = dt * 32 + g * 8 + half * 4;
        const f32x4 dv = *reinterpret_cast<const f32x4*>(od + d0);
        bf16x4 wr;
#pragma unroll
        for (int e = 0; e < 4; ++e) wr[e] = all_kept ? (bf16_t)0.0f : (bf16_t)(dv[e] - o[dt][g * 4 + e] * inv);
        *reinterpret_cast<bf16x4*>(p.res_out + orow + d0) = wr;
      }
    }
    return;
  }

  bf16_t* dst = p.out + orow;
  const bool has_res = MODE == kSparse && p.res != nullptr;
  const bf16_t* rsrc = has_res ? p.res + orow : nullptr;
  const float c = p.res_scale.v[h];
  float* dst32 = (MODE == kSparse && p.o32_out != nullptr)
                     ? p.o32_out + ((int64_t)bh * p.N + qrow) * D : nullptr;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + g * 8 + half * 4;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][g * 4 + e] * inv;
      if (dst32 != nullptr) {  // fp32 output for a later merge (no epilogue on this path)
        *reinterpret_cast<f32x4*>(dst32 + d0) = v;
        continue;
      }
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

// ------------------------------------------------------------------------------------------
// Coarse tail of RECAP's attention-level reconstruction (paperpeel.com RECAP Sec. 3.2: for the
// omitted interactions, block means give initial estimates of the normalisation mass and the
// value). For query token t of query block i, over the pooled key blocks j outside i's kept
// set: weights n_j * exp(s * q_t . K̄_j), values V̄_j. The coarse log-mass is ln of the summed
// weights, the coarse output the weighted mean of the V̄_j. Zeroth order: the key-variance and
// value-key-covariance refinements the page names are not applied.
// Same tile math as attn_kernel (4 wavefronts, 128 query rows, 64 pooled keys per tile, one
// LDS stage: a row has only ceil(M / 64) tiles), with the pooled scores from the hi + lo key
// pair. Kept blocks and pooled keys past M get score -inf; the last pooled key's weight
// carries its shorter block.
// ------------------------------------------------------------------------------------------
// Pooled keys as a pair of bf16 values, hi = bf16(K̄) and lo = bf16(K̄ - hi) (about 16
// significant bits, so the pooled scores are as accurate as the token scores, whose bf16
// operands are exact), pooled values as bf16. Element e of [B*H][mpad][D]; rows >= M are zero.
template <int D>
__global__ __launch_bounds__(256) void tail_keys_kernel(const float* __restrict__ kbar,
                                                        const float* __restrict__ vbar, int M,
                                                        int mpad, int64_t total,
                                                        bf16_t* __restrict__ kb_hi,
                                                        bf16_t* __restrict__ kb_lo,
                                                        bf16_t* __restrict__ vb16) {
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t bh = e / ((int64_t)mpad * D);
    const int64_t r = e - bh * mpad * D;
    const int j = (int)(r / D), d = (int)(r - (int64_t)j * D);
    const int64_t src = (bh * M + j) * D + d;
    const float kx = j < M ? kbar[src] : 0.f;
    const bf16_t hi = (bf16_t)kx;
    kb_hi[e] = hi;
    kb_lo[e] = (bf16_t)(kx - (float)hi);
    vb16[e] = (bf16_t)(j < M ? vbar[src] : 0.f);
  }
}

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void tail_kernel(TailParams p) {
  constexpr int NW = 4, QROWS = 128, TB = Tiles<D, NW>::TILE_BYTES;
  // K̄ hi and lo: one stage, the next tile's loads issued as soon as this tile's QK^T products
  // have read it; V̄^T: two stages, the next tile's loads issued at the top of each step.
  // 64 KB at D = 128, so two work-groups share a CU.
  __shared__ __align__(256) unsigned char kbuf[TB];
  __shared__ __align__(256) unsigned char klbuf[TB];
  __shared__ __align__(256) unsigned char vbuf[2 * TB];
  __shared__ uint32_t kept_bits[2][kMaxBlocks / 32];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / p.mq, qi = tile - bh * p.mq;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t base = b * p.st.b + h * p.st.h;
  const int qrow = qi * QROWS + wave * 32 + n;
  LaneConsts<D, NW> lc;
  lc.init(lane, wave, (int64_t)D, p.mpad);
  bf16x8 qf[D / 16];
  {
    const bf16_t* src = p.q + base + (int64_t)min(qrow, p.N - 1) * p.st.n + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  }
  // kept-block bitmaps of the query blocks of this work-group
  const int nb = QROWS / p.block;  // 2 for block 64, 1 for block 128
  for (int w = threadIdx.x; w < nb * kMaxBlocks / 32; w += NW * 64)
    kept_bits[w / (kMaxBlocks / 32)][w % (kMaxBlocks / 32)] = 0u;
  __syncthreads();
  for (int lb = 0; lb < nb; ++lb) {
    const int blk = (qi * QROWS) / p.block + lb;
    if (blk >= p.M) break;
    const int64_t row = (int64_t)bh * p.M + blk;
    const int cnt = min(max(p.count[row], 0), p.M);
    for (int c = threadIdx.x; c < cnt; c += NW * 64) {
      const int jj = min(max(p.idx[row * p.M + c], 0), p.M - 1);
      atomicOr(&kept_bits[lb][jj >> 5], 1u << (jj & 31));
    }
  }
  __syncthreads();
  const uint32_t* own = kept_bits[(wave * 32) / p.block];

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  SoftmaxState sm{-INFINITY, 0.f};
  KeptAcc<D> none;
  const uint32_t kb0 = lds_base(kbuf), kl0 = lds_base(klbuf), vb0 = lds_base(vbuf);
  const bf16_t* kp = p.kb + (int64_t)bh * p.mpad * D;
  const bf16_t* klp = p.kb_lo + (int64_t)bh * p.mpad * D;
  const bf16_t* vtp = p.vt + (int64_t)bh * D * p.mpad;
  const int ntile = (p.M + kKeyTile - 1) / kKeyTile;
  issue_v<D, NW>(vb0, vtp, p.mpad, 0, wave, lc);
  issue_k<D, NW>(kb0, kp, (int64_t)D, p.M, 0, wave, lane, lc);
  issue_k<D, NW>(kl0, klp, (int64_t)D, p.M, 0, wave, lane, lc);
  for (int t = 0; t < ntile; ++t) {
    const int key0 = t * kKeyTile;
    const uint32_t vt = vb0 + (t & 1) * TB;
    // this wavefront's loads of tile t (V̄ issued one step ago, K̄ in the previous step's
    // middle) have landed; the barrier makes them everyone's and frees the other V̄ stage
    wait_vmem<0>();
    lds_barrier();
    if (t + 1 < ntile) issue_v<D, NW>(vb0 + ((t + 1) & 1) * TB, vtp, p.mpad, key0 + kKeyTile, wave, lc);
    f32x16 s0, s1;
    tile_qk<D, NW>(kb0, qf, lc, s0, s1);
    tile_qk<D, NW, true>(kl0, qf, lc, s0, s1);  // + q . (K̄ - hi)
    lds_barrier();  // every wavefront has read K̄ of tile t
    if (t + 1 < ntile) {
      issue_k<D, NW>(kb0, kp, (int64_t)D, p.M, key0 + kKeyTile, wave, lane, lc);
      issue_k<D, NW>(kl0, klp, (int64_t)D, p.M, key0 + kKeyTile, wave, lane, lc);
    }
    // scores in log2 units; kept blocks and pooled keys past M get -inf, the last pooled key
    // the log2 of its share of a full block. Keys key0 + kr and key0 + 32 + kr are bit kr of
    // words key0 / 32 and key0 / 32 + 1 of the kept bitmap (key0 is a multiple of 64; a word
    // past the bitmap's end only holds keys >= M, masked anyway).
    const uint32_t w0 = own[key0 >> 5], w1 = own[(key0 >> 5) + 1];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int kr = ((r >> 2) << 3) + half * 4 + (r & 3);
      const int j0 = key0 + kr, j1 = key0 + 32 + kr;
      const bool m0 = j0 >= p.M || ((w0 >> kr) & 1u);
      const bool m1 = j1 >= p.M || ((w1 >> kr) & 1u);
      const float x0 = s0[r] * p.scale_log2, x1 = s1[r] * p.scale_log2;
      s0[r] = m0 ? -INFINITY : (j0 == p.M - 1 ? x0 + p.last_bias : x0);
      s1[r] = m1 ? -INFINITY : (j1 == p.M - 1 ? x1 + p.last_bias : x1);
    }
    // the mask depends only on the key and the wavefront's query block: a tile is either
    // fully masked for all lanes of a wavefront (no raise) or has a finite maximum for all
    raise_max<D, false>(tile_rowmax(s0, s1, 1.0f), sm, o, none);
    // while every key so far is masked, m = -inf: use +inf so the weights are 0, not NaN
    bf16x8 pf[4];
    sm.l += tile_exp(s0, s1, 1.0f, sm.m == -INFINITY ? INFINITY : sm.m, pf);
    tile_pv<D, NW>(vt, pf, lc, o, none, false);
  }
  const float lt = cross_half_sum(sm.l);
  if (qrow >= p.N) return;
  const int64_t srow = (int64_t)bh * p.N + qrow;
  if (half == 0) p.tail_lse[srow] = lt > 0.f ? (sm.m + log2f(lt)) * kLn2 + p.ln_block : -INFINITY;
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  float* to = p.tail_o + srow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = o[dt][g * 4 + e] * inv;
      *reinterpret_cast<f32x4*>(to + dt * 32 + g * 8 + half * 4) = x;
    }
  }
}

// Discrepancy and merge of RECAP's reconstruction (paperpeel.com RECAP Sec. 3.2: a tail
// quantity y_t = coarse + discrepancy; the discrepancy d_h taken exactly at a dense refresh is
// cached, and later sparse steps use coarse + d_h). One thread per (token, 4 head dims); the
// fp32 arrays are [B*H][N] and [B*H][N][D] contiguous, `out` is bf16 in the q layout.
// mode 0: d_lse = exact_lse - coarse_lse (0 when both are -inf: no keys outside the kept set),
//         d_o = exact_o - coarse_o (fp32: d_o is a difference of tail outputs, as large as the
//         values, and a bf16 copy would add its rounding to every later merge);
// mode 1: lT = coarse_lse + d_lse, oT = coarse_o + d_o (d optional), and with the sparse
//         output O_s of log-mass lse_s: out = w O_s + (1 - w) oT, w = 1 / (1 + exp(lT - lse_s))
//         (w = 1 when lT = -inf).
template <int D>
__global__ __launch_bounds__(256) void tail_combine_kernel(int mode, int H, int N, Strides st,
                                                           int64_t total,
                                                           const float* __restrict__ a_lse,
                                                           const float* __restrict__ a_o,
                                                           const float* __restrict__ c_lse,
                                                           const float* __restrict__ c_o,
                                                           const float* __restrict__ d_lse,
                                                           const float* __restrict__ d_o,
                                                           float* __restrict__ d_lse_out,
                                                           float* __restrict__ d_o_out,
                                                           bf16_t* __restrict__ out) {
  constexpr int G = D / 4;
  for (int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x; e < total;
       e += (int64_t)gridDim.x * 256) {
    const int64_t row = e / G;  // (b*H + h)*N + t
    const int d0 = (int)(e - row * G) * 4;
    const f32x4 co = *reinterpret_cast<const f32x4*>(c_o + row * D + d0);
    const f32x4 ao = *reinterpret_cast<const f32x4*>(a_o + row * D + d0);
    const float cl = c_lse[row];
    const float al = a_lse[row];
    if (mode == 0) {
      if (d0 == 0) d_lse_out[row] = (al == -INFINITY && cl == -INFINITY) ? 0.f : al - cl;
      *reinterpret_cast<f32x4*>(d_o_out + row * D + d0) = ao - co;
    } else {
      const bool has_d = d_lse != nullptr;
      const float lT = cl + (has_d ? d_lse[row] : 0.f);
      const float w = lT == -INFINITY ? 1.f : 1.0f / (1.0f + __expf(lT - al));
      const f32x4 dd = has_d ? *reinterpret_cast<const f32x4*>(d_o + row * D + d0) : f32x4{};
      const int64_t bh = row / N;
      const int t = (int)(row - bh * N);
      const int64_t b = bh / H, h = bh - b * H;
      bf16x4 w4;
#pragma unroll
      for (int i = 0; i < 4; ++i) w4[i] = (bf16_t)(w * ao[i] + (1.f - w) * (co[i] + dd[i]));
      *reinterpret_cast<bf16x4*>(out + b * st.b + h * st.h + (int64_t)t * st.n + d0) = w4;
    }
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_tail_keys(const float* kbar, const float* vbar, int BH, int M, int D, int mpad,
                            bf16_t* kb_hi, bf16_t* kb_lo, bf16_t* vb16, hipStream_t stream) {
  const int64_t total = (int64_t)BH * mpad * D;
  const int grid = (int)(total < 65536LL * 256 ? (total + 255) / 256 : 65536);
  if (D == 128)
    tail_keys_kernel<128><<<grid, 256, 0, stream>>>(kbar, vbar, M, mpad, total, kb_hi, kb_lo,
                                                    vb16);
  else
    tail_keys_kernel<64><<<grid, 256, 0, stream>>>(kbar, vbar, M, mpad, total, kb_hi, kb_lo,
                                                   vb16);
  return hipGetLastError();
}

hipError_t launch_tail(TailParams p, int B, int D, hipStream_t stream) {
  p.mq = (p.N + 127) / 128;
  const int grid = B * p.H * p.mq;
  if (D == 128)
    tail_kernel<128><<<grid, 256, 0, stream>>>(p);
  else
    tail_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

hipError_t launch_tail_combine(int mode, int B, int H, int N, int D, Strides st,
                               const float* a_lse, const float* a_o, const float* c_lse,
                               const float* c_o, const float* d_lse, const float* d_o,
                               float* d_lse_out, float* d_o_out, bf16_t* out,
                               hipStream_t stream) {
  const int64_t total = (int64_t)B * H * N * (D / 4);
  const int grid = (int)(total < 65536LL * 256 ? (total + 255) / 256 : 65536);
  if (D == 128)
    tail_combine_kernel<128><<<grid, 256, 0, stream>>>(mode, H, N, st, total, a_lse, a_o, c_lse,
                                                       c_o, d_lse, d_o, d_lse_out, d_o_out, out);
  else
    tail_combine_kernel<64><<<grid, 256, 0, stream>>>(mode, H, N, st, total, a_lse, a_o, c_lse,
                                                      c_o, d_lse, d_o, d_lse_out, d_o_out, out);
  return hipGetLastError();
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
  if constexpr (NW == 4) {  // dense modes always run 4-wavefront work-groups
    if (mode == kDense) return (void)(attn_kernel<D, 4, kDense><<<grid, 256, 0, stream>>>(p));
    if (mode == kDenseCapture)
      return (void)(attn_kernel<D, 4, kDenseCapture><<<grid, 256, 0, stream>>>(p));
    if (mode == kDenseTail)
      return (void)(attn_kernel<D, 4, kDenseTail><<<grid, 256, 0, stream>>>(p));
  }
  if (mode == kSparse) attn_kernel<D, NW, kSparse><<<grid, NW * 64, 0, stream>>>(p);
  if (mode == kCaptureR) attn_kernel<D, NW, kCaptureR><<<grid, NW * 64, 0, stream>>>(p);
}

// Dense work-groups always cover 128 query rows (4 wavefronts sharing every K/V tile); the
// list modes cover one query block (block / 32 wavefronts).
hipError_t launch_attention(AttnParams p, int B, int D, AttnMode mode, hipStream_t stream) {
  const bool dense = mode == kDense || mode == kDenseCapture || mode == kDenseTail;
  const bool pair = RECAP_PAIR && mode == kSparse && p.block == 64;  // two query blocks per WG
  const int nw = (dense || pair) ? 4 : p.block / 32;
  p.mq = dense ? (p.N + 127) / 128 : pair ? (p.M + 1) / 2 : p.M;
  const int grid = B * p.H * p.mq;
  if (D == 128) {
    if (nw == 2) launch_mode<128, 2>(p, grid, mode, stream);
    else launch_mode<128, 4>(p, grid, mode, stream);
  } else {
    if (nw == 2) launch_mode<64, 2>(p, grid, mode, stream);
    else launch_mode<64, 4>(p, grid, mode, stream);
  }
  return hipGetLastError();
}

}  // namespace recap
