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
//   O^T += V^T P^T  A = V^T (row = head dim), read from the row-major V tile in LDS with
//                transpose reads, B = P^T taken straight from the S^T registers after bf16
//                rounding. The 16-key contraction step pairs lane half 0 with keys
//                {0-3, 8-11} and half 1 with {4-7, 12-15}, which is what the S^T
//                accumulator already holds.
// K and V tiles go global -> LDS directly (global_load_lds, 16 bytes per lane) into separate
// buffers, loaded while earlier tiles are multiplied (see the phase drivers below).
#include "attn_device.h"

// Build-time pipeline choices (defaults are the measured best on MI355X):
//   RECAP_STAGES4   LDS stages of the 4-wavefront (128-row) work-groups: 1 or 2
//   RECAP_PAIR      sparse calls with 64-row blocks run two query blocks per work-group
//   RECAP_PRIO      raise the wavefront priority around MFMA bursts
//   RECAP_WPE       wavefronts per SIMD targeted by register allocation
//   RECAP_PIPE      software-pipelined tile loop (next tile's QK^T under this tile's softmax)
//   RECAP_RES_LATE  pipelined sparse loop: the epilogue's residual rows go global -> LDS into
//                   the K buffers at the start of the last tile step (no K tile is read after
//                   it), so their latency hides under that step's work
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
#ifndef RECAP_PIPE  // two-stage phases without capture overlap QK^T(t+1) with tile t's weights
#define RECAP_PIPE 1
#endif
#ifndef RECAP_RES_LATE
#define RECAP_RES_LATE 1
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
//  position c ^ (key & (CH-1)), which makes the 16-byte K fragment reads bank-conflict free
//  and reduces them to "lane base XOR (ks << 5)" plus an immediate offset per 32-row tile.
//  V tile in LDS: row-major like K (row `key` holds V[key][0..D)), chunk c stored at position
//  c ^ vsw(key) (vsw below). The PV products read it with LDS transpose reads: within each
//  group of 16 lanes, ds_read_b64_tr_b16 hands lane i element i % 4 of the 8-byte chunks that
//  lanes i / 4 + {0, 4, 8, 12} of the group address. Lane s of group g addresses V[row][d0..d0+4)
//  with row = 4 (g / 2) + s / 4 and d0 = 16 (g % 2) + 4 (s % 4) (plus the k-step and d tile), so
//  lane l receives four consecutive keys at d = l % 32; two reads (keys +0 and +8) give the
//  A operand of the 32x32x16 product: keys 4h + [0, 4) and 8 + 4h + [0, 4) for lane half h,
//  which is the order of the P^T operand taken from the S^T accumulators.
template <int D>
__host__ __device__ constexpr int vsw(int key) {
  // 16-byte chunk swizzle of V rows: the 8 rows of one transpose read (4 consecutive keys per
  // lane half) land on distinct 64-byte bank groups
  return D == 128 ? ((key & 3) << 2) : (((key >> 1) & 1) << 2);
}
template <int D, int NW>
struct LaneConsts {
  static constexpr int LD = Tiles<D, NW>::LD;
  // K offsets repeat with the instruction index mod 4. With enough instructions per wavefront
  // that index is a compile-time constant; otherwise the wavefront's own instructions are
  // folded in at init (never a run-time register index).
  static constexpr int KP = LD >= 4 ? 4 : LD;
  uint32_t k_rd, v_rd;   // LDS read offsets (bytes) within a tile buffer
  uint32_t k_voff[KP];   // K DMA source offsets (bytes)
  uint32_t v_voff;       // V DMA source offset (bytes; the same for every instruction)
  __device__ void init(int lane, int wave, int64_t sn) {
    constexpr int CH = Tiles<D, NW>::CH, ROWB = Tiles<D, NW>::ROWB, KROWS = Tiles<D, NW>::KROWS;
    const int n = lane & 31, half = lane >> 5;
    k_rd = opaque(n * ROWB + ((half ^ (n & (CH - 1))) << 4));
    {
      const int g = lane >> 4, sl = lane & 15, t = sl >> 2;
      const int row = 4 * (g >> 1) + t;
      const int chunk = 2 * (g & 1) + ((sl & 3) >> 1);  // + 4 * dt, applied by XOR at the read
      v_rd = opaque((uint32_t)(row * ROWB + ((chunk ^ vsw<D>(row)) << 4) + (sl & 1) * 8));
    }
#pragma unroll
    for (int r = 0; r < KP; ++r) {
      const int x = LD >= 4 ? r : wave * LD + r;
      const int key = x * KROWS + lane / CH;  // row inside the tile (swizzle period 4 in x)
      const int c = (lane % CH) ^ (key & (CH - 1));
      k_voff[r] = opaque((uint32_t)((lane / CH) * sn * 2 + c * 16));
    }
    // rows of one V instruction are x * KROWS + lane / CH, and KROWS is a multiple of the
    // swizzle's period, so the source chunk depends on the lane only
    v_voff = opaque((uint32_t)((lane / CH) * sn * 2 + (((lane % CH) ^ vsw<D>(lane / CH)) * 16)));
  }
  __device__ uint32_t kv(int x, int it) const { return k_voff[LD >= 4 ? (x & 3) : it]; }
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

// Issue the global -> LDS loads of one 64-key V tile (rows [key0, key0 + 64) of this head,
// row-major, swizzled by vsw): the same DMA pattern as K, rows past N clamped to row N-1 (their
// weights are zero).
template <int D, int NW>
__device__ __forceinline__ void issue_v(uint32_t vbuf, const bf16_t* vp, int64_t sn, int N,
                                        int key0, int wave, int lane,
                                        const LaneConsts<D, NW>& lc) {
  constexpr int CH = Tiles<D, NW>::CH, LD = Tiles<D, NW>::LD, KROWS = Tiles<D, NW>::KROWS;
  const char* tile_base = (const char*)(vp + (int64_t)key0 * sn);
  const uint32_t row_bytes = (uint32_t)(sn * 2);
  if (key0 + 64 <= N) {
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int x = wave * LD + it;
      load_lds16(tile_base, (uint32_t)(x * KROWS * row_bytes + lc.v_voff), vbuf + x * 1024);
    }
  } else {
    asm volatile("" ::: "memory");  // the rare last tile: keep its address math out of the loop
    const int last = N - 1 - key0;
    const int ln = (int)opaque((uint32_t)lane);
#pragma unroll
    for (int it = 0; it < LD; ++it) {
      const int slot0 = (wave * LD + it) * 64;
      const int slot = slot0 + ln;
      const int key = slot / CH;
      const int c = (slot % CH) ^ vsw<D>(key);
      load_lds16(tile_base, (uint32_t)(min(key, last) * row_bytes + c * 16), vbuf + slot0 * 16);
    }
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

// The next tile's S^T = K Q^T (into n0, n1, from K tile kb) fused with this tile's weights
// (tile_exp on s0, s1): the two are independent, so the products run on the matrix cores while
// the vector ALUs compute the exponentials. The scheduling groups interleave them: after each
// product, a sixteenth of the weight computation.
template <int D, int NW>
__device__ __forceinline__ float tile_qk_exp(uint32_t kb, const bf16x8 (&qf)[D / 16],
                                             const LaneConsts<D, NW>& lc, f32x16& n0,
                                             f32x16& n1, const f32x16& s0, const f32x16& s1,
                                             float scale_log2, float m, bf16x8 (&pf)[4]) {
  constexpr int ROWB = Tiles<D, NW>::ROWB;
  constexpr int KS = D / 16;
  constexpr int VALU_PER = (96 + 2 * KS - 1) / (2 * KS);  // tile_exp: 96 vector instructions
  n0 = f32x16{};
  n1 = f32x16{};
  const uint32_t base = opaque(kb + lc.k_rd);
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const uint32_t a = base ^ (uint32_t)(ks << 5);
    const bf16x8 ka = lds_read16(a);
    const bf16x8 kb2 = lds_read16(a + 32 * ROWB);
    n0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[ks], n0, 0, 0, 0);
    n1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kb2, qf[ks], n1, 0, 0, 0);
  }
  const float acc = tile_exp(s0, s1, scale_log2, m, pf);
#pragma unroll
  for (int ks = 0; ks < 2 * KS; ++ks) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                 // one product
    __builtin_amdgcn_sched_group_barrier(0x002 | 0x400, VALU_PER, 0);  // vector + transcendental
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

// The A operand (V^T: 32 channels x 16 keys) of k-step ks and channel tile dt: two transpose
// reads of the row-major V tile (keys 4h + [0, 4) and 8 + 4h + [0, 4) of the k-step).
template <int D>
__device__ __forceinline__ bf16x8 v_operand(uint32_t base, int ks, int dt) {
  constexpr int ROWB = D * 2;
  typedef __attribute__((ext_vector_type(4))) short i16x4;
  typedef __attribute__((ext_vector_type(8))) short i16x8;
  typedef __attribute__((address_space(3))) i16x4* lds_i16x4;
  const uint32_t a = (base ^ (uint32_t)(dt << 6)) + ks * 16 * ROWB;
  const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(size_t)a);
  const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4)(size_t)(a + 8 * ROWB));
  return __builtin_bit_cast(bf16x8, (i16x8)__builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
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
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(base, ks, dt), pf[ks], o[dt],
                                                      0, 0, 0);
  }
  if (kept) {
    const uint32_t kbase = opaque(vb + lc.v_rd);  // fresh reads, not values held from above
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
        ka.o[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(v_operand<D>(kbase, ks, dt), pf[ks],
                                                           ka.o[dt], 0, 0, 0);
    }
  }
  mfma_prio_lo();
}

// Software-pipelined two-stage phase (no capture): step t computes tile t's weights and PV
// product while the next tile's QK^T runs on the matrix cores (tile_qk_exp). K runs one tile
// ahead of V: at the start of step t (one barrier), K(t+1) and V(t) have landed, K(t+2) goes
// into the buffer K(t) used and V(t+1) into the one V(t-1) used. SKIP as in attend_phase.
template <int D, int NW, bool SKIP, class Seq, class Hook>
__device__ __forceinline__ void attend_phase_pipe(Seq& seq, unsigned char* kbuf,
                                                  unsigned char* vbuf, const bf16_t* kp,
                                                  const bf16_t* vp, int64_t sn, int N,
                                                  int block, float scale_log2,
                                                  const bf16x8 (&qf)[D / 16],
                                                  f32x16 (&o)[D / 32], SoftmaxState& sm,
                                                  int wave, int lane, const LaneConsts<D, NW>& lc,
                                                  KeptAcc<D>& ka, const uint32_t* own,
                                                  Hook& last_step) {
  constexpr int LD = Tiles<D, NW>::LD, TB = Tiles<D, NW>::TILE_BYTES;
  const int half = lane >> 5;
  TileCur cur{seq.first(), 0};
  if (cur.j < 0) {
    last_step();
    return;
  }
  const uint32_t kb0 = lds_base(kbuf), vb0 = lds_base(vbuf);
  auto key0_of = [&](TileCur t) { return t.j * block + t.st * kKeyTile; };
  auto active_for = [&](TileCur t) {
    return t.j >= 0 && (!SKIP || ((own[t.j >> 5] >> (t.j & 31)) & 1u));
  };
  TileCur nxt = advance(cur, seq, block, N);
  issue_k<D, NW>(kb0, kp, sn, N, key0_of(cur), wave, lane, lc);
  issue_v<D, NW>(vb0, vp, sn, N, key0_of(cur), wave, lane, lc);
  if (nxt.j >= 0) {
    issue_k<D, NW>(kb0 + TB, kp, sn, N, key0_of(nxt), wave, lane, lc);
    wait_vmem<2 * LD>();  // K(0) landed; V(0), K(1) may be in flight
  } else {
    wait_vmem<LD>();
  }
  lds_barrier();
  f32x16 sa0, sa1, sb0, sb1;
  bool act = active_for(cur);
  if (act) tile_qk<D, NW>(kb0, qf, lc, sa0, sa1);
  int b = 0;  // K(cur + 1) is in K buffer b ^ 1, V(cur) in V buffer b
  auto step = [&](f32x16& s0, f32x16& s1, f32x16& n0, f32x16& n1) -> bool {
    const TileCur nxt2 = advance(nxt, seq, block, N);
    const bool has1 = nxt.j >= 0;
    wait_vmem<0>();  // V(cur) and K(nxt) landed
    lds_barrier();   // every wave is past the previous step: K buffer b, V buffer b ^ 1 free
    // the last tile: its scores are computed, so no wavefront reads a K buffer any more
    if (!has1) last_step();
    if (nxt2.j >= 0) issue_k<D, NW>(kb0 + b * TB, kp, sn, N, key0_of(nxt2), wave, lane, lc);
    if (has1) issue_v<D, NW>(vb0 + (b ^ 1) * TB, vp, sn, N, key0_of(nxt), wave, lane, lc);
    const bool act1 = active_for(nxt);
    if (act) {
      mask_tail(s0, s1, key0_of(cur), N, half);  // finite max: a tile has a valid key
      raise_max<D, false>(tile_rowmax(s0, s1, scale_log2), sm, o, ka);
      bf16x8 pf[4];
      // (the plain arm takes the max through an opaque copy: identical arms would let the
      // compiler hoist the exponentials out of the fused block, away from the products)
      const float acc =
          act1 ? tile_qk_exp<D, NW>(kb0 + (b ^ 1) * TB, qf, lc, n0, n1, s0, s1, scale_log2,
                                    sm.m, pf)
               : tile_exp(s0, s1, scale_log2, opaque_f(sm.m), pf);
      sm.l += acc;
      tile_pv<D, NW>(vb0 + b * TB, pf, lc, o, ka, false);
    } else if (act1) {
      tile_qk<D, NW>(kb0 + (b ^ 1) * TB, qf, lc, n0, n1);
    }
    act = act1;
    cur = nxt;
    nxt = nxt2;
    b ^= 1;
    return has1;
  };
  // two steps per trip, so that the current and next score tiles swap registers by name
  while (step(sa0, sa1, sb0, sb1) && step(sb0, sb1, sa0, sa1)) {
  }
}

// One attention phase over a block sequence, continuing the online-softmax state (m, l, o).
// STAGES = 1: one K and one V^T buffer; K(t+1) loads during softmax + PV of tile t and
//             V^T(t+1) during the QK^T of tile t+1 (four barriers per tile).
// STAGES = 2: two buffers each; tile t+2 loads into the buffers tile t has just released, so
//             every tile has a full tile of compute to land (two barriers per tile).
// SKIP: the work-group streams the union of two query blocks' kept sets; each wavefront
//       computes only the tiles of its own block's kept set (bitmap `own`).
struct NoHook {
  __device__ void operator()() const {}
};

template <int D, int NW, int STAGES, bool CAP, bool SKIP = false, class Seq, class Hook = NoHook>
__device__ __forceinline__ void attend_phase(Seq& seq, unsigned char* kbuf, unsigned char* vbuf,
                                             const bf16_t* kp, const bf16_t* vp, int64_t sn,
                                             int N, int block, float scale_log2,
                                             const bf16x8 (&qf)[D / 16], f32x16 (&o)[D / 32],
                                             SoftmaxState& sm, int wave, int lane,
                                             const LaneConsts<D, NW>& lc, KeptAcc<D>& ka,
                                             const uint32_t* own = nullptr,
                                             Hook last_step = Hook{}) {
  if constexpr (RECAP_PIPE && STAGES == 2 && !CAP) {
    attend_phase_pipe<D, NW, SKIP>(seq, kbuf, vbuf, kp, vp, sn, N, block, scale_log2, qf, o,
                                   sm, wave, lane, lc, ka, own, last_step);
    return;
  }
  constexpr int LD = Tiles<D, NW>::LD, TB = Tiles<D, NW>::TILE_BYTES;
  const int half = lane >> 5;
  TileCur cur{seq.first(), 0};
  if (cur.j < 0) return;
  const uint32_t kb0 = lds_base(kbuf), vb0 = lds_base(vbuf);
  auto issue_both = [&](TileCur t, int buf) {
    const int key0 = t.j * block + t.st * kKeyTile;
    issue_k<D, NW>(kb0 + buf * TB, kp, sn, N, key0, wave, lane, lc);
    issue_v<D, NW>(vb0 + buf * TB, vp, sn, N, key0, wave, lane, lc);
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
      issue_v<D, NW>(vb0, vp, sn, N, nxt.j * block + nxt.st * kKeyTile, wave, lane, lc);
      cur = nxt;
    }
  }
}

// The end of the grid: work-groups of unequal walks (paired kept lists of 20 to 420 tiles at
// 720p) leave the launch's last waves of work-groups unbalanced, all the more where a launch is
// only a few waves of work-groups long (480p). The last G tiles of a paired sparse grid
// therefore run longest walk first: end_order_kernel sorts them by the two query blocks' kept
// counts summed (descending, ties by tile index) into a table in the call's workspace, and the
// work-group at position r of that group takes the tile of rank r (a dispatch model of the kept
// lists: 720p 2.9% -> 1.7% imbalance, Wan-14B 480p 9.5% -> 4.5%, Wan-1.3B 480p 23% -> 10%).
// One work-group of kEndOrderTiles threads: a bitonic sort of (key, index) words in LDS.
__global__ __launch_bounds__(kEndOrderTiles) void end_order_kernel(const int32_t* __restrict__ counts,
                                                                   int M, int mq, int n, int G,
                                                                   int32_t* __restrict__ order) {
  __shared__ uint32_t key[kEndOrderTiles];
  const int j = threadIdx.x;
  uint32_t w = 0xffffffffu;  // padding sorts last
  if (j < G) {
    const int t = n - G + j, bh = t / mq, pq = t - bh * mq;
    const int32_t* c = counts + (int64_t)bh * M;
    const int c0 = min(max(c[2 * pq], 0), M);
    const int c1 = 2 * pq + 1 < M ? min(max(c[2 * pq + 1], 0), M) : 0;
    // ascending words: longer walks first (c0 + c1 <= 2 * kMaxBlocks < 32768), then index
    w = ((uint32_t)(32767 - (c0 + c1)) << 10) | (uint32_t)j;
  }
  key[j] = w;
  __syncthreads();
  for (int k = 2; k <= kEndOrderTiles; k <<= 1) {
    for (int st = k >> 1; st > 0; st >>= 1) {
      const int l = j ^ st;
      if (l > j) {
        const uint32_t a = key[j], b = key[l];
        if ((a > b) == ((j & k) == 0)) {
          key[j] = b;
          key[l] = a;
        }
      }
      __syncthreads();
    }
  }
  if (j < G) order[j] = (int32_t)(key[j] & (kEndOrderTiles - 1));
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
  // (or a pair). Runs of tiles per XCD, the XCDs in turn (all on one head), rather than one
  // range per XCD: 3% faster dense capture and sparse calls at 720p. Paired sparse walks take
  // runs of 8 pairs: with 256 pairs per head (480p) runs of 64 gave every head's same four
  // stretches of frames to the same four XCDs, and the middle frames, whose kept lists are
  // longer, loaded XCDs 1, 2, 5, 6 with up to 1.19x the mean work (Wan-14B 480p sparse call
  // 3.14 -> 2.71 ms with runs of 8, 720p -0.9%); single-block walks (block 128) keep 64.
  const bool short_runs = MODE == kSparse && NW == 4 && RECAP_PAIR && p.block == 64;
  int tile = short_runs ? xcd_runs<8>(blockIdx.x, gridDim.x) : xcd_runs<64>(blockIdx.x, gridDim.x);
  if (MODE == kSparse && p.end_order != nullptr) {  // the grid's last tiles, longest walk first
    const int g0 = (int)gridDim.x - p.end_order_g;
    if (tile >= g0) tile = g0 + min(max(((cptr_i32)p.end_order)[tile - g0], 0), p.end_order_g - 1);
  }
  const int bh = tile / p.mq, qi = tile - bh * p.mq;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t base = b * p.st.b + h * p.st.h;
  const bf16_t* kp = p.k + base;
  const bf16_t* vp = p.v + base;
  const int qrow = qi * QROWS + wave * 32 + n;
  LaneConsts<D, NW> lc;
  lc.init(lane, wave, p.st.n);

  bf16x8 qf[D / 16];
  {
    const bf16_t* src = p.q + base + (int64_t)min(qrow, p.N - 1) * p.st.n + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
  }
  // The epilogue's residual rows, requested with Q (they are read once, at the end): the
  // work-group then does not wait for them after its last tile.
  const bool has_res = MODE == kSparse && p.res != nullptr && p.o32_out == nullptr;
  // (not with the pipelined loop, whose second score tile needs these registers)
  constexpr bool PREFETCH_RES = MODE == kSparse && !RECAP_PIPE;
  // pipelined sparse loop: the residual rows go to LDS during the last tile step (rows of
  // D * 2 bytes, 16-byte chunk c of row r at position c ^ (r mod CH): conflict-free reads)
  constexpr bool LATE_RES = MODE == kSparse && RECAP_PIPE && RECAP_RES_LATE && STAGES == 2;
  constexpr int RES_WAVE_BYTES = 32 * D * 2;  // one wavefront's rows
  static_assert(!LATE_RES || NW * RES_WAVE_BYTES <= STAGES * Tiles<D, NW>::TILE_BYTES,
                "residual rows must fit in the K buffers");
  bf16x4 rpre[D / 32][4];
  if (PREFETCH_RES && has_res) {
    const bf16_t* rsrc = p.res + base + (int64_t)min(qrow, p.N - 1) * p.st.n;
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        rpre[dt][g] = *reinterpret_cast<const bf16x4*>(rsrc + dt * 32 + g * 8 + half * 4);
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
    // kept-block bitmaps of the query blocks covered by this work-group. The counts and the
    // first NW * 64 entries of each list are requested together (and with Q above), so the
    // prologue waits for one round trip, not one per count and list; entries past a count are
    // read but unused (a list row always holds M entries).
    const int nb = QROWS / p.block;  // 2 for block 64, 1 for block 128
    const int wpr = (p.M + 31) / 32;
    const int blk0 = (qi * QROWS) / p.block;
    qb = (qi * QROWS + wave * 32) / p.block;
    // unconditional loads at clamped (in-bounds) addresses, conditions applied afterwards: a
    // load behind a branch gets its wait at the branch's end
    int cnt[BLKS], first[BLKS];
#pragma unroll
    for (int lb = 0; lb < BLKS; ++lb) {
      const int64_t row = (int64_t)bh * p.M + min(blk0 + lb, p.M - 1);
      cnt[lb] = p.count[row];
      first[lb] = p.idx[row * p.M + min((int)threadIdx.x, p.M - 1)];
    }
#pragma unroll
    for (int lb = 0; lb < BLKS; ++lb)
      cnt[lb] = (lb < nb && blk0 + lb < p.M) ? min(max(cnt[lb], 0), p.M) : 0;
    for (int w = threadIdx.x; w < nb * wpr; w += NW * 64) kept_bits[w / wpr][w % wpr] = 0u;
    if (threadIdx.x < BLKS) blk_flag[threadIdx.x] = 0;
    __syncthreads();
#pragma unroll
    for (int lb = 0; lb < BLKS; ++lb) {
      if ((int)threadIdx.x < cnt[lb]) {
        const int jj = min(max(first[lb], 0), p.M - 1);
        atomicOr(&kept_bits[lb][jj >> 5], 1u << (jj & 31));
      }
      const int64_t row = (int64_t)bh * p.M + min(blk0 + lb, p.M - 1);
      for (int c = threadIdx.x + NW * 64; c < cnt[lb]; c += NW * 64) {
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

  // consume the Q fragments (and the residual rows) here, so the compiler's waits for these
  // loads sit before the loop (the tile loads in the loop are invisible to its wait-count
  // bookkeeping)
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
  if (PREFETCH_RES && has_res) {
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
      for (int g = 0; g < 4; ++g) asm volatile("" ::"v"(rpre[dt][g]));
  }

  int nlist = 0;
  auto last_step = [&]() {
    if constexpr (LATE_RES) {
      if (has_res) {
        constexpr int CH = D / 8;  // 16-byte chunks per row
        const int r0 = min(qi * QROWS + wave * 32, p.N - 1);  // the wavefront's first row
        const char* rbase = (const char*)(p.res + base + (int64_t)r0 * p.st.n);
        const uint32_t dst = lds_base(kbuf) + wave * RES_WAVE_BYTES;
        const int ln = (int)opaque((uint32_t)lane);
#pragma unroll
        for (int x = 0; x < RES_WAVE_BYTES / 1024; ++x) {
          const int slot = x * 64 + ln, row = slot / CH, pos = slot % CH;
          const int c = pos ^ (row & (CH - 1));
          const int rr = min(r0 + row, p.N - 1) - r0;  // rows past N read row N - 1 (unused)
          load_lds16(rbase, (uint32_t)(rr * (uint32_t)(p.st.n * 2) + c * 16), dst + x * 1024);
        }
      }
    }
  };
  if (PAIRABLE && pair) {
    UnionSeq seq{kept_bits[0], kept_bits[1], p.M, 0};
    attend_phase<D, NW, STAGES, false, true>(seq, kbuf, vbuf, kp, vp, p.st.n, p.N, p.block,
                                     p.scale_log2, qf, o, sm, wave, lane, lc, ka,
                                     kept_bits[(wave * 32) / p.block], last_step);
  } else if (MODE == kDense || CAP) {
    // staggered start at the diagonal: neighbouring work-groups stream the same K/V tiles at
    // nearly the same time, which keeps them in L2
    AllSeq seq{0, p.M, min((qi * QROWS) / p.block, p.M - 1)};
    attend_phase<D, NW, STAGES, CAP>(seq, kbuf, vbuf, kp, vp, p.st.n, p.N, p.block,
                             p.scale_log2, qf, o, sm, wave, lane, lc, ka);
  } else {
    const int32_t* lst = p.idx + (int64_t)tile * p.M;  // one query block per work-group here
    nlist = min(max(((cptr_i32)p.count)[tile], 0), p.M);
    if (MODE == kCaptureR && ((cptr_u8)p.flags)[tile] == 0) return;  // done in the dense pass
    ListSeq seq{lst, nlist, 0, p.M};
    attend_phase<D, NW, STAGES, false>(seq, kbuf, vbuf, kp, vp, p.st.n, p.N, p.block,
                               p.scale_log2, qf, o, sm, wave, lane, lc, ka, nullptr,
                               last_step);
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

  // this wavefront's residual rows are in LDS (waited for before any lane leaves: a wavefront
  // whose rows all lie past N ends here, with no load of its own still in flight)
  if (LATE_RES && has_res) wait_vmem<0>();
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
  const float c = p.res_scale.v[h];
  const uint32_t res_lds = lds_base(kbuf) + wave * RES_WAVE_BYTES + n * (D * 2) + half * 8;
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
        bf16x4 r4;
        if constexpr (PREFETCH_RES) r4 = rpre[dt][g];
        else if constexpr (LATE_RES)
          r4 = *reinterpret_cast<const __attribute__((address_space(3))) bf16x4*>(
              (size_t)(res_lds + (((dt * 4 + g) ^ (n & (D / 8 - 1))) << 4)));
        else r4 = *reinterpret_cast<const bf16x4*>(p.res + orow + d0);
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
// weights, the coarse output the weighted mean of the V̄_j. With the moment refinements (MOM)
// each weight's exponent also gets (s^2 / 2) * sum_d q_d^2 var_jd from the block's key
// variances, and the output gets s * C q_t from the pooled within-block value-key covariance C.
// Same tile math as attn_kernel (4 wavefronts, 128 query rows, 64 pooled keys per tile, one
// LDS stage: a row has only ceil(M / 64) tiles), with the pooled scores from the hi + lo key
// pair. Kept blocks and pooled keys past M get score -inf; the last pooled key's weight
// carries its shorter block.
// ------------------------------------------------------------------------------------------
// Pooled keys as a pair of bf16 values, hi = bf16(K̄) and lo = bf16(K̄ - hi) (about 16
// significant bits, so the pooled scores are as accurate as the token scores, whose bf16
// operands are exact), pooled values as bf16. Element e of [B*H][mpad][D]; rows >= M are zero.
// With the moment refinements, also the per-dimension key variances scaled by s/2 (the factor
// that makes their product with q^2 the second-order log-mass term once the scores are scaled
// by s), bf16, in the same layout.
template <int D>
__global__ __launch_bounds__(256) void tail_keys_kernel(const float* __restrict__ kbar,
                                                        const float* __restrict__ vbar,
                                                        const float* __restrict__ var,
                                                        float var_scale, int M, int mpad,
                                                        int64_t total,
                                                        bf16_t* __restrict__ kb_hi,
                                                        bf16_t* __restrict__ kb_lo,
                                                        bf16_t* __restrict__ vb16,
                                                        bf16_t* __restrict__ sv16) {
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
    if (var != nullptr) sv16[e] = (bf16_t)(j < M ? var_scale * var[src] : 0.f);
  }
}

// Kept lists -> one bitmap row per query block (bit j set: key block j kept), wbits words with
// the last one zero, so that a 64-key tile's two words can always be read.
__global__ __launch_bounds__(64) void kept_bits_kernel(const int32_t* __restrict__ count,
                                                       const int32_t* __restrict__ idx, int M,
                                                       int wbits, uint32_t* __restrict__ bits) {
  __shared__ uint32_t w[kMaxBlocks / 32 + 1];
  const int64_t row = blockIdx.x;
  for (int i = threadIdx.x; i < wbits; i += 64) w[i] = 0u;
  __syncthreads();
  const int cnt = min(max(count[row], 0), M);
  for (int c = threadIdx.x; c < cnt; c += 64) {
    const int jj = min(max(idx[row * M + c], 0), M - 1);
    atomicOr(&w[jj >> 5], 1u << (jj & 31));
  }
  __syncthreads();
  for (int i = threadIdx.x; i < wbits; i += 64) bits[row * wbits + i] = w[i];
}

// ------------------------------------------------------------------------------------------
// Moment statistics of the key and value blocks for the refined coarse tail (paperpeel.com
// RECAP Sec. 3.2: key variance refines the block log-mass at second order, the pooled
// value-key covariance refines the value at first order). Work-group = (b*h, slice of
// kStatSlice key blocks). Per block, thread (token pair tp, 8-dim chunk c) loads 16 bytes of K
// and of V for two adjacent tokens per pass (coalesced rows), subtracts the block means (fp32),
// adds the squared key deviations to eight per-thread sums (reduced over the token pairs in
// LDS: the per-dimension variance, population form) and writes the centred keys and values,
// bf16, transposed into LDS ([dim][token], two tokens per 4-byte write, rows padded by 16
// bytes). The four wavefronts then add the block's (v - V̄)(k - K̄)^T to a D x D accumulator
// with bf16 MFMA 32x32x16 (A: value rows, B: key rows, contraction over the tokens; wave w
// owns value rows 32w.. at D = 128, one 32 x 32 tile at D = 64). The slice's sum is written
// as one fp32 partial; tail_cov_reduce_kernel adds the slices in a fixed order.
// ------------------------------------------------------------------------------------------
template <int D, int BLK>
__global__ __launch_bounds__(256) void tail_stats_kernel(const bf16_t* __restrict__ k,
                                                         const bf16_t* __restrict__ v,
                                                         Strides st, int H, int N, int M,
                                                         int nslice,
                                                         const float* __restrict__ kbar,
                                                         const float* __restrict__ vbar,
                                                         float* __restrict__ var,
                                                         float* __restrict__ cov_part) {
  constexpr int CH = D / 8;              // 16-byte chunks per token row
  constexpr int TPW = 256 / CH;          // token pairs per pass
  constexpr int PASSES = BLK / (2 * TPW);
  constexpr int RS = BLK + 8;            // LDS row stride (bf16 elements)
  constexpr int TILES = D == 128 ? 4 : 1;  // 32 x 32 output tiles per wavefront
  __shared__ __align__(16) bf16_t kt[D * RS];
  __shared__ __align__(16) bf16_t vt[D * RS];
  __shared__ float vred[TPW][D];
  const int bh = blockIdx.x / nslice, slice = blockIdx.x - bh * nslice;
  const int b = bh / H, h = bh - b * H;
  const bf16_t* kp = k + b * st.b + h * st.h;
  const bf16_t* vp = v + b * st.b + h * st.h;
  const int c = threadIdx.x % CH, tp = threadIdx.x / CH;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int rt = D == 128 ? wave : wave >> 1;  // this wavefront's row tile of the output
  f32x16 acc[TILES];
#pragma unroll
  for (int t = 0; t < TILES; ++t) acc[t] = f32x16{};
  typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
  const int j0 = slice * kStatSlice, j1 = min(M, j0 + kStatSlice);
  for (int j = j0; j < j1; ++j) {
    const int t0 = j * BLK, nj = min(BLK, N - t0);
    const float* kmp = kbar + ((int64_t)bh * M + j) * D + c * 8;
    const float* vmp = vbar + ((int64_t)bh * M + j) * D + c * 8;
    float km[8], vm[8], sq[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      km[e] = kmp[e];
      vm[e] = vmp[e];
      sq[e] = 0.f;
    }
#pragma unroll
    for (int ps = 0; ps < PASSES; ++ps) {
      const int u0 = ps * 2 * TPW + 2 * tp;  // this thread's first token of the pass
      bf16x8 kx[2], vx[2];
#pragma unroll
      for (int w = 0; w < 2; ++w) {
        const int u = u0 + w;
        if (u < nj) {
          kx[w] = *reinterpret_cast<const bf16x8*>(kp + (int64_t)(t0 + u) * st.n + c * 8);
          vx[w] = *reinterpret_cast<const bf16x8*>(vp + (int64_t)(t0 + u) * st.n + c * 8);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        bf16x2 kw, vw;
#pragma unroll
        for (int w = 0; w < 2; ++w) {
          const bool ok = u0 + w < nj;
          const float kd = ok ? (float)kx[w][e] - km[e] : 0.f;
          const float vd = ok ? (float)vx[w][e] - vm[e] : 0.f;
          sq[e] += kd * kd;
          kw[w] = (bf16_t)kd;
          vw[w] = (bf16_t)vd;
        }
        *reinterpret_cast<bf16x2*>(&kt[(c * 8 + e) * RS + u0]) = kw;
        *reinterpret_cast<bf16x2*>(&vt[(c * 8 + e) * RS + u0]) = vw;
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) vred[tp][c * 8 + e] = sq[e];
    __syncthreads();
    if (threadIdx.x < D) {
      float tot = 0.f;
#pragma unroll
      for (int q = 0; q < TPW; ++q) tot += vred[q][threadIdx.x];
      var[((int64_t)bh * M + j) * D + threadIdx.x] = tot / (float)nj;
    }
#pragma unroll
    for (int ks = 0; ks < BLK / 16; ++ks) {
      const int u0 = ks * 16 + half * 8;
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(&vt[(rt * 32 + n) * RS + u0]);
#pragma unroll
      for (int t = 0; t < TILES; ++t) {
        const int ct = D == 128 ? t : (wave & 1);
        const bf16x8 bb = *reinterpret_cast<const bf16x8*>(&kt[(ct * 32 + n) * RS + u0]);
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bb, acc[t], 0, 0, 0);
      }
    }
    __syncthreads();  // LDS rows and vred are rewritten by the next block
  }
  float* dst = cov_part + ((int64_t)bh * nslice + slice) * D * D;
#pragma unroll
  for (int t = 0; t < TILES; ++t) {
    const int ct = D == 128 ? t : (wave & 1);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = rt * 32 + ((r >> 2) << 3) + half * 4 + (r & 3);  // value dimension
      dst[row * D + ct * 32 + n] = acc[t][r];
    }
  }
}

// x = scale * (sum over the slices of cov_part[bh][slice][r][c]), written as a bf16 pair:
// cov16[e] = bf16(x) and cov16[total + e] = bf16(x - bf16(x)) (about 16 significant bits)
template <int D>
__global__ __launch_bounds__(256) void tail_cov_reduce_kernel(const float* __restrict__ cov_part,
                                                              int nslice, float scale,
                                                              int64_t total,
                                                              bf16_t* __restrict__ cov16) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= total) return;
  const int64_t bh = e / (D * D), rc = e - bh * (D * D);
  const float* src = cov_part + bh * nslice * D * D + rc;
  float acc = 0.f;
  for (int sl = 0; sl < nslice; ++sl) acc += src[(int64_t)sl * D * D];
  const float x = scale * acc;
  const bf16_t hi = (bf16_t)x;
  cov16[e] = hi;
  cov16[total + e] = (bf16_t)(x - (float)hi);
}

// MOM: the moment refinements. The block log-mass gains (s^2/2) sum_d q_d^2 Var_j(k_d): one
// more product per tile, of bf16(q^2) (held in registers like the Q fragments) with the
// scaled variances (an LDS tile loaded with the pooled keys), added to the same score
// accumulators; the output gains s C q, computed after the loop as C Q^T from two (D = 128) or
// one (D = 64) 64-row tiles of the scaled covariance loaded into the pooled-key buffers.
// Kept blocks come from bitmap rows in global memory (two words per tile, read through the
// scalar cache), which leaves LDS to the tiles: 80 KB with the variance tile at D = 128, two
// work-groups per CU.
template <int D, bool MOM>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void tail_kernel(TailParams p) {
  constexpr int NW = 4, QROWS = 128, TB = Tiles<D, NW>::TILE_BYTES;
  // K̄ hi and lo (and the variance tile): one stage, the next tile's loads issued as soon as
  // this tile's QK^T products have read it; V̄^T: two stages, the next tile's loads issued at
  // the top of each step.
  __shared__ __align__(256) unsigned char kbuf[TB];
  __shared__ __align__(256) unsigned char klbuf[TB];
  __shared__ __align__(256) unsigned char vbuf[2 * TB];
  __shared__ __align__(256) unsigned char sbuf[MOM ? TB : 256];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / p.mq, qi = tile - bh * p.mq;
  const int b = bh / p.H, h = bh - b * p.H;
  const int64_t base = b * p.st.b + h * p.st.h;
  const int qrow = qi * QROWS + wave * 32 + n;
  LaneConsts<D, NW> lc;
  lc.init(lane, wave, (int64_t)D);
  bf16x8 qf[D / 16];
  bf16x8 q2f[MOM ? D / 16 : 1];
  {
    const bf16_t* src = p.q + base + (int64_t)min(qrow, p.N - 1) * p.st.n + half * 8;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) qf[ks] = *reinterpret_cast<const bf16x8*>(src + ks * 16);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));
    if constexpr (MOM) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = (float)qf[ks][e];
          q2f[ks][e] = (bf16_t)(x * x);
        }
    }
  }
  // this wavefront's kept-block bitmap row (its query block; rows past the last block clamp)
  const int blk = min((qi * QROWS + wave * 32) / p.block, p.M - 1);
  const cptr_u32 own = (cptr_u32)(p.bits + ((int64_t)bh * p.M + blk) * p.wbits);

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  SoftmaxState sm{-INFINITY, 0.f};
  KeptAcc<D> none;
  const uint32_t kb0 = lds_base(kbuf), kl0 = lds_base(klbuf), vb0 = lds_base(vbuf);
  const uint32_t sb0 = MOM ? lds_base(sbuf) : 0u;
  const bf16_t* kp = p.kb + (int64_t)bh * p.mpad * D;
  const bf16_t* klp = p.kb_lo + (int64_t)bh * p.mpad * D;
  const bf16_t* svp = MOM ? p.sv + (int64_t)bh * p.mpad * D : nullptr;
  const bf16_t* vbp = p.vb + (int64_t)bh * p.mpad * D;  // rows >= M are zero
  const int ntile = (p.M + kKeyTile - 1) / kKeyTile;
  issue_v<D, NW>(vb0, vbp, (int64_t)D, p.mpad, 0, wave, lane, lc);
  issue_k<D, NW>(kb0, kp, (int64_t)D, p.M, 0, wave, lane, lc);
  issue_k<D, NW>(kl0, klp, (int64_t)D, p.M, 0, wave, lane, lc);
  if constexpr (MOM) issue_k<D, NW>(sb0, svp, (int64_t)D, p.M, 0, wave, lane, lc);
  for (int t = 0; t < ntile; ++t) {
    const int key0 = t * kKeyTile;
    const uint32_t vt = vb0 + (t & 1) * TB;
    // this wavefront's loads of tile t (V̄ issued one step ago, K̄ in the previous step's
    // middle) have landed; the barrier makes them everyone's and frees the other V̄ stage
    wait_vmem<0>();
    lds_barrier();
    if (t + 1 < ntile)
      issue_v<D, NW>(vb0 + ((t + 1) & 1) * TB, vbp, (int64_t)D, p.mpad, key0 + kKeyTile, wave, lane, lc);
    f32x16 s0, s1;
    tile_qk<D, NW>(kb0, qf, lc, s0, s1);
    tile_qk<D, NW, true>(kl0, qf, lc, s0, s1);  // + q . (K̄ - hi)
    if constexpr (MOM) tile_qk<D, NW, true>(sb0, q2f, lc, s0, s1);  // + q^2 . (s/2) Var
    lds_barrier();  // every wavefront has read K̄ of tile t
    if (t + 1 < ntile) {
      issue_k<D, NW>(kb0, kp, (int64_t)D, p.M, key0 + kKeyTile, wave, lane, lc);
      issue_k<D, NW>(kl0, klp, (int64_t)D, p.M, key0 + kKeyTile, wave, lane, lc);
      if constexpr (MOM) issue_k<D, NW>(sb0, svp, (int64_t)D, p.M, key0 + kKeyTile, wave, lane, lc);
    }
    // scores in log2 units; kept blocks and pooled keys past M get -inf, the last pooled key
    // the log2 of its share of a full block. Keys key0 + kr and key0 + 32 + kr are bit kr of
    // words key0 / 32 and key0 / 32 + 1 of the kept bitmap (key0 is a multiple of 64; the
    // row's last word is zero, and every bit past M is masked anyway).
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
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if constexpr (MOM) {
    // value compensation s C q: C (scaled by s/N) as a bf16 pair hi + lo, in 64-row tiles, in
    // the pooled-key and variance buffers (no wavefront reads them after the last tile's
    // second barrier) and, at D = 128, in the V̄ stage the last tile did not use (every
    // wavefront finished reading it before the last tile's first barrier)
    const bf16_t* cp = p.cov + (int64_t)bh * D * D;
    const bf16_t* cpl = cp + (int64_t)p.BH * D * D;
    const uint32_t free_v = vb0 + (((ntile - 1) & 1) ^ 1) * TB;
    issue_k<D, NW>(kb0, cp, (int64_t)D, D, 0, wave, lane, lc);
    issue_k<D, NW>(kl0, cpl, (int64_t)D, D, 0, wave, lane, lc);
    if (D == 128) {
      issue_k<D, NW>(sb0, cp, (int64_t)D, D, 64, wave, lane, lc);
      issue_k<D, NW>(free_v, cpl, (int64_t)D, D, 64, wave, lane, lc);
    }
    wait_vmem<0>();
    lds_barrier();
    f32x16 c0, c1;
    tile_qk<D, NW>(kb0, qf, lc, c0, c1);
    tile_qk<D, NW, true>(kl0, qf, lc, c0, c1);
    if (lt > 0.f) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        o[0][r] = o[0][r] * inv + c0[r];
        o[1][r] = o[1][r] * inv + c1[r];
      }
    }
    if constexpr (D == 128) {
      tile_qk<D, NW>(sb0, qf, lc, c0, c1);
      tile_qk<D, NW, true>(free_v, qf, lc, c0, c1);
      if (lt > 0.f) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          o[2][r] = o[2][r] * inv + c0[r];
          o[3][r] = o[3][r] * inv + c1[r];
        }
      }
    }
  }
  if (qrow >= p.N) return;
  const int64_t srow = (int64_t)bh * p.N + qrow;
  if (half == 0) p.tail_lse[srow] = lt > 0.f ? (sm.m + log2f(lt)) * kLn2 + p.ln_block : -INFINITY;
  const float scale_out = MOM ? (lt > 0.f ? 1.0f : 0.f) : inv;  // MOM: already normalised
  float* to = p.tail_o + srow * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = o[dt][g * 4 + e] * scale_out;
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
hipError_t launch_tail_keys(const float* kbar, const float* vbar, const float* var,
                            float var_scale, int BH, int M, int D, int mpad, bf16_t* kb_hi,
                            bf16_t* kb_lo, bf16_t* vb16, bf16_t* sv16, hipStream_t stream) {
  const int64_t total = (int64_t)BH * mpad * D;
  const int grid = (int)(total < 65536LL * 256 ? (total + 255) / 256 : 65536);
  if (D == 128)
    tail_keys_kernel<128><<<grid, 256, 0, stream>>>(kbar, vbar, var, var_scale, M, mpad, total,
                                                    kb_hi, kb_lo, vb16, sv16);
  else
    tail_keys_kernel<64><<<grid, 256, 0, stream>>>(kbar, vbar, var, var_scale, M, mpad, total,
                                                   kb_hi, kb_lo, vb16, sv16);
  return hipGetLastError();
}

hipError_t launch_kept_bits(const int32_t* count, const int32_t* idx, int rows, int M, int wbits,
                            uint32_t* bits, hipStream_t stream) {
  kept_bits_kernel<<<rows, 64, 0, stream>>>(count, idx, M, wbits, bits);
  return hipGetLastError();
}

hipError_t launch_tail_stats(const bf16_t* k, const bf16_t* v, Strides st, int B, int H, int N,
                             int D, int block, const float* kbar, const float* vbar, float* var,
                             float* cov_part, float cov_scale, bf16_t* cov16,
                             hipStream_t stream) {
  const int M = (N + block - 1) / block;
  const int nslice = (M + kStatSlice - 1) / kStatSlice;
  const int grid = B * H * nslice;
  if (D == 128) {
    if (block == 64)
      tail_stats_kernel<128, 64><<<grid, 256, 0, stream>>>(k, v, st, H, N, M, nslice, kbar,
                                                           vbar, var, cov_part);
    else
      tail_stats_kernel<128, 128><<<grid, 256, 0, stream>>>(k, v, st, H, N, M, nslice, kbar,
                                                            vbar, var, cov_part);
  } else {
    if (block == 64)
      tail_stats_kernel<64, 64><<<grid, 256, 0, stream>>>(k, v, st, H, N, M, nslice, kbar, vbar,
                                                          var, cov_part);
    else
      tail_stats_kernel<64, 128><<<grid, 256, 0, stream>>>(k, v, st, H, N, M, nslice, kbar,
                                                           vbar, var, cov_part);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t total = (int64_t)B * H * D * D;
  const int rgrid = (int)((total + 255) / 256);
  if (D == 128)
    tail_cov_reduce_kernel<128><<<rgrid, 256, 0, stream>>>(cov_part, nslice, cov_scale, total,
                                                           cov16);
  else
    tail_cov_reduce_kernel<64><<<rgrid, 256, 0, stream>>>(cov_part, nslice, cov_scale, total,
                                                          cov16);
  return hipGetLastError();
}

hipError_t launch_tail(TailParams p, int B, int D, hipStream_t stream) {
  p.mq = (p.N + 127) / 128;
  const int grid = B * p.H * p.mq;
  const bool mom = p.sv != nullptr;
  if (D == 128) {
    if (mom) tail_kernel<128, true><<<grid, 256, 0, stream>>>(p);
    else tail_kernel<128, false><<<grid, 256, 0, stream>>>(p);
  } else {
    if (mom) tail_kernel<64, true><<<grid, 256, 0, stream>>>(p);
    else tail_kernel<64, false><<<grid, 256, 0, stream>>>(p);
  }
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

int sparse_end_order_tiles(int B, int H, int M, int block) {
  if (!(RECAP_PAIR && block == 64)) return 0;  // paired walks only: single-block walks are short
  const int64_t n = (int64_t)B * H * ((M + 1) / 2);
  return (int)(n < kEndOrderTiles ? n : kEndOrderTiles);
}

hipError_t launch_end_order(const int32_t* counts, int B, int H, int M, int G, int32_t* order,
                            hipStream_t stream) {
  const int mq = (M + 1) / 2;
  end_order_kernel<<<1, kEndOrderTiles, 0, stream>>>(counts, M, mq, B * H * mq, G, order);
  return hipGetLastError();
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
