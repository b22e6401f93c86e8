// FP8 variant of the block-sparse attention products on gfx950 (MXFP8, E4M3 elements).
//
// The pages name FP8 quantisation with fused kernels for sparse video attention (the RECAP
// page at thelatestinai.com, second abstract) without a format. Here it is the one gfx950's
// matrix cores consume natively: OCP microscaling FP8, E4M3 elements with one power-of-two
// (E8M0) scale per 32 consecutive elements of each product's contraction dimension, fed to
// v_mfma_scale_f32_32x32x64_f8f6f4. Its 64 contraction slots of a row or column are held by
// two lanes (l and l + 32, 32 bytes each) and form two scale blocks: block b is bytes 16b..16b+15
// of both lanes, scaled by the scale operand of lane l + 32b (measured on the device; a lane's
// own 32 bytes are not one block). Each operand is laid out so that block b is one MX group.
//
//   S^T = K Q^T   A = K tile (row = key), B = Q^T (column = query). For head dims 64m..64m+63,
//                 lane half h holds dims 64m + 16h + [0, 16) and 64m + 32 + 16h + [0, 16), so
//                 block b = dims 64m + 32b + [0, 32), the MX group whose scale lane half b gives.
//                 D/64 instructions per 32 keys.
//   O^T += V^T P^T A = V^T tile (row = channel), B = P^T straight from the S^T accumulators:
//                 with the key tile in natural order, lane half h holds keys
//                 32(e/16) + 8((e%16)/4) + 4h + e%4 at slot e, so block b = keys 32b..32b+31.
//                 The weights of each block get one exponent (from the block's largest score,
//                 folded into the exp2 argument, so the largest weight lands in [128, 256)); V
//                 is scaled per channel and 32-key group, its bytes stored in the slots' key
//                 order. D/32 instructions per 64 keys.
// The softmax is the bf16 kernel's (exp2 with the scale folded into one FMA, lazy rescale);
// the row sum is a fifth product per tile (all-ones A operand) over the FP8-rounded weights the
// O^T product uses. Sparse mode only: 128 query rows per work-group (two 64-row query blocks
// over the union of their kept lists, or one 128-row block), LDS stages of 8.25 KB K and V
// tiles (D = 128) DMA'd with 16-byte lanes, one barrier per tile.
#include "attn_device.h"

namespace recap {

typedef __attribute__((ext_vector_type(8))) int i32x8;
typedef __attribute__((ext_vector_type(4))) int i32x4;

// ---- MX encoding, shared by every packer ---------------------------------------------------
// Block exponent E = floor(log2(amax)) - 7 in [-127, 127] (-127 for an all-zero block), so the
// largest scaled magnitude lies in [128, 256) and the E4M3 conversion (round to nearest even,
// no saturation on this part) never overflows.
__device__ __forceinline__ int mx_exponent(float amax) {
  if (!(amax > 0.f)) return -127;
  const int e = __builtin_amdgcn_frexp_expf(amax) - 8;  // amax = f * 2^k, f in [0.5, 1)
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}
// 32 values -> 8 dwords of E4M3 bytes (element i in byte i % 4 of dword i / 4); returns E + 127.
__device__ __forceinline__ uint32_t mx_encode32(const float (&x)[32], uint32_t (&w)[8]) {
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(x[i]));
  const int e = mx_exponent(amax);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = __builtin_amdgcn_ldexpf(x[4 * i], -e), b = __builtin_amdgcn_ldexpf(x[4 * i + 1], -e);
    const float c = __builtin_amdgcn_ldexpf(x[4 * i + 2], -e), d = __builtin_amdgcn_ldexpf(x[4 * i + 3], -e);
    int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
    w[i] = (uint32_t)v;
  }
  return (uint32_t)(e + 127);
}
__device__ __forceinline__ void load32_bf16(const bf16_t* src, float (&x)[32]) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(src + 8 * c);
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * c + e] = (float)v[e];
  }
}
__device__ __forceinline__ void store32(uint8_t* dst, const uint32_t (&w)[8]) {
  *reinterpret_cast<i32x4*>(dst) = i32x4{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
  *reinterpret_cast<i32x4*>(dst + 16) = i32x4{(int)w[4], (int)w[5], (int)w[6], (int)w[7]};
}

// Key (inside a 64-key tile) of P^T / V^T operand slot e of lane half h.
__device__ __forceinline__ int pv_key(int h, int e) {
  return 32 * (e >> 4) + 8 * ((e & 15) >> 2) + 4 * h + (e & 3);
}

// ---- packers -------------------------------------------------------------------------------
// Token-major MX encoding along the head dimension, one thread per (token, 32-dim group):
// codes [B*H][N][D], scales [B*H][N][D/32] (the Q operand, and the test/export layout).
template <int D>
__global__ __launch_bounds__(256) void mx_rows_kernel(const bf16_t* __restrict__ x, Strides st,
                                                      int H, int N, int64_t total,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  constexpr int G = D / 32;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * 256) {
    const int64_t row = g / G;  // (b*H + h)*N + t
    const int grp = (int)(g - row * G);
    const int64_t bh = row / N;
    const int t = (int)(row - bh * N);
    const int64_t b = bh / H, h = bh - b * H;
    float v[32];
    load32_bf16(x + b * st.b + h * st.h + (int64_t)t * st.n + grp * 32, v);
    uint32_t w[8];
    const uint32_t s = mx_encode32(v, w);
    store32(codes + row * D + grp * 32, w);
    scales[row * G + grp] = (uint8_t)s;
  }
}

// Channel-major MX encoding along the tokens (32-token groups from token 0), the V operand's
// grouping, in the test/export layout: codes [B*H][N][D] (token-major), scales
// [B*H][ceil(N/32)][D]. One thread per (32-token group, channel).
template <int D>
__global__ __launch_bounds__(256) void mx_cols_kernel(const bf16_t* __restrict__ x, Strides st,
                                                      int H, int N, int64_t total,
                                                      uint8_t* __restrict__ codes,
                                                      uint8_t* __restrict__ scales) {
  const int NG = (N + 31) / 32;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * 256) {
    const int d = (int)(g % D);
    const int64_t rg = g / D;  // (b*H + h)*NG + group
    const int64_t bh = rg / NG;
    const int tg = (int)(rg - bh * NG);
    const int64_t b = bh / H, h = bh - b * H;
    const bf16_t* src = x + b * st.b + h * st.h + d;
    float v[32];
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      const int t = tg * 32 + i;
      v[i] = t < N ? (float)src[(int64_t)t * st.n] : 0.f;
    }
    uint32_t w[8];
    const uint32_t s = mx_encode32(v, w);
    uint8_t* dst = codes + (bh * N + (int64_t)tg * 32) * D + d;
#pragma unroll
    for (int i = 0; i < 32; ++i)
      if (tg * 32 + i < N) dst[(int64_t)i * D] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    scales[rg * D + d] = (uint8_t)s;
  }
}

// Packed K tiles for the attention kernel: per (b*h, 64-key tile) 64 rows of D code bytes
// (keys in order; keys >= N zero) followed by 2*D scale bytes laid out as the lanes read them:
// [half h][row n][s][m] = scale of key 32 s + n, dims 64 m + 32 h ..+31. One thread per
// (key, 32-dim group).
template <int D>
__global__ __launch_bounds__(256) void mx_k_tiles_kernel(const bf16_t* __restrict__ k,
                                                         Strides st, int H, int N, int ntile,
                                                         int64_t total,
                                                         uint8_t* __restrict__ out) {
  constexpr int G = D / 32, TS = 66 * D;
  for (int64_t g = (int64_t)blockIdx.x * 256 + threadIdx.x; g < total;
       g += (int64_t)gridDim.x * 256) {
    const int grp = (int)(g % G);
    const int i = (int)((g / G) & 63);
    const int64_t tl = g / (64 * G);  // bh * ntile + tile
    const int64_t bh = tl / ntile;
    const int tile = (int)(tl - bh * ntile);
    const int key = tile * 64 + i;
    const int64_t b = bh / H, h = bh - b * H;
    float v[32];
    if (key < N) {
      load32_bf16(k + b * st.b + h * st.h + (int64_t)key * st.n + grp * 32, v);
    } else {
#pragma unroll
      for (int e = 0; e < 32; ++e) v[e] = 0.f;
    }
    uint32_t w[8];
    const uint32_t s = mx_encode32(v, w);
    uint8_t* t0 = out + tl * TS;
    store32(t0 + i * D + grp * 32, w);
    const int n = i & 31, si = i >> 5, m = grp >> 1, hh = grp & 1;
    t0[64 * D + ((hh * 32 + n) * 2 + si) * (D / 64) + m] = (uint8_t)s;
  }
}

// Packed V tiles: per (b*h, 64-key tile) D rows (channels) of 64 code bytes, byte 32 h + e
// holding key pv_key(h, e) (keys >= N zero), followed by 2*D scale bytes laid out as the lanes
// read them: [half h][row n][dt] = scale of channel 32 dt + n, keys 32 h .. 32 h + 31 (the MX
// groups are 32 consecutive keys). One work-group per tile: the 64 x D bf16 tile is staged
// through LDS, then one thread per (channel, group) encodes its 32 keys.
template <int D>
__global__ __launch_bounds__(256) void mx_v_tiles_kernel(const bf16_t* __restrict__ v,
                                                         Strides st, int H, int N, int ntile,
                                                         uint8_t* __restrict__ out) {
  constexpr int TS = 66 * D;
  __shared__ float tile[64][D + 1];
  const int64_t tl = blockIdx.x;
  const int64_t bh = tl / ntile;
  const int t = (int)(tl - bh * ntile);
  const int64_t b = bh / H, h = bh - b * H;
  const bf16_t* src = v + b * st.b + h * st.h;
  for (int s = threadIdx.x; s < 64 * (D / 8); s += 256) {
    const int key = s / (D / 8), c = s - key * (D / 8);
    const int tok = t * 64 + key;
    bf16x8 x = {};
    if (tok < N) x = *reinterpret_cast<const bf16x8*>(src + (int64_t)tok * st.n + c * 8);
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[key][c * 8 + e] = (float)x[e];
  }
  __syncthreads();
  if (threadIdx.x >= 2 * D) return;
  const int d = threadIdx.x >> 1, g = threadIdx.x & 1;
  float x[32];
#pragma unroll
  for (int i = 0; i < 32; ++i) x[i] = tile[g * 32 + i][d];
  uint32_t w[8];
  const uint32_t s = mx_encode32(x, w);  // group g: keys 32 g .. 32 g + 31
  uint8_t* t0 = out + tl * TS;
  // key 32 g + i sits at slot e of lane half h with pv_key(h, e) = 32 g + i:
  // e = 16 g + 4 (i / 8) + i % 4, h = (i / 4) % 2
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int h = (i >> 2) & 1, e = 16 * g + 4 * (i >> 3) + (i & 3);
    t0[d * 64 + 32 * h + e] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
  }
  t0[64 * D + (g * 32 + (d & 31)) * (D / 32) + (d >> 5)] = (uint8_t)s;
}

// ---- attention -----------------------------------------------------------------------------
// 16-byte LDS read as 4 ints
__device__ __forceinline__ i32x4 lds_read16i(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) i32x4*>((size_t)addr);
}
__device__ __forceinline__ i32x8 join(i32x4 a, i32x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ uint32_t lds_read_u32(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint32_t*>((size_t)addr);
}
__device__ __forceinline__ uint32_t lds_read_u16(uint32_t addr) {
  return *reinterpret_cast<const __attribute__((address_space(3))) uint16_t*>((size_t)addr);
}
// Scaled FP8 product, both operands E4M3, scales in byte 0 of sa / sb.
__device__ __forceinline__ f32x16 mx_mfma(i32x8 a, i32x8 b, f32x16 c, uint32_t sa, uint32_t sb) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, (int)sa, 0, (int)sb);
}
// This instruction reads its operand registers (bytes and scales) during its passes, not only
// at issue (measured: with the result registers overlapping A or a scale operand, or an operand
// register rewritten right after issue, scores came out wrong), which the compiler's register
// allocation does not model for it. So every operand is kept alive until an instruction that
// reads the product's result: the empty asm below takes the operand together with a value
// that a real vector instruction computed from that result (the compiler inserts the wait
// states of that read), so it can only sit after the product has finished, and no operand
// register is reused before.
__device__ __forceinline__ void hold(const i32x8& x, float after) {
  const i32x4 lo = __builtin_shufflevector(x, x, 0, 1, 2, 3);
  const i32x4 hi = __builtin_shufflevector(x, x, 4, 5, 6, 7);
  asm volatile("" ::"v"(lo), "v"(hi), "v"(after));
}
__device__ __forceinline__ void hold(uint32_t x, float after) {  // a scale operand
  asm volatile("" ::"v"(x), "v"(after));
}
template <int B>
struct IntC {  // a compile-time int as a value
  static constexpr int value = B;
};
// Wait until at most n tiles of NPT loads each are still in flight (n <= K, n uniform).
template <int NPT, int K>
__device__ __forceinline__ void wait_tiles(int n) {
  if constexpr (K == 0) {
    wait_vmem<0>();
  } else {
    if (n >= K) wait_vmem<K * NPT>();
    else wait_tiles<NPT, K - 1>(n);
  }
}
// LDS stages of the FP8 attention loop (2 to 4): tiles in flight ahead of the one computed
#ifndef RECAP_MX_STAGES
#define RECAP_MX_STAGES 2
#endif
constexpr int kMxStages = RECAP_MX_STAGES;
static_assert(kMxStages >= 2 && kMxStages <= 4, "2 to 4 LDS stages");

template <int D>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void attn_mx_kernel(
    MxParams p) {
  constexpr int TS = 66 * D;                  // packed tile bytes (codes + scales)
  constexpr int TB = (TS + 255) & ~255;       // LDS tile buffer stride
  constexpr int CH = D / 16, RPB = 256 / D;   // K row: 16-byte chunks; K rows per 256 bytes
  constexpr int LDK = D / 64;                 // code DMA instructions per wavefront per tile
  constexpr int SL = D / 32;                  // scale DMA lanes per wavefront per tile
  constexpr int NPT = 2 * (LDK + 1);          // DMA instructions per wavefront per tile
  constexpr int NS = kMxStages;
  __shared__ __align__(256) unsigned char kbuf[NS * TB];
  __shared__ __align__(256) unsigned char vbuf[NS * TB];
  __shared__ uint32_t kept_bits[2][kMaxBlocks / 32];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int n = lane & 31, half = lane >> 5;
  const int tile = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = tile / p.mq, qi = tile - bh * p.mq;
  const int b = bh / p.H, h = bh - b * p.H;
  const bool pair = p.block == 64;
  const int qrow = qi * 128 + wave * 32 + n;
  const int qc = min(qrow, p.N - 1);

  // Q^T operand bytes and scales (byte m of qsc = scale of dims 64 m + 32 half ..+31)
  i32x8 qf[D / 64];
  uint32_t qsc = 0;
  {
    const uint8_t* src = p.q8 + ((int64_t)bh * p.N + qc) * D + half * 16;
    const uint8_t* ssrc = p.qs + ((int64_t)bh * p.N + qc) * (D / 32) + half;
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      qf[m] = join(*reinterpret_cast<const i32x4*>(src + 64 * m),
                   *reinterpret_cast<const i32x4*>(src + 64 * m + 32));
      qsc |= (uint32_t)ssrc[2 * m] << (8 * m);
    }
    // consume the fragments here so the compiler's waits for these loads sit before the loop
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      const i32x4 lo = __builtin_shufflevector(qf[m], qf[m], 0, 1, 2, 3);
      const i32x4 hi = __builtin_shufflevector(qf[m], qf[m], 4, 5, 6, 7);
      asm volatile("" ::"v"(lo), "v"(hi));
    }
    asm volatile("" ::"v"(qsc));
  }

  // kept bitmaps (pairs) and the block sequence
  const int nb = pair ? 2 : 1;
  const int words = (p.M + 31) / 32;
  for (int w = threadIdx.x; w < nb * words; w += 256) kept_bits[w / words][w % words] = 0u;
  __syncthreads();
  for (int lb = 0; lb < nb; ++lb) {
    const int blk = pair ? 2 * qi + lb : qi;
    if (blk >= p.M) break;
    const int64_t row = (int64_t)bh * p.M + blk;
    const int cnt = min(max(p.count[row], 0), p.M);
    for (int c = threadIdx.x; c < cnt; c += 256) {
      const int jj = min(max(p.idx[row * p.M + c], 0), p.M - 1);
      atomicOr(&kept_bits[lb][jj >> 5], 1u << (jj & 31));
    }
  }
  __syncthreads();
  const uint32_t* own = kept_bits[pair ? (wave >> 1) : 0];
  UnionSeq seq{kept_bits[0], kept_bits[pair ? 1 : 0], p.M, 0};

  // per-lane DMA source offsets inside a packed tile
  uint32_t koff[LDK], voff[LDK];
#pragma unroll
  for (int it = 0; it < LDK; ++it) {
    const int x = wave * LDK + it;
    const int kr = x * (1024 / D) + lane / CH;
    koff[it] = opaque((uint32_t)(kr * D + (((lane % CH) ^ ((kr / RPB) & (CH - 1))) << 4)));
    const int vr = x * 16 + (lane >> 2);
    voff[it] = opaque((uint32_t)(vr * 64 + (((lane & 3) ^ ((vr >> 2) & 3)) << 4)));
  }
  const uint32_t soff = opaque((uint32_t)(64 * D + (wave * SL + lane) * 16));  // scale lanes
  const uint32_t kb0 = lds_base(kbuf), vb0 = lds_base(vbuf);

  // per-lane LDS read addresses in stage 0 (stage 1, keys 32..63 and channel groups are
  // immediate offsets): K row n, chunks (4m + half) ^ ksw and (4m + 2 + half) ^ ksw; V row n,
  // chunks 2 half ^ vsw and (2 half + 1) ^ vsw; the lane's K and V scale words
  const int ksw = (n / RPB) & (CH - 1), vsw = (n >> 2) & 3;
  uint32_t kra[D / 64][2];
#pragma unroll
  for (int m = 0; m < D / 64; ++m) {
    kra[m][0] = opaque(kb0 + (uint32_t)(n * D + (((4 * m + half) ^ ksw) << 4)));
    kra[m][1] = opaque(kb0 + (uint32_t)(n * D + (((4 * m + 2 + half) ^ ksw) << 4)));
  }
  const uint32_t vra0 = opaque(vb0 + (uint32_t)(n * 64 + (((2 * half) ^ vsw) << 4)));
  const uint32_t vra1 = opaque(vb0 + (uint32_t)(n * 64 + (((2 * half + 1) ^ vsw) << 4)));
  constexpr int SCW = D / 32;  // scale bytes per operand row (one word at D = 128)
  const uint32_t ksa = opaque(kb0 + (uint32_t)(64 * D + (half * 32 + n) * SCW));
  const uint32_t vsa = opaque(vb0 + (uint32_t)(64 * D + (half * 32 + n) * SCW));

  f32x16 o[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) o[dt] = f32x16{};
  // Row sums on the matrix cores: an all-ones A operand (E4M3 1.0, scale 2^0) times P^T gives
  // every register of a lane its query's sum of the rounded, scaled weights of the tile.
  // (both held in registers for the whole loop: a constant would be rematerialised into
  // registers the compiler may rewrite while the product still reads them)
  f32x16 lsum = {};
  i32x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (int)opaque(0x38383838u);
  const uint32_t one_scale = opaque(127u);
  float m_run = -INFINITY;

  const uint8_t* khead = p.kt + (int64_t)bh * p.ntile * TS;
  const uint8_t* vhead = p.vt + (int64_t)bh * p.ntile * TS;
  auto issue = [&](TileCur t, int buf) {
    const int tix = (t.j * p.block) / 64 + t.st;
    const uint8_t* ks = khead + (int64_t)tix * TS;
    const uint8_t* vs = vhead + (int64_t)tix * TS;
#pragma unroll
    for (int it = 0; it < LDK; ++it) {
      const int x = wave * LDK + it;
      load_lds16(ks, koff[it], kb0 + buf * TB + x * 1024);
      load_lds16(vs, voff[it], vb0 + buf * TB + x * 1024);
    }
    if (lane < SL) {
      load_lds16(ks, soff, kb0 + buf * TB + 64 * D + wave * SL * 16);
      load_lds16(vs, soff, vb0 + buf * TB + 64 * D + wave * SL * 16);
    }
  };

  // Operands of the last tile's O^T and row-sum products. They are kept alive until the next
  // step has passed its barrier, where a compiler-generated copy of each product's result is
  // made (see hold()): the products drain while the wavefront waits at the barrier.
  i32x8 pend_va[D / 32], pend_pb;
  uint32_t pend_vss[D / 32], pend_psc = 0;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    pend_va[dt] = i32x8{};
    pend_vss[dt] = 0;
  }
  pend_pb = i32x8{};
  auto retire = [&]() __attribute__((always_inline)) {
    {
      float done = lsum[15];
      asm volatile("" : "+v"(done));
      hold(ones, done);
      hold(one_scale, done);
      hold(pend_pb, done);
      hold(pend_psc, done);
    }
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      float done = o[dt][15];
      asm volatile("" : "+v"(done));
      hold(pend_va[dt], done);
      hold(pend_vss[dt], done);
      hold(pend_pb, done);
      hold(pend_psc, done);
    }
  };

  // one tile from LDS stage B (a compile-time constant, so its offset is an immediate)
  auto compute = [&](auto stage, TileCur cur) __attribute__((always_inline)) {
    constexpr uint32_t SO = decltype(stage)::value * TB;
    const int key0 = cur.j * p.block + cur.st * 64;
    // S^T = K Q^T: s0 = keys 0..31 of the tile, s1 = keys 32..63; register r of lane half h
    // holds key 8 (r / 4) + 4 h + r % 4 (+32 in s1)
    const uint32_t ksc = D == 128 ? lds_read_u32(ksa + SO) : lds_read_u16(ksa + SO);
    i32x8 ka[2][D / 64];  // K operands, all in distinct registers until the scores are read
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      ka[0][m] = join(lds_read16i(kra[m][0] + SO), lds_read16i(kra[m][1] + SO));
      ka[1][m] = join(lds_read16i(kra[m][0] + SO + 32 * D), lds_read16i(kra[m][1] + SO + 32 * D));
    }
    uint32_t kss[2][D / 64], qss[D / 64];  // per-lane scale operands, held like the bytes
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      kss[0][m] = ksc >> (8 * m);
      kss[1][m] = ksc >> (8 * (D / 64 + m));
      qss[m] = qsc >> (8 * m);
    }
    f32x16 s0 = {}, s1 = {};
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      s0 = mx_mfma(ka[0][m], qf[m], s0, kss[0][m], qss[m]);
      s1 = mx_mfma(ka[1][m], qf[m], s1, kss[1][m], qss[m]);
    }
    if (key0 + 64 > p.N) {  // last, partial tile
      asm volatile("" ::: "memory");
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int kr = 8 * (r >> 2) + 4 * half + (r & 3);
        if (key0 + kr >= p.N) s0[r] = -INFINITY;
        if (key0 + 32 + kr >= p.N) s1[r] = -INFINITY;
      }
    }
    // online softmax (base 2, lazy rescale by more than kLazy); the per-block maxima of the
    // scores (keys 0..31 and 32..63) also set the weights' two MX exponents (fmaxf first: a
    // compiler-generated read, so the products have finished before the inline-asm max3
    // reads their results)
    float lm0 = fmaxf(s0[0], s0[1]), lm1 = fmaxf(s1[0], s1[1]);
#pragma unroll
    for (int r = 2; r < 16; r += 2) {
      lm0 = max3(lm0, s0[r], s0[r + 1]);
      lm1 = max3(lm1, s1[r], s1[r + 1]);
    }
#pragma unroll
    for (int m = 0; m < D / 64; ++m) {
      hold(ka[0][m], lm0);
      hold(ka[1][m], lm1);
      hold(kss[0][m], lm0);
      hold(kss[1][m], lm1);
      hold(qss[m], lm0);
      hold(qss[m], lm1);
    }
    const float c0 = cross_half_max(lm0), c1 = cross_half_max(lm1);
    const float mt = fmaxf(c0, c1) * p.scale_log2;
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kLazy) != 0) {
      const float mn = fmaxf(m_run, mt);
      const float alpha = __builtin_amdgcn_exp2f(m_run - mn);
      m_run = mn;
      lsum *= alpha;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) o[dt] *= alpha;
    }
    // block exponents: the block's largest weight 2^(x - e) lands in [128, 256); an all-masked
    // block (x = -inf) gets the smallest, -127
    const float f0 = __builtin_floorf(fmaxf(c0 * p.scale_log2 - m_run, -120.f)) - 7.f;
    const float f1 = __builtin_floorf(fmaxf(c1 * p.scale_log2 - m_run, -120.f)) - 7.f;
    const float neg0 = -(m_run + f0), neg1 = -(m_run + f1);
    i32x8 pb;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      float x[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        x[i] = w < 4 ? __builtin_amdgcn_exp2f(__builtin_fmaf(s0[4 * w + i], p.scale_log2, neg0))
                     : __builtin_amdgcn_exp2f(__builtin_fmaf(s1[4 * (w - 4) + i], p.scale_log2, neg1));
      // the first conversion keeps the upper half of its old value, which the second one
      // overwrites: pass a dead register rather than a zero that would need a move
      const int v = __builtin_amdgcn_cvt_pk_fp8_f32(x[0], x[1], __float_as_int(x[0]), false);
      pb[w] = __builtin_amdgcn_cvt_pk_fp8_f32(x[2], x[3], v, true);
    }
    // O^T += V^T P^T, row sums += 1 P^T
    const uint32_t vsc = D == 128 ? lds_read_u32(vsa + SO) : lds_read_u16(vsa + SO);
    const uint32_t psc = (uint32_t)((int)(half == 0 ? f0 : f1) + 127);  // lane half b: block b
    i32x8 va[D / 32];  // V operands, distinct registers until the products are read
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt)
      va[dt] = join(lds_read16i(vra0 + SO + 2048 * dt), lds_read16i(vra1 + SO + 2048 * dt));
    uint32_t vss[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) vss[dt] = vsc >> (8 * dt);
    lsum = mx_mfma(ones, pb, lsum, one_scale, psc);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) o[dt] = mx_mfma(va[dt], pb, o[dt], vss[dt], psc);
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) {
      pend_va[dt] = va[dt];
      pend_vss[dt] = vss[dt];
    }
    pend_pb = pb;
    pend_psc = psc;
  };

  // NS-stage pipeline, one barrier per tile: at the step that computes tile t (stage t mod NS)
  // the tiles up to t + NS - 2 are in flight, and tile t + NS - 1 is loaded into the stage
  // that tile t - 1 used, which every wavefront has left once it passes this step's barrier.
  TileCur q[NS];  // q[0]: the tile of this step; q[1 .. NS - 2]: issued after it
  q[0] = TileCur{seq.first(), 0};
  if (q[0].j >= 0) {
    issue(q[0], 0);
#pragma unroll
    for (int i = 1; i < NS - 1; ++i) {
      q[i] = advance(q[i - 1], seq, p.block, p.N);
      if (q[i].j >= 0) issue(q[i], i);
    }
    // one tile from stage B; false once the last tile is done
    auto step = [&](auto stage) __attribute__((always_inline)) -> bool {
      constexpr int B = decltype(stage)::value;
      int inflight = 0;
#pragma unroll
      for (int i = 1; i < NS - 1; ++i) inflight += q[i].j >= 0 ? 1 : 0;
      wait_tiles<NPT, NS - 2>(inflight);  // this wavefront's loads of tile q[0] have landed
      lds_barrier();                      // ... every wavefront's; all are done with stage B - 1
      q[NS - 1] = advance(q[NS - 2], seq, p.block, p.N);
      if (q[NS - 1].j >= 0) issue(q[NS - 1], (B + NS - 1) % NS);
      retire();  // the previous tile's products have drained while this wavefront waited above
      if ((own[q[0].j >> 5] >> (q[0].j & 31)) & 1u) compute(stage, q[0]);
      if (q[1].j < 0) return false;
#pragma unroll
      for (int i = 0; i < NS - 1; ++i) q[i] = q[i + 1];
      return true;
    };
    while (step(IntC<0>{}) && step(IntC<1 % NS>{}) && (NS < 3 || step(IntC<2 % NS>{})) &&
           (NS < 4 || step(IntC<3 % NS>{}))) {
    }
    retire();
  }


  // epilogue: O = O^T / l (+ c_h R), bf16 in the q layout; optional log-sum-exp
  const float lt = lsum[0];  // the query's whole row sum, in both lane halves
  const float inv = lt > 0.f ? 1.0f / lt : 0.f;
  if (qrow >= p.N) return;
  if (p.lse_out != nullptr && half == 0)
    p.lse_out[(int64_t)bh * p.N + qrow] = lt > 0.f ? (m_run + log2f(lt)) * kLn2 : -INFINITY;
  const int64_t orow = b * p.st.b + h * p.st.h + (int64_t)qrow * p.st.n;
  const bool has_res = p.res != nullptr;
  const float c = p.res_scale.v[h];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int d0 = dt * 32 + g * 8 + half * 4;
      f32x4 v;
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = o[dt][g * 4 + e] * inv;
      if (has_res) {
        const bf16x4 r4 = *reinterpret_cast<const bf16x4*>(p.res + orow + d0);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[e] += c * (float)r4[e];
      }
      bf16x4 w;
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = (bf16_t)v[e];
      *reinterpret_cast<bf16x4*>(p.out + orow + d0) = w;
    }
  }
}

// ---- launchers -----------------------------------------------------------------------------
static int grid_for(int64_t total) {
  return (int)(total < 65536LL * 256 ? (total + 255) / 256 : 65536);
}

hipError_t launch_mx_rows(const bf16_t* x, Strides st, int B, int H, int N, int D,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t total = (int64_t)B * H * N * (D / 32);
  if (D == 128)
    mx_rows_kernel<128><<<grid_for(total), 256, 0, stream>>>(x, st, H, N, total, codes, scales);
  else
    mx_rows_kernel<64><<<grid_for(total), 256, 0, stream>>>(x, st, H, N, total, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_cols(const bf16_t* x, Strides st, int B, int H, int N, int D,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream) {
  const int64_t total = (int64_t)B * H * ((N + 31) / 32) * D;
  if (D == 128)
    mx_cols_kernel<128><<<grid_for(total), 256, 0, stream>>>(x, st, H, N, total, codes, scales);
  else
    mx_cols_kernel<64><<<grid_for(total), 256, 0, stream>>>(x, st, H, N, total, codes, scales);
  return hipGetLastError();
}

hipError_t launch_mx_kv_tiles(const bf16_t* k, const bf16_t* v, Strides st, int B, int H, int N,
                              int D, int ntile, uint8_t* kt, uint8_t* vt, hipStream_t stream) {
  const int64_t total = (int64_t)B * H * ntile * 64 * (D / 32);
  const int vgrid = B * H * ntile;
  if (D == 128) {
    mx_k_tiles_kernel<128><<<grid_for(total), 256, 0, stream>>>(k, st, H, N, ntile, total, kt);
    mx_v_tiles_kernel<128><<<vgrid, 256, 0, stream>>>(v, st, H, N, ntile, vt);
  } else {
    mx_k_tiles_kernel<64><<<grid_for(total), 256, 0, stream>>>(k, st, H, N, ntile, total, kt);
    mx_v_tiles_kernel<64><<<vgrid, 256, 0, stream>>>(v, st, H, N, ntile, vt);
  }
  return hipGetLastError();
}

hipError_t launch_attention_mx(MxParams p, int B, int D, hipStream_t stream) {
  p.mq = p.block == 64 ? (p.M + 1) / 2 : p.M;
  const int grid = B * p.H * p.mq;
  if (D == 128)
    attn_mx_kernel<128><<<grid, 256, 0, stream>>>(p);
  else
    attn_mx_kernel<64><<<grid, 256, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace recap
