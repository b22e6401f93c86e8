// Mask prediction on gfx950: block mean pooling, block-pair softmax scores, top-p selection.
//
// RECAP (paperpeel.com/paper/2610.26244) Sec. 3.2 uses block means as coarse estimates of
// the attention each block receives; the first abstract on the RECAP page at
// thelatestinai.com describes online top-p mask prediction with per-head thresholds, and
// CalibAtt (thelatestinai.com/papers/2603.05503) Fig. 5 thresholds the top key blocks of
// every query block. Pooling and top-p are bound by HBM bandwidth and latency; the scores are
// a small fp32 contraction done on the fp32 matrix cores.
#include <atomic>
#include <type_traits>

#include "common.h"

namespace recap {

// ------------------------------------------------------------------------------------------
// Pooling: one wavefront per (tensor, b, h, block). Lanes stride over the block's rows with
// 16-byte loads (CH lanes cover one row, G rows per load), all of a lane's loads issued before
// the first is summed, and non-temporal (Q and K are read once here: 8-9% faster than cached
// loads issued four at a time); then fp32 sums in row order, a reduction across the row groups
// with lane shuffles, and the fp32 mean row.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void pool_kernel(const bf16_t* __restrict__ q,
                                                   const bf16_t* __restrict__ k, Strides st,
                                                   int H, int N, int block, int M, int rows,
                                                   float* __restrict__ qbar,
                                                   float* __restrict__ kbar) {
  constexpr int CH = D / 8;   // 16-byte chunks per row
  constexpr int G = 64 / CH;  // rows loaded per wavefront instruction
  const int lane = threadIdx.x & 63;
  const int task = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (task >= 2 * rows) return;
  const int which = task >= rows;
  const int row = task - which * rows;
  const int j = row % M;
  const int bh = row / M;
  const int b = bh / H, h = bh - b * H;
  const bf16_t* src = (which ? k : q) + b * st.b + h * st.h;
  const int t0 = j * block;
  const int t1 = min(N, t0 + block);
  const int c = lane % CH, g = lane / CH;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  // NIT loads per lane cover the block (NIT * G >= t1 - t0); past the block's last row the
  // address is clamped to it and the value left out of the sum
  auto pool_rows = [&](auto nit) {
    constexpr int NIT = decltype(nit)::value;
    bf16x8 xs[NIT];
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      const int t = min(t0 + g + it * G, t1 - 1);
      xs[it] = __builtin_nontemporal_load(
          reinterpret_cast<const bf16x8*>(src + (int64_t)t * st.n + c * 8));
    }
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      if (t0 + g + it * G < t1) {
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] += (float)xs[it][e];
      }
    }
  };
  if (t1 - t0 <= 64) pool_rows(std::integral_constant<int, 64 / G>{});
  else pool_rows(std::integral_constant<int, 128 / G>{});  // block <= 128 (validated)
#pragma unroll
  for (int off = CH; off < 64; off <<= 1) {
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] += __shfl_xor(acc[e], off);
  }
  if (g == 0) {
    const float n = (float)(t1 - t0);
    float* dst = (which ? kbar : qbar) + (int64_t)row * D + c * 8;
    f32x4 lo, hi;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      lo[e] = acc[e] / n;
      hi[e] = acc[e + 4] / n;
    }
    *reinterpret_cast<f32x4*>(dst) = lo;
    *reinterpret_cast<f32x4*>(dst + 4) = hi;
  }
}

// ------------------------------------------------------------------------------------------
// Scores: work-group = (b*h, tile of 32 query blocks); its 4 wavefronts split the key-block
// tiles. Each 32x32 tile is computed transposed, S^T = K̄ Q̄^T, with the fp32 MFMA 32x32x2:
// lane (n, half) then owns query block n and 16 key blocks of the tile, so the row softmax
// runs in-lane. Pass 1 gathers the per-row max and sum (online, combined across halves and
// wavefronts); pass 2 recomputes the identical tiles and writes exp2(x - m) / l.
// The contraction over D is split as D index = half * D/2 + s, s = 0..D/2-1, identically
// for both operands.
// ------------------------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ f32x16 score_tile(const float* __restrict__ kb, int key0, int M,
                                             const float (&qv)[D / 2], int m_lane, int half) {
  const int key = min(key0 + m_lane, M - 1);
  const float* src = kb + (int64_t)key * D + half * (D / 2);
  float kv[D / 2];
#pragma unroll
  for (int s = 0; s < D / 2; s += 4) {
    const f32x4 x = *reinterpret_cast<const f32x4*>(src + s);
    kv[s] = x[0];
    kv[s + 1] = x[1];
    kv[s + 2] = x[2];
    kv[s + 3] = x[3];
  }
  f32x16 a0 = {}, a1 = {};
#pragma unroll
  for (int s = 0; s < D / 2; s += 2) {
    a0 = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[s], qv[s], a0, 0, 0, 0);
    a1 = __builtin_amdgcn_mfma_f32_32x32x2f32(kv[s + 1], qv[s + 1], a1, 0, 0, 0);
  }
  return a0 + a1;
}

template <int D>
__global__ __launch_bounds__(256) void score_kernel(const float* __restrict__ qbar,
                                                    const float* __restrict__ kbar, int M,
                                                    float scale_log2, float* __restrict__ probs) {
  __shared__ float red_m[4][32];
  __shared__ float red_l[4][32];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 31, half = lane >> 5;
  const int nqt = (M + 31) >> 5;
  const int bh = blockIdx.x / nqt, qt = blockIdx.x - bh * nqt;
  const float* qb = qbar + (int64_t)bh * M * D;
  const float* kb = kbar + (int64_t)bh * M * D;
  const int qrow = qt * 32 + n;
  float qv[D / 2];
  {
    const float* src = qb + (int64_t)min(qrow, M - 1) * D + half * (D / 2);
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + s);
      qv[s] = x[0];
      qv[s + 1] = x[1];
      qv[s + 2] = x[2];
      qv[s + 3] = x[3];
    }
  }
  const int nkt = (M + 31) >> 5;
  float m = -INFINITY, l = 0.f;
  for (int kt = wave; kt < nkt; kt += 4) {
    const f32x16 acc = score_tile<D>(kb, kt * 32, M, qv, n, half);
    float x[16];
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      x[r] = key < M ? acc[r] * scale_log2 : -INFINITY;
      mx = fmaxf(mx, x[r]);
    }
    const float mn = fmaxf(m, mx);
    float add = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) add += __builtin_amdgcn_exp2f(x[r] - mn);
    l = l * __builtin_amdgcn_exp2f(m - mn) + add;
    m = mn;
  }
  // combine the two halves of the wavefront, then the four wavefronts
  {
    const float mo = __shfl_xor(m, 32), lo = __shfl_xor(l, 32);
    const float mn = fmaxf(m, mo);
    l = (m == -INFINITY ? 0.f : l * __builtin_amdgcn_exp2f(m - mn)) +
        (mo == -INFINITY ? 0.f : lo * __builtin_amdgcn_exp2f(mo - mn));
    m = mn;
  }
  if (half == 0) {
    red_m[wave][n] = m;
    red_l[wave][n] = l;
  }
  __syncthreads();
  float mrow = -INFINITY;
#pragma unroll
  for (int w = 0; w < 4; ++w) mrow = fmaxf(mrow, red_m[w][n]);
  float lrow = 0.f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float mw = red_m[w][n];
    if (mw != -INFINITY) lrow += red_l[w][n] * __builtin_amdgcn_exp2f(mw - mrow);
  }
  const float inv = 1.0f / lrow;
  // Lanes past the last query block stay active: every lane also supplies key rows to the
  // collective MFMA operands, so only their stores are skipped.
  const bool qvalid = qrow < M;
  float* prow = probs + ((int64_t)bh * M + min(qrow, M - 1)) * M;
  for (int kt = wave; kt < nkt; kt += 4) {
    const f32x16 acc = score_tile<D>(kb, kt * 32, M, qv, n, half);
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int key = kt * 32 + (r >> 2) * 8 + half * 4 + (r & 3);
      if (qvalid && key < M) prow[key] = __builtin_amdgcn_exp2f(acc[r] * scale_log2 - mrow) * inv;
    }
  }
}

// Wavefront-wide reductions without LDS: DPP steps inside each row of 16 lanes (xor 1, xor 2,
// rotate by 4 and by 8 within the row), then the four row results combined from lanes 0, 16,
// 32 and 48. The result is uniform across the wavefront.
template <class Op>
__device__ __forceinline__ uint32_t row_reduce_u(uint32_t x, Op op) {
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0xb1, 0xf, 0xf, false));   // quad [1,0,3,2]
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x4e, 0xf, 0xf, false));   // quad [2,3,0,1]
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x124, 0xf, 0xf, false));  // row_ror:4
  x = op(x, (uint32_t)__builtin_amdgcn_mov_dpp((int)x, 0x128, 0xf, 0xf, false));  // row_ror:8
  return x;
}
__device__ __forceinline__ uint32_t wave_min_u(uint32_t x) {
  auto mn = [](uint32_t a, uint32_t b) { return a < b ? a : b; };
  x = row_reduce_u(x, mn);
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return mn(mn(a, b), mn(c, d));
}
__device__ __forceinline__ uint32_t wave_max_u(uint32_t x) {
  auto mx = [](uint32_t a, uint32_t b) { return a > b ? a : b; };
  x = row_reduce_u(x, mx);
  const uint32_t a = __builtin_amdgcn_readlane(x, 0), b = __builtin_amdgcn_readlane(x, 16);
  const uint32_t c = __builtin_amdgcn_readlane(x, 32), d = __builtin_amdgcn_readlane(x, 48);
  return mx(mx(a, b), mx(c, d));
}
__device__ __forceinline__ float wave_sum_f(float x) {
  auto add = [](uint32_t a, uint32_t b) { return __float_as_uint(__uint_as_float(a) + __uint_as_float(b)); };
  const uint32_t r = row_reduce_u(__float_as_uint(x), add);
  const float a = __uint_as_float(__builtin_amdgcn_readlane(r, 0));
  const float b = __uint_as_float(__builtin_amdgcn_readlane(r, 16));
  const float c = __uint_as_float(__builtin_amdgcn_readlane(r, 32));
  const float d = __uint_as_float(__builtin_amdgcn_readlane(r, 48));
  return (a + b) + (c + d);
}

__device__ __forceinline__ float wave_max_f(float x) {
  auto mx = [](uint32_t a, uint32_t b) { return __float_as_uint(fmaxf(__uint_as_float(a), __uint_as_float(b))); };
  const uint32_t r = row_reduce_u(__float_as_uint(x), mx);
  const float a = __uint_as_float(__builtin_amdgcn_readlane(r, 0));
  const float b = __uint_as_float(__builtin_amdgcn_readlane(r, 16));
  const float c = __uint_as_float(__builtin_amdgcn_readlane(r, 32));
  const float d = __uint_as_float(__builtin_amdgcn_readlane(r, 48));
  return fmaxf(fmaxf(a, b), fmaxf(c, d));
}

// ------------------------------------------------------------------------------------------
// Scores in one pass for rows that fit in LDS: work-group = (b*h, strip of 16 query blocks).
// The strip's scaled logits are computed once into LDS with the fp32 MFMA 16x16x4, as
// S^T = K̄ Q̄^T so that lane l owns query block l % 16 and four consecutive key blocks of each
// 16-key tile (the contraction over D is split as D index = (l / 16) * D/4 + step, identically
// for both operands). Eight wavefronts share a strip: each multiplies every eighth key tile,
// then normalises two rows: row max and sum from LDS, and the normalised row written with
// consecutive lanes on consecutive key blocks.
// ------------------------------------------------------------------------------------------
constexpr int kStripRows = 16;
// Rows of up to kStripMaxM blocks run in one pass: 16 rows x 1268 fp32 of LDS (79.25 KB, two
// work-groups per CU) and up to kStripVals values per lane in registers
constexpr int kStripMaxM = 1264;
constexpr int kStripVals = 20;

__host__ __device__ constexpr int strip_stride(int M) { return ((M + 15) / 16) * 16 + 4; }
// wavefronts per strip work-group: 16 per CU with two work-groups, which the registers allow
constexpr int kStripWaves = 8;

// CAND: scores restricted to candidate lists (the reduced search of the GSRS abstract on the
// RECAP page at thelatestinai.com). The strip's logits are computed the same way; each row is
// then normalised over its candidates only, gathered from the LDS strip at the listed blocks,
// and written at the candidate positions.
template <int D, bool CAND>
__global__ __launch_bounds__(kStripWaves * 64) void score_strip_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar, int M,
                                                          float scale_log2,
                                                          const int32_t* __restrict__ ccount,
                                                          const int32_t* __restrict__ cidx,
                                                          float* __restrict__ probs) {
  extern __shared__ float srow[];  // [kStripRows][strip_stride(M)]
  constexpr int KS = D / 4;        // contraction steps; lane group g covers D indices [g*KS, ..)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int nst = (M + kStripRows - 1) / kStripRows;
  // strips of one head on one XCD, so that head's K̄ stays in that XCD's L2
  const int wg = xcd_remap(blockIdx.x, gridDim.x);
  const int bh = wg / nst, st = wg - bh * nst;
  const int stride = strip_stride(M);
  const float* qb = qbar + (int64_t)bh * M * D;
  const float* kb = kbar + (int64_t)bh * M * D;
  float qv[KS];
  {
    const float* src = qb + (int64_t)min(st * kStripRows + col, M - 1) * D + grp * KS;
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + s);
      qv[s] = x[0];
      qv[s + 1] = x[1];
      qv[s + 2] = x[2];
      qv[s + 3] = x[3];
    }
  }
  const int nkt = (M + 15) >> 4;
  // K̄ rows of a 16-key tile; the next tile's are loaded while this one is multiplied
  auto load_k = [&](int kt, float (&kv)[KS]) {
    const float* src = kb + (int64_t)min(kt * 16 + col, M - 1) * D + grp * KS;
#pragma unroll
    for (int s = 0; s < KS; s += 4) {
      const f32x4 x = *reinterpret_cast<const f32x4*>(src + s);
      kv[s] = x[0];
      kv[s + 1] = x[1];
      kv[s + 2] = x[2];
      kv[s + 3] = x[3];
    }
  };
  float kn[KS];
  if (wave < nkt) load_k(wave, kn);
  for (int kt = wave; kt < nkt; kt += kStripWaves) {
    float kv[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) kv[s] = kn[s];
    if (kt + kStripWaves < nkt) load_k(kt + kStripWaves, kn);
    f32x4 a0 = {}, a1 = {};
#pragma unroll
    for (int s = 0; s < KS; s += 2) {
      a0 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[s], qv[s], a0, 0, 0, 0);
      a1 = __builtin_amdgcn_mfma_f32_16x16x4f32(kv[s + 1], qv[s + 1], a1, 0, 0, 0);
    }
    // lane holds S^T[key = kt*16 + 4*grp + r][query = col], r = 0..3
    f32x4 x;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int key = kt * 16 + grp * 4 + r;
      x[r] = key < M ? (a0[r] + a1[r]) * scale_log2 : -INFINITY;
    }
    *reinterpret_cast<f32x4*>(srow + col * stride + kt * 16 + grp * 4) = x;
  }
  __syncthreads();
  // each wavefront normalises kStripRows / kStripWaves rows; a row (M <= 64 * kStripVals) sits in registers
  for (int rr = 0; rr < kStripRows / kStripWaves; ++rr) {
    const int r = wave * (kStripRows / kStripWaves) + rr;
    const int qrow = st * kStripRows + r;
    if (qrow >= M) break;  // uniform per wavefront
    const float* x = srow + r * stride;
    const int64_t grow = (int64_t)bh * M + qrow;
    const int n = CAND ? min(max(ccount[grow], 0), M) : M;  // values of the row
    if (CAND && n == 0) continue;  // no candidates: nothing to write (uniform per wavefront)
    const int32_t* crow = CAND ? cidx + grow * M : nullptr;
    float e[kStripVals];
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < kStripVals; ++i) {
      const int j = i * 64 + lane;
      if (CAND) e[i] = j < n ? x[min(max(crow[j], 0), M - 1)] : -INFINITY;
      else e[i] = j < M ? x[j] : -INFINITY;
      mx = fmaxf(mx, e[i]);
    }
    mx = wave_max_f(mx);
    float l = 0.f;
#pragma unroll
    for (int i = 0; i < kStripVals; ++i) {
      e[i] = __builtin_amdgcn_exp2f(e[i] - mx);  // 0 past M
      l += e[i];
    }
    const float inv = 1.0f / wave_sum_f(l);
    float* prow = probs + ((int64_t)bh * M + qrow) * M;
#pragma unroll
    for (int i = 0; i < kStripVals; ++i) {
      const int j = i * 64 + lane;
      if (j < n) prow[j] = e[i] * inv;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Top-p: one work-group of 256 threads per query-block row. Keys (orderable probability bits
// << 32 | ~index) are bitonic-sorted descending in LDS, which orders probabilities descending
// and equal values by lower index first. Running mass: fp64 block scan over the sorted
// values; k* = first prefix reaching p (inclusive), M when p >= 1 or none reaches it. Kept
// blocks are flagged by index, then compacted in ascending index order with a second scan.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t orderable(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float from_orderable(uint32_t u) {
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

// Inclusive block scan of one value per thread (256 threads); returns the exclusive prefix.
template <typename T>
__device__ __forceinline__ T block_exclusive_scan(T v, T* wave_tot, T& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const T y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  T base = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const T t = wave_tot[w];
    if (w < wave) base += t;
    all += t;
  }
  total = all;
  __syncthreads();
  return base + x - v;
}

__global__ __launch_bounds__(256) void topp_kernel(const float* __restrict__ probs, int H, int M,
                                                   int P, HeadScalars top_p,
                                                   const int32_t* __restrict__ ccount,
                                                   const int32_t* __restrict__ cidx,
                                                   int32_t* __restrict__ count,
                                                   int32_t* __restrict__ idx,
                                                   uint8_t* __restrict__ mask,
                                                   float* __restrict__ mass) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint64_t* keys = reinterpret_cast<uint64_t*>(smem);  // P entries
  uint8_t* flag = smem + (size_t)P * 8;                 // P entries
  __shared__ double wtot_d[4];
  __shared__ int wtot_i[4];
  __shared__ int kstar_s;
  __shared__ double mass_s;

  const int tid = threadIdx.x;
  const int64_t row = blockIdx.x;
  const int h = (int)((row / M) % H);
  const float p = top_p.v[h];
  const float* pr = probs + row * M;
  // with candidate lists the row is the first n positions, position r standing for block
  // cidx[r] (ascending); otherwise position = block
  const int n = ccount != nullptr ? min(max(ccount[row], 0), M) : M;
  const int32_t* crow = cidx != nullptr ? cidx + row * M : nullptr;
  auto block_of = [&](int pos) { return crow != nullptr ? min(max(crow[pos], 0), M - 1) : pos; };

  for (int t = tid; t < P; t += 256) {
    keys[t] = t < n ? ((uint64_t)orderable(pr[t]) << 32) | (uint64_t)(0xffffffffu - (uint32_t)t)
                    : 0ull;
    flag[t] = 0;
  }
  if (tid == 0) kstar_s = n;
  __syncthreads();

  for (int kk = 2; kk <= P; kk <<= 1) {
    for (int j = kk >> 1; j > 0; j >>= 1) {
      for (int i = tid; i < (P >> 1); i += 256) {
        const int a = ((i & ~(j - 1)) << 1) | (i & (j - 1));
        const int bb = a + j;
        const uint64_t x = keys[a], y = keys[bb];
        const bool desc = (a & kk) == 0;
        if ((x < y) == desc) {
          keys[a] = y;
          keys[bb] = x;
        }
      }
      __syncthreads();
    }
  }

  // fp64 running mass over the sorted values: each thread owns E consecutive positions.
  const int E = (P + 255) / 256;
  const int lo = tid * E;
  double local = 0.0;
  for (int e = 0; e < E; ++e) {
    const int pos = lo + e;
    if (pos < n) local += (double)from_orderable((uint32_t)(keys[pos] >> 32));
  }
  double total;
  const double base = block_exclusive_scan<double>(local, wtot_d, total);
  if (p < 1.0f) {
    double c = base;
    for (int e = 0; e < E; ++e) {
      const int pos = lo + e;
      if (pos >= n) break;
      c += (double)from_orderable((uint32_t)(keys[pos] >> 32));
      if (c >= (double)p) {
        atomicMin(&kstar_s, pos + 1);
        break;
      }
    }
  }
  __syncthreads();
  const int kstar = kstar_s;  // n when p >= 1 or when no prefix reaches p
  if (kstar == n) {
    if (tid == 0) mass_s = total;
  } else if (kstar - 1 >= lo && kstar - 1 < lo + E) {
    // the owner of position k*-1 recomputes the prefix it crossed p with
    double c = base;
    for (int pos = lo; pos < kstar; ++pos) c += (double)from_orderable((uint32_t)(keys[pos] >> 32));
    mass_s = c;
  }
  for (int pos = tid; pos < kstar; pos += 256) {
    const uint32_t j = 0xffffffffu - (uint32_t)(keys[pos] & 0xffffffffull);
    flag[j] = 1;
  }
  __syncthreads();

  // ascending compaction of the flagged positions (ascending blocks)
  int cnt = 0;
  for (int e = 0; e < E; ++e) {
    const int jj = lo + e;
    if (jj < n) cnt += flag[jj];
  }
  int tot_i;
  int off = block_exclusive_scan<int>(cnt, wtot_i, tot_i);
  int32_t* out_idx = idx + row * M;
  for (int e = 0; e < E; ++e) {
    const int jj = lo + e;
    if (jj < n && flag[jj]) out_idx[off++] = block_of(jj);
  }
  if (mask != nullptr) {
    uint8_t* mrow = mask + row * M;
    if (crow == nullptr) {
      for (int jj = tid; jj < M; jj += 256) mrow[jj] = flag[jj];
    } else {  // zeros everywhere, then ones at the kept blocks, ordered by a fence + barrier
      for (int jj = tid; jj < M; jj += 256) mrow[jj] = 0;
      __threadfence_block();
      __syncthreads();
      for (int jj = tid; jj < n; jj += 256)
        if (flag[jj]) mrow[block_of(jj)] = 1;
    }
  }
  if (tid == 0) {
    count[row] = kstar;
    if (mass != nullptr) mass[row] = (float)mass_s;
  }
}

// ------------------------------------------------------------------------------------------
// Top-p, one wavefront per row (rows of up to 64 * VPL blocks). The row stays in registers
// (lane l holds blocks l, l+64, ...). Probabilities are non-negative, so their fp32 bit
// patterns order like their values; a search over bit patterns finds the k*-th largest
// value v* = the largest value t with mass(>= t) >= p (mass accumulated in fp64). Every block
// above v* is kept; blocks equal to v* are taken in ascending index order until the running
// mass reaches p. This is the same set as sorting by (probability desc, index asc) and
// keeping the shortest prefix whose mass reaches p. No LDS, no barriers.
// The search keeps a bracket [lo, hi) with mass(>= lo) >= p > mass(>= hi), shrunk to the
// smallest and largest value inside it and split between them, so it ends once a single
// distinct value remains (about log2 M steps). Each mass test is first made in fp32: with
// n additions on any path the fp32 sum is within n * 2^-24 * total of the exact sum, and the
// fp64 sum is evaluated only when the fp32 one lies that close to p, so every decision is the
// one the fp64 sum gives.
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Rows of 16 or 20 values per lane (up to 1280 blocks: the 720p and HunyuanVideo rows) run at
// six wavefronts per SIMD instead of the four their default register allocation gives (one
// register is held in scratch across the threshold search: one store and one load per row);
// longer rows would spill inside the search, shorter ones reach that occupancy anyway.
__host__ __device__ constexpr int topp_min_waves(int vpl) { return vpl == 16 || vpl == 20 ? 6 : 1; }

template <int VPL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(topp_min_waves(VPL)))) void topp_wave_kernel(const float* __restrict__ probs, int H,
                                                        int M, int rows, HeadScalars top_p,
                                                        const int32_t* __restrict__ ccount,
                                                        const int32_t* __restrict__ cidx,
                                                        int32_t* __restrict__ count,
                                                        int32_t* __restrict__ idx,
                                                        uint8_t* __restrict__ mask,
                                                        float* __restrict__ mass) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // the whole wavefront
  const int h = (row / M) % H;
  const float p = top_p.v[h];
  const float* pr = probs + (int64_t)row * M;
  // with candidate lists the row is the first n positions, position r standing for block
  // cidx[r] (ascending); otherwise position = block
  const int n = ccount != nullptr ? min(max(ccount[row], 0), M) : M;
  const int32_t* crow = cidx != nullptr ? cidx + (int64_t)row * M : nullptr;
  // slots past n hold value 0: they add no mass, and the selection below never takes them
  uint32_t u[VPL];
  float val[VPL];
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const int j = i * 64 + lane;
    const float x = j < n ? pr[j] : 0.f;
    val[i] = x > 0.f ? x : 0.f;  // probabilities are >= 0; -0 and NaN map to 0
    u[i] = __float_as_uint(val[i]);
  }
  auto mass_at_least = [&](uint32_t t) {
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      if (u[i] >= t) acc += (double)val[i];
    return wave_sum(acc);
  };
  auto valid = [&](int i) { return i * 64 + lane < n; };

  bool kept[VPL];
  double kmass;  // mass of the kept set (output only)
  // the row total in fp32. An fp32 sum here (VPL terms per lane, then six reduction levels)
  // is within (VPL + 6) * 2^-24 * total of its exact value, so `slack` is more than twice that
  // bound: a comparison with p decided by more than `slack` is exact, closer ones go to fp64
  float t32 = 0.f;
#pragma unroll
  for (int i = 0; i < VPL; ++i) t32 += val[i];
  double total = (double)wave_sum_f(t32);
  const double slack = (double)(VPL + 8) * 0x1p-23 * total;
  bool all = p >= 1.0f;
  if (!all && total - (double)p <= slack) {
    total = mass_at_least(0u);  // within the error bound of p (or below): decide in fp64
    all = total < (double)p;
  }
  if (all) {
    // p >= 1, or rounding left the total below p: every block is kept
#pragma unroll
    for (int i = 0; i < VPL; ++i) kept[i] = valid(i);
    kmass = total;
  } else {
    // largest t with mass(>= t) >= p (p = 0 behaves like the smallest positive mass, so v* is
    // the maximum and exactly one block is kept)
    const double target = p > 0.f ? (double)p : 1e-300;
    // bracket [vmin, vmax]: the values between lo and hi; start with the whole row
    uint32_t a0 = 0xffffffffu, z0 = 0u;
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      a0 = min(a0, u[i]);
      z0 = max(z0, u[i]);
    }
    uint32_t vmin = wave_min_u(a0), vmax = wave_max_u(z0);
    // fp32 masses at the bracket ends, mass(>= vmin) and mass(>= vmax + 1); they only place the
    // next split point
    float m_lo = (float)total, m_hi = 0.f;
    const float tf = (float)target;
    int pass = 0;
    // invariant: mass(>= vmin) >= target > mass(>= vmax + 1)
    while (vmin < vmax) {
      // split where the mass, taken as linear in the value between the bracket ends, reaches
      // the target (about 7 passes on the 720p rows against 10 for halving the bit range); any
      // split in (vmin, vmax] keeps the invariant, and after 16 passes plain halving bounds the
      // count
      uint32_t mid;
      if (pass < 16) {
        const float fl = __uint_as_float(vmin), fh = __uint_as_float(vmax);
        const float frac = fminf(fmaxf((m_lo - tf) / fmaxf(m_lo - m_hi, 1e-30f), 0.f), 1.f);
        mid = min(max(__float_as_uint(fl + frac * (fh - fl)), vmin + 1u), vmax);
      } else {
        mid = vmin + ((vmax - vmin + 1u) >> 1);  // vmin < mid <= vmax
      }
      ++pass;
      // one pass: mass of values >= mid (fp32), smallest value >= mid, largest value < mid
      float acc = 0.f;
      uint32_t a = 0xffffffffu, z = 0u;
#pragma unroll
      for (int i = 0; i < VPL; ++i) {
        const bool ge = u[i] >= mid;
        acc += ge ? val[i] : 0.f;
        a = min(a, ge ? u[i] : 0xffffffffu);
        z = max(z, ge ? 0u : u[i]);
      }
      const float accs = wave_sum_f(acc);
      const double d = (double)accs - target;
      const bool up = d > slack ? true : d < -slack ? false : mass_at_least(mid) >= target;
      // values outside [vmin, vmax] lie below vmin or above vmax, so the smallest value >= mid
      // is inside the bracket (vmax is a candidate), and so is the largest value < mid (vmin)
      if (up) {  // mass(>= mid) >= target: the answer is >= mid
        vmin = wave_min_u(a);
        m_lo = accs;
      } else {  // mass(>= mid) < target: the answer is < mid
        vmax = wave_max_u(z);
        m_hi = accs;
      }
    }
    const uint32_t T = vmin;
    const float vstar = __uint_as_float(T);
    int nties = 0;  // blocks holding v*
#pragma unroll
    for (int i = 0; i < VPL; ++i)
      nties += (int)__builtin_popcountll(__builtin_amdgcn_ballot_w64(u[i] == T && valid(i)));
    int need = 0;  // number of tie blocks to keep
    if (nties == 1) {
      // mass(> v*) < p <= mass(>= v*) holds exactly (the search's invariant): the one block
      // at v* is kept, and the kept mass is only reported (fp32 sum)
      need = 1;
      float c32 = 0.f;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (u[i] > T) c32 += val[i];
      kmass = (double)wave_sum_f(c32) + (double)vstar;
    } else {
      // ties at v*, ascending index: position (i, lane) is index i*64 + lane; the running
      // mass from mass(> v*) in fp64
      double c = 0.0;
#pragma unroll
      for (int i = 0; i < VPL; ++i)
        if (u[i] > T) c += (double)val[i];
      double cc = wave_sum(c);
      bool done = false;
      for (int i = 0; i < VPL && !done; ++i) {
        uint64_t m = __builtin_amdgcn_ballot_w64(u[i] == T && valid(i));
        while (m != 0ull) {
          cc += (double)vstar;
          ++need;
          m &= m - 1ull;
          if (cc >= (double)p) { done = true; break; }
        }
      }
      kmass = cc;
    }
    int seen = 0;  // tie blocks before the current group of 64
#pragma unroll
    for (int i = 0; i < VPL; ++i) {
      const bool eq = u[i] == T && valid(i);
      const uint64_t m = __builtin_amdgcn_ballot_w64(eq);
      const int rank = seen + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull));
      kept[i] = u[i] > T || (eq && rank < need);  // u > T >= 0 excludes the zero slots
      seen += (int)__builtin_popcountll(m);
    }
  }

  // ascending compaction, optional byte mask
  int32_t* out_idx = idx + (int64_t)row * M;
  auto block_of = [&](int pos) { return crow != nullptr ? min(max(crow[pos], 0), M - 1) : pos; };
  int base = 0;
  if (mask != nullptr && crow != nullptr) {  // zeros first; the kept blocks are set below
    for (int j = lane; j < M; j += 64) mask[(int64_t)row * M + j] = 0;
    __threadfence_block();
  }
#pragma unroll
  for (int i = 0; i < VPL; ++i) {
    const uint64_t m = __builtin_amdgcn_ballot_w64(kept[i]);
    if (kept[i])
      out_idx[base + (int)__builtin_popcountll(m & ((1ull << lane) - 1ull))] = block_of(i * 64 + lane);
    base += (int)__builtin_popcountll(m);
    if (mask != nullptr) {
      if (crow == nullptr) {
        if (i * 64 + lane < M) mask[(int64_t)row * M + i * 64 + lane] = kept[i] ? 1 : 0;
      } else if (kept[i]) {
        mask[(int64_t)row * M + block_of(i * 64 + lane)] = 1;
      }
    }
  }
  if (lane == 0) {
    count[row] = base;
    if (mass != nullptr) mass[row] = (float)kmass;
  }
}

// ------------------------------------------------------------------------------------------
// Scores restricted to candidate key blocks (the reduced search of the GSRS abstract on the
// RECAP page at thelatestinai.com: later searches run over a candidate set found earlier). One
// wavefront per query-block row: for position r < n of the row's candidate list (block
// j = cidx[r]) the logit s * Q̄_i . K̄_j is computed in fp32 (Q̄_i from LDS, K̄_j read as whole
// 16-byte chunks) and parked in the output row; then the row max and sum over the candidates
// (DPP reductions) and the normalised values written back at the same positions.
// ------------------------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void score_cand_kernel(const float* __restrict__ qbar,
                                                         const float* __restrict__ kbar, int M,
                                                         int rows, float scale_log2,
                                                         const int32_t* __restrict__ ccount,
                                                         const int32_t* __restrict__ cidx,
                                                         float* __restrict__ probs) {
  __shared__ __align__(16) float qs[4][D];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int row = blockIdx.x * 4 + wave;
  if (row >= rows) return;  // the whole wavefront; no block-wide barrier follows
  const int64_t bh = row / M;
  for (int d = lane; d < D; d += 64) qs[wave][d] = qbar[(int64_t)row * D + d];
  __builtin_amdgcn_wave_barrier();
  const float* kb = kbar + bh * M * D;
  const int n = min(max(ccount[row], 0), M);
  const int32_t* crow = cidx + (int64_t)row * M;
  float* out = probs + (int64_t)row * M;
  float mx = -INFINITY;
  for (int r = lane; r < n; r += 64) {
    const float* kr = kb + (int64_t)min(max(crow[r], 0), M - 1) * D;
    float acc = 0.f;
#pragma unroll 8
    for (int d = 0; d < D; d += 4) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(&qs[wave][d]);
      const f32x4 b = *reinterpret_cast<const f32x4*>(kr + d);
      acc = __builtin_fmaf(a[0], b[0], acc);
      acc = __builtin_fmaf(a[1], b[1], acc);
      acc = __builtin_fmaf(a[2], b[2], acc);
      acc = __builtin_fmaf(a[3], b[3], acc);
    }
    const float x = acc * scale_log2;
    out[r] = x;  // read back by this lane only
    mx = fmaxf(mx, x);
  }
  mx = wave_max_f(mx);
  float l = 0.f;
  for (int r = lane; r < n; r += 64) l += __builtin_amdgcn_exp2f(out[r] - mx);
  const float inv = 1.0f / wave_sum_f(l);
  for (int r = lane; r < n; r += 64) out[r] = __builtin_amdgcn_exp2f(out[r] - mx) * inv;
}

// ------------------------------------------------------------------------------------------
// Drift of the block means between two steps, per (b, h): ||X̄ - X̄_ref||_F / ||X̄_ref||_F for
// X = Q and X = K, sums in fp64 over the M x D means (one 1024-thread work-group per (b, h),
// 16-byte loads; a fixed reduction order, so the result is deterministic); a caller reuses
// the mask of the reference step while both stay under its threshold.
// ------------------------------------------------------------------------------------------
__global__ __launch_bounds__(1024) void mean_drift_kernel(const float* __restrict__ qbar,
                                                          const float* __restrict__ kbar,
                                                          const float* __restrict__ qref,
                                                          const float* __restrict__ kref,
                                                          int64_t per_head,
                                                          float* __restrict__ drift) {
  __shared__ double red[16][4];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t off = (int64_t)blockIdx.x * per_head;  // per_head = M * D, a multiple of 64
  double dq = 0.0, rq = 0.0, dk = 0.0, rk = 0.0;
  for (int64_t t = threadIdx.x * 4; t < per_head; t += 1024 * 4) {
    const f32x4 a = *reinterpret_cast<const f32x4*>(qbar + off + t);
    const f32x4 ar = *reinterpret_cast<const f32x4*>(qref + off + t);
    const f32x4 b = *reinterpret_cast<const f32x4*>(kbar + off + t);
    const f32x4 br = *reinterpret_cast<const f32x4*>(kref + off + t);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const double x = (double)a[e] - (double)ar[e], y = (double)b[e] - (double)br[e];
      dq += x * x;
      rq += (double)ar[e] * (double)ar[e];
      dk += y * y;
      rk += (double)br[e] * (double)br[e];
    }
  }
  double v[4] = {dq, rq, dk, rk};
#pragma unroll
  for (int c = 0; c < 4; ++c) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v[c] += __shfl_xor(v[c], o);
    if (lane == 0) red[wave][c] = v[c];
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    double t[4] = {0.0, 0.0, 0.0, 0.0};
    for (int w = 0; w < 16; ++w)
      for (int c = 0; c < 4; ++c) t[c] += red[w][c];
    drift[2 * blockIdx.x] = (float)(t[1] > 0.0 ? sqrt(t[0] / t[1]) : (t[0] > 0.0 ? INFINITY : 0.0));
    drift[2 * blockIdx.x + 1] =
        (float)(t[3] > 0.0 ? sqrt(t[2] / t[3]) : (t[2] > 0.0 ? INFINITY : 0.0));
  }
}

// ------------------------------------------------------------------------------------------
hipError_t launch_pool(const bf16_t* q, const bf16_t* k, Strides st, int B, int H, int N, int D,
                       int block, float* qbar, float* kbar, hipStream_t stream) {
  if (block < 1 || block > 128) return hipErrorInvalidValue;  // the kernel's loads cover 128 rows
  const int M = (N + block - 1) / block;
  const int rows = B * H * M;
  const int grid = (2 * rows + 3) / 4;
  if (D == 128)
    pool_kernel<128><<<grid, 256, 0, stream>>>(q, k, st, H, N, block, M, rows, qbar, kbar);
  else
    pool_kernel<64><<<grid, 256, 0, stream>>>(q, k, st, H, N, block, M, rows, qbar, kbar);
  return hipGetLastError();
}

// Raise a kernel's dynamic-LDS limit to `bytes` once per device (the launches below then stay
// plain stream work, with no driver call per launch).
static hipError_t allow_lds_once(const void* kernel, int bytes, std::atomic<uint32_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint32_t bit = dev < 32 ? 1u << dev : 0u;
  if (bit != 0u && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit != 0u) done.fetch_or(bit, std::memory_order_acq_rel);
  return e;
}

hipError_t launch_scores(const float* qbar, const float* kbar, int BH, int M, int D,
                         float scale_log2, float* probs, hipStream_t stream) {
  const size_t lds = (size_t)kStripRows * strip_stride(M) * sizeof(float);
  static_assert(kStripMaxM <= 64 * kStripVals, "a row must fit in the lanes' registers");
  static_assert(kStripRows * strip_stride(kStripMaxM) * sizeof(float) <= 80 * 1024,
                "two strips per CU");
  if (M <= kStripMaxM) {  // rows fit in LDS and registers: one pass
    const int sgrid = BH * ((M + kStripRows - 1) / kStripRows);
    constexpr int kMaxLds = kStripRows * strip_stride(kStripMaxM) * sizeof(float);
    static std::atomic<uint32_t> lds128{0u}, lds64{0u};
    if (D == 128) {
      const hipError_t e =
          allow_lds_once((const void*)score_strip_kernel<128, false>, kMaxLds, lds128);
      if (e != hipSuccess) return e;
      score_strip_kernel<128, false><<<sgrid, kStripWaves * 64, lds, stream>>>(qbar, kbar, M, scale_log2,
                                                                  nullptr, nullptr, probs);
    } else {
      const hipError_t e =
          allow_lds_once((const void*)score_strip_kernel<64, false>, kMaxLds, lds64);
      if (e != hipSuccess) return e;
      score_strip_kernel<64, false><<<sgrid, kStripWaves * 64, lds, stream>>>(qbar, kbar, M, scale_log2,
                                                                 nullptr, nullptr, probs);
    }
    return hipGetLastError();
  }
  const int grid = BH * ((M + 31) / 32);
  if (D == 128)
    score_kernel<128><<<grid, 256, 0, stream>>>(qbar, kbar, M, scale_log2, probs);
  else
    score_kernel<64><<<grid, 256, 0, stream>>>(qbar, kbar, M, scale_log2, probs);
  return hipGetLastError();
}

hipError_t launch_topp(const float* probs, int B, int H, int M, const HeadScalars& top_p,
                       const int32_t* ccount, const int32_t* cidx, int32_t* count, int32_t* idx,
                       uint8_t* mask, float* mass, hipStream_t stream) {
  const int rows = B * H * M;
  const int grid = (rows + 3) / 4;
  if (M <= 512) {
    topp_wave_kernel<8><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  if (M <= 768) {
    topp_wave_kernel<12><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  if (M <= 1024) {
    topp_wave_kernel<16><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  if (M <= 1280) {
    topp_wave_kernel<20><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  if (M <= 1536) {
    topp_wave_kernel<24><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  if (M <= 2048) {
    topp_wave_kernel<32><<<grid, 256, 0, stream>>>(probs, H, M, rows, top_p, ccount, cidx, count,
                                                   idx, mask, mass);
    return hipGetLastError();
  }
  // longer rows: one work-group per row, bitonic sort in LDS
  int P = 64;
  while (P < M) P <<= 1;
  const size_t lds = (size_t)P * 9;
  static std::atomic<uint32_t> lds_topp{0u};
  const hipError_t e = allow_lds_once((const void*)topp_kernel, kMaxBlocks * 9, lds_topp);
  if (e != hipSuccess) return e;
  topp_kernel<<<B * H * M, 256, lds, stream>>>(probs, H, M, P, top_p, ccount, cidx, count, idx,
                                                mask, mass);
  return hipGetLastError();
}

hipError_t launch_scores_cand(const float* qbar, const float* kbar, int BH, int M, int D,
                              float scale_log2, const int32_t* ccount, const int32_t* cidx,
                              float* probs, hipStream_t stream) {
  if (M <= kStripMaxM) {  // the one-pass strip kernel, normalising over the candidates
    const size_t lds = (size_t)kStripRows * strip_stride(M) * sizeof(float);
    const int sgrid = BH * ((M + kStripRows - 1) / kStripRows);
    constexpr int kMaxLds = kStripRows * strip_stride(kStripMaxM) * sizeof(float);
    static std::atomic<uint32_t> lds128{0u}, lds64{0u};
    if (D == 128) {
      const hipError_t e =
          allow_lds_once((const void*)score_strip_kernel<128, true>, kMaxLds, lds128);
      if (e != hipSuccess) return e;
      score_strip_kernel<128, true><<<sgrid, kStripWaves * 64, lds, stream>>>(qbar, kbar, M, scale_log2,
                                                                 ccount, cidx, probs);
    } else {
      const hipError_t e =
          allow_lds_once((const void*)score_strip_kernel<64, true>, kMaxLds, lds64);
      if (e != hipSuccess) return e;
      score_strip_kernel<64, true><<<sgrid, kStripWaves * 64, lds, stream>>>(qbar, kbar, M, scale_log2,
                                                                ccount, cidx, probs);
    }
    return hipGetLastError();
  }
  const int rows = BH * M;
  const int grid = (rows + 3) / 4;
  if (D == 128)
    score_cand_kernel<128><<<grid, 256, 0, stream>>>(qbar, kbar, M, rows, scale_log2, ccount,
                                                     cidx, probs);
  else
    score_cand_kernel<64><<<grid, 256, 0, stream>>>(qbar, kbar, M, rows, scale_log2, ccount,
                                                    cidx, probs);
  return hipGetLastError();
}

hipError_t launch_mean_drift(const float* qbar, const float* kbar, const float* qref,
                             const float* kref, int BH, int M, int D, float* drift,
                             hipStream_t stream) {
  mean_drift_kernel<<<BH, 1024, 0, stream>>>(qbar, kbar, qref, kref, (int64_t)M * D, drift);
  return hipGetLastError();
}

}  // namespace recap
