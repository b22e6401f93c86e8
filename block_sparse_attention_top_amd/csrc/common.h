// Internal declarations shared by the HIP kernels and the C-ABI host layer (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace recap {

typedef __bf16 bf16_t;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(4))) __bf16 bf16x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) float f32x4;

constexpr int kMaxHeads = 128;
constexpr int kMaxBlocks = 8192;  // M upper bound (include/recap.h RECAP_MAX_BLOCKS)
constexpr int kKeyTile = 64;  // keys per attention inner-loop tile
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

struct HeadScalars {
  float v[kMaxHeads];
};

// Strided bf16 tensor [B,H,N,D] view (element strides, D contiguous).
struct Strides {
  int64_t b, h, n;
};

// Work-group index remap so that each XCD (8 per MI355X, work-groups dispatched round-robin
// across them) receives one contiguous range of logical tiles: neighbouring query blocks of
// one head then share key/value lines in that XCD's L2. A bijection on [0, n) whatever the
// dispatch order, so correctness does not depend on it.
__host__ __device__ __forceinline__ int xcd_remap(int wg, int n) {
  const int q = n >> 3, r = n & 7;
  const int xcd = wg & 7, k = wg >> 3;
  return (xcd < r) ? xcd * (q + 1) + k : r * (q + 1) + (xcd - r) * q + k;
}
// The other remap: each XCD receives runs of C consecutive logical tiles in turn, so at any
// time the eight XCDs work on neighbouring tiles of one head. That head's K/V then stays in
// the last-level cache all XCDs share, while each XCD's L2 still serves runs of neighbouring
// query tiles. (With one range per XCD, eight heads' K/V are in flight at once, about 310 MB
// at 720p.) A bijection on [0, n): runs on the largest multiple of 8C, identity after.
template <int C>
__host__ __device__ __forceinline__ int xcd_runs(int wg, int n) {
  const int full = (n / (8 * C)) * (8 * C);
  if (wg >= full) return wg;
  const int xcd = wg & 7, k = wg >> 3;
  return (k / C) * 8 * C + xcd * C + (k % C);
}

// ---- launchers (defined in the kernel sources; all asynchronous on `stream`) ----
hipError_t launch_pool(const bf16_t* q, const bf16_t* k, Strides st, int B, int H, int N, int D,
                       int block, float* qbar, float* kbar, hipStream_t stream);
hipError_t launch_scores(const float* qbar, const float* kbar, int BH, int M, int D,
                         float scale_log2, float* probs, hipStream_t stream);
hipError_t launch_topp(const float* probs, int B, int H, int M, const HeadScalars& top_p,
                       const int32_t* ccount, const int32_t* cidx, int32_t* count, int32_t* idx,
                       uint8_t* mask, float* mass, hipStream_t stream);
hipError_t launch_scores_cand(const float* qbar, const float* kbar, int BH, int M, int D,
                              float scale_log2, const int32_t* ccount, const int32_t* cidx,
                              float* probs, hipStream_t stream);
hipError_t launch_mean_drift(const float* qbar, const float* kbar, const float* qref,
                             const float* kref, int BH, int M, int D, float* drift,
                             hipStream_t stream);

enum AttnMode { kSparse = 0, kDense = 1, kCaptureR = 2, kDenseCapture = 3, kDenseTail = 4 };

struct AttnParams {
  const bf16_t* q;
  const bf16_t* k;
  const bf16_t* v;   // V, bf16, the layout and strides of q and k
  Strides st;
  int H, N, M, block, npad;
  int mq;  // query tiles per (b, h); set by launch_attention
  float scale_log2;
  const int32_t* count;  // [B*H*M]
  const int32_t* idx;    // [B*H*M*M]
  const bf16_t* res;     // optional residual (sparse mode)
  bf16_t* out;
  bf16_t* res_out;  // capture: residual output
  float* od_ws;     // capture: fp32 dense output [B*H][npad][D] of blocks left to the residual pass
  uint8_t* flags;   // capture: [B*H*M] 1 = residual of this query block left to the residual pass
  float* lse_out;   // optional [B*H][N]: natural-log log-sum-exp of the attended scores
  float* kmass_out; // optional [B*H][N] (capture mode): kept share of the dense attention mass
  float* o32_out;   // optional [B*H][N][D] (sparse mode): fp32 output instead of bf16 `out`
  float* tail_lse;  // kDenseTail: [B*H][N] log-mass of the keys outside the kept set
  float* tail_o;    // kDenseTail: [B*H][N][D] attention output over those keys
  HeadScalars res_scale;
  const int32_t* end_order;  // optional (sparse mode): ranks of the grid's last end_order_g tiles
  int end_order_g;
};

hipError_t launch_attention(AttnParams p, int B, int D, AttnMode mode, hipStream_t stream);

// The last tiles of a paired sparse grid run longest walk first: number of tiles ordered (0 when
// the call does not order), and the one-work-group kernel that writes their order (int32 [G]).
constexpr int kEndOrderTiles = 1024;
int sparse_end_order_tiles(int B, int H, int M, int block);
hipError_t launch_end_order(const int32_t* counts, int B, int H, int M, int G, int32_t* order,
                            hipStream_t stream);

// Coarse tail of the attention-level reconstruction: attention over the pooled key blocks
// outside each query block's kept set (block means stand for their tokens).
struct TailParams {
  const bf16_t* q;
  Strides st;          // q strides
  const bf16_t* kb;    // pooled keys, bf16 [B*H][mpad][D] (rows >= M zero): hi part
  const bf16_t* kb_lo; // bf16(K̄ - hi), same layout
  const bf16_t* vb;    // pooled values, bf16 [B*H][mpad][D] (rows >= M zero)
  int H, N, M, block, mpad, mq;
  float scale_log2;
  float last_bias;     // added to the log2-unit score of pooled key M-1: log2(n_last / block)
  float ln_block;      // ln(block): each pooled key stands for `block` tokens
  const uint32_t* bits; // kept-block bitmaps [B*H][M][wbits] (bit j of row i: j kept)
  int wbits;            // words per bitmap row: ceil(M / 32) + 1 (the last one zero)
  float* tail_lse;     // [B*H][N]
  float* tail_o;       // [B*H][N][D]
  // moment refinements (null when off)
  const bf16_t* sv;    // (s/2) * per-dimension key variance, bf16 [B*H][mpad][D], rows >= M 0
  const bf16_t* cov;   // (s/N) * pooled value-key covariance as a bf16 pair: hi [B*H][D][D]
                       // (row: value dim), then lo in the same layout
  int BH;              // B * H (offset of the lo half of cov)
};
hipError_t launch_tail_keys(const float* kbar, const float* vbar, const float* var,
                            float var_scale, int BH, int M, int D, int mpad, bf16_t* kb_hi,
                            bf16_t* kb_lo, bf16_t* vb16, bf16_t* sv16, hipStream_t stream);
hipError_t launch_tail(TailParams p, int B, int D, hipStream_t stream);
// Kept lists -> bitmaps [B*H*M][wbits] (wbits = ceil(M/32) + 1 words, the last one zero).
hipError_t launch_kept_bits(const int32_t* count, const int32_t* idx, int rows, int M, int wbits,
                            uint32_t* bits, hipStream_t stream);
// Moment statistics of the key/value blocks: per-dimension key variance var [B*H][M][D] and
// the pooled within-block value-key covariance, as per-slice partial sums
// cov_part [B*H][nslice][D][D], reduced to cov16 = cov_scale * sum as a bf16 pair (hi
// [B*H][D][D], then lo).
constexpr int kStatSlice = 32;  // key blocks per slice of the covariance sums
hipError_t launch_tail_stats(const bf16_t* k, const bf16_t* v, Strides st, int B, int H, int N,
                             int D, int block, const float* kbar, const float* vbar, float* var,
                             float* cov_part, float cov_scale, bf16_t* cov16,
                             hipStream_t stream);
// mode 0: d = exact - coarse (d_lse [B*H][N], d_o [B*H][N][D], fp32);
// mode 1: out (bf16, q layout) = merge of the fp32 sparse output (log-mass lse_s) with the
// tail (coarse + d, d optional)
hipError_t launch_tail_combine(int mode, int B, int H, int N, int D, Strides st,
                               const float* a_lse, const float* a_o, const float* c_lse,
                               const float* c_o, const float* d_lse, const float* d_o,
                               float* d_lse_out, float* d_o_out, bf16_t* out,
                               hipStream_t stream);

// FP8 (MXFP8) block-sparse attention: Q codes and scales token-major, K and V as packed
// 64-key tiles (codes then scales, 66*D bytes each).
struct MxParams {
  const uint8_t* q8;  // [B*H][N][D] E4M3 codes
  const uint8_t* qs;  // [B*H][N][D/32] E8M0 scales
  const uint8_t* kt;  // [B*H][ntile] packed K tiles
  const uint8_t* vt;  // [B*H][ntile] packed V tiles
  Strides st;         // out / residual strides
  int H, N, M, block, ntile, mq;
  float scale_log2;
  const int32_t* count;
  const int32_t* idx;
  const bf16_t* res;  // optional residual (epilogue O + c_h R)
  bf16_t* out;
  float* lse_out;     // optional [B*H][N]
  HeadScalars res_scale;
};
hipError_t launch_mx_rows(const bf16_t* x, Strides st, int B, int H, int N, int D,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_cols(const bf16_t* x, Strides st, int B, int H, int N, int D,
                          uint8_t* codes, uint8_t* scales, hipStream_t stream);
hipError_t launch_mx_kv_tiles(const bf16_t* k, const bf16_t* v, Strides st, int B, int H, int N,
                              int D, int ntile, uint8_t* kt, uint8_t* vt, hipStream_t stream);
hipError_t launch_attention_mx(MxParams p, int B, int D, hipStream_t stream);

}  // namespace recap
