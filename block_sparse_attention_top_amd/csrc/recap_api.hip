// C-ABI entry points: argument validation (before any HIP call), workspace carving and
// kernel launches. The operations themselves are documented in include/recap.h.
#include <math.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "../../include/recap.h"
#include "common.h"

using namespace recap;

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxStrideN = (int64_t)1 << 24;  // elements
inline size_t align_up(size_t x) { return (x + kAlign - 1) & ~(kAlign - 1); }

int validate_desc(const recap_desc* d) {
  if (d == nullptr) return RECAP_E_NULL;
  if (d->batch < 1 || d->heads < 1 || d->heads > RECAP_MAX_HEADS || d->seq < 1) return RECAP_E_SHAPE;
  if (d->head_dim != 64 && d->head_dim != 128) return RECAP_E_SHAPE;
  if (d->block != 64 && d->block != 128) return RECAP_E_SHAPE;
  if (d->reserved != 0) return RECAP_E_SHAPE;
  const int64_t m = ((int64_t)d->seq + d->block - 1) / d->block;
  if (m > RECAP_MAX_BLOCKS) return RECAP_E_SHAPE;
  // products used in 32-bit grid arithmetic
  if ((int64_t)d->batch * d->heads * m > (int64_t)1 << 30) return RECAP_E_SHAPE;
  const int64_t s[3] = {d->stride_b, d->stride_h, d->stride_n};
  for (int i = 0; i < 3; ++i)
    if (s[i] <= 0 || (s[i] % 8) != 0) return RECAP_E_STRIDE;
  // the attention kernels address the rows of one key tile (up to 128 tokens) as 32-bit byte
  // offsets from the tile's first row: 128 * stride_n * 2 bytes must stay below 2^32
  if (d->stride_n >= kMaxStrideN) return RECAP_E_STRIDE;
  // no two (b, h, n) index triples may address the same row: sort the three dimensions by
  // stride and require each stride to clear the full extent of the next-smaller one
  int64_t ext[3] = {d->batch, d->heads, d->seq};
  int64_t st[3] = {d->stride_b, d->stride_h, d->stride_n};
  for (int i = 0; i < 3; ++i)
    for (int j = i + 1; j < 3; ++j)
      if (st[j] < st[i]) {
        int64_t t = st[i]; st[i] = st[j]; st[j] = t;
        t = ext[i]; ext[i] = ext[j]; ext[j] = t;
      }
  int64_t span = d->head_dim;  // elements covered by the dimensions below
  for (int i = 0; i < 3; ++i) {
    if (ext[i] > 1 && st[i] < span) return RECAP_E_STRIDE;
    // the whole tensor must be addressable with 64-bit element offsets
    if (ext[i] > 1 && st[i] > (INT64_MAX - span) / (ext[i] - 1)) return RECAP_E_STRIDE;
    span = st[i] * (ext[i] - 1) + span;
  }
  return RECAP_OK;
}

inline int num_blocks(const recap_desc* d) { return (d->seq + d->block - 1) / d->block; }
// Sparse calls with paired 64-token blocks: the order of the grid's last tiles (int32 each).
size_t end_order_bytes(const recap_desc* d) {
  const int g = sparse_end_order_tiles(d->batch, d->heads, num_blocks(d), d->block);
  return g > 0 ? align_up((size_t)g * sizeof(int32_t)) : 0;
}

inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

size_t pooled_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * num_blocks(d) * d->head_dim * sizeof(float));
}
size_t snapshot_bytes(const recap_desc* d) {
  const size_t npad = (size_t)num_blocks(d) * d->block;
  return align_up((size_t)d->batch * d->heads * npad * d->head_dim * sizeof(float));
}

size_t flag_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * num_blocks(d));
}

// Coarse tail: pooled keys and values padded to whole 64-key tiles.
inline int pooled_pad(const recap_desc* d) { return (num_blocks(d) + 63) / 64 * 64; }
size_t pooled16_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * pooled_pad(d) * d->head_dim * 2);
}
size_t row_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * d->seq * sizeof(float));
}
size_t row_d_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * d->seq * d->head_dim * sizeof(float));
}
// kept-block bitmaps of the coarse tail: wbits words per query block (the last one zero)
inline int bit_words(const recap_desc* d) { return (num_blocks(d) + 31) / 32 + 1; }
size_t bits_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * num_blocks(d) * bit_words(d) * 4);
}
// moment refinements: per-slice covariance partial sums (fp32) and the reduced covariance (bf16)
inline int stat_slices(const recap_desc* d) { return (num_blocks(d) + kStatSlice - 1) / kStatSlice; }
size_t cov_part_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * stat_slices(d) * d->head_dim * d->head_dim * 4);
}
size_t cov16_bytes(const recap_desc* d) {  // hi and lo halves
  return align_up((size_t)d->batch * d->heads * d->head_dim * d->head_dim * 2 * 2);
}
// K̄, V̄ (fp32), K̄ hi and lo, V̄ (bf16), the kept bitmaps, and for the moment refinements the
// key variances (fp32), their scaled bf16 copy and the covariance
size_t tail_estimate_bytes(const recap_desc* d) {
  return 2 * pooled_bytes(d) + 3 * pooled16_bytes(d) + bits_bytes(d) + pooled_bytes(d) +
         pooled16_bytes(d) + cov_part_bytes(d) + cov16_bytes(d);
}
// one attention part (log-sum-exp, fp32 output); the coarse tail (same); the estimate
size_t tail_merge_bytes(const recap_desc* d) {
  return 2 * (row_bytes(d) + row_d_bytes(d)) + tail_estimate_bytes(d);
}

// FP8 sparse call: Q codes [B*H][N][D] and scales [B*H][N][D/32], packed K and V tiles
// (66*D bytes per 64-key tile)
inline int64_t fp8_tiles(const recap_desc* d) {
  return (int64_t)d->batch * d->heads * ((int64_t)num_blocks(d) * d->block / 64);
}
size_t fp8_q_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * d->seq * d->head_dim);
}
size_t fp8_qs_bytes(const recap_desc* d) {
  return align_up((size_t)d->batch * d->heads * d->seq * (d->head_dim / 32));
}
size_t fp8_tile_bytes(const recap_desc* d) {
  return align_up((size_t)fp8_tiles(d) * 66 * d->head_dim);
}
size_t fp8_bytes(const recap_desc* d) {
  return fp8_q_bytes(d) + fp8_qs_bytes(d) + 2 * fp8_tile_bytes(d);
}

size_t workspace_for(int op, const recap_desc* d) {
  switch (op) {
    case RECAP_OP_BLOCK_SCORES: return 2 * pooled_bytes(d);
    case RECAP_OP_TOPP: return 0;
    case RECAP_OP_SPARSE: return end_order_bytes(d);
    case RECAP_OP_DENSE: return 0;
    case RECAP_OP_DENSE_CAPTURE: return snapshot_bytes(d) + flag_bytes(d);
    case RECAP_OP_TAIL: return tail_estimate_bytes(d);
    case RECAP_OP_DENSE_TAIL:
    case RECAP_OP_SPARSE_TAIL: return tail_merge_bytes(d);
    case RECAP_OP_SPARSE_FP8: return fp8_bytes(d);
    default: return 0;
  }
}

int check_workspace(int op, const recap_desc* d, const void* ws, size_t ws_bytes) {
  const size_t need = workspace_for(op, d);
  if (need == 0) return RECAP_OK;
  if (ws == nullptr || ws_bytes < need) return RECAP_E_WORKSPACE;
  if (((uintptr_t)ws & (kAlign - 1)) != 0) return RECAP_E_ALIGN;
  return RECAP_OK;
}

// Per-device "is gfx950" cache, filled once per device.
constexpr int kMaxDevices = 64;
std::atomic<int> g_dev_ok[kMaxDevices];  // 0 unknown, 1 ok, -1 unsupported
std::mutex g_dev_mu;

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return RECAP_E_DEVICE;
  }
  int state = g_dev_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    std::lock_guard<std::mutex> lk(g_dev_mu);
    state = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (state == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
        (void)hipGetLastError();
        return RECAP_E_DEVICE;
      }
      state = strncmp(prop.gcnArchName, "gfx950", 6) == 0 ? 1 : -1;
      g_dev_ok[dev].store(state, std::memory_order_release);
    }
  }
  return state == 1 ? RECAP_OK : RECAP_E_DEVICE;
}

// Fixed device scratch of recap_block_scores_noalloc: the pooled means of one call (2 x fp32
// [B*H][M][D]). A file-scope device array, so the library never allocates it; each device
// holds its own copy (at its own address) from the code object's load until the process ends.
// Host code must not pass `scratch` itself to a kernel (in host code it names a host-side
// stand-in): the device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) unsigned char scratch[RECAP_NOALLOC_SCRATCH_BYTES];

std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

// The current device's address of `scratch`, looked up on the first call on that device with
// that device current.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return RECAP_E_DEVICE;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || addr == nullptr) {
        (void)hipGetLastError();
        return RECAP_E_DEVICE;
      }
      g_scratch[dev].store(addr, std::memory_order_release);
      p = addr;
    }
  }
  *out = p;
  return RECAP_OK;
}

inline Strides strides_of(const recap_desc* d) { return Strides{d->stride_b, d->stride_h, d->stride_n}; }

int launched(hipError_t e) {
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return RECAP_E_LAUNCH;
  }
  return RECAP_OK;
}

int validate_block_scores(const recap_desc* d, const void* q, const void* k, float sm_scale,
                          const float* probs) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || probs == nullptr) return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(probs)) return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  return RECAP_OK;
}

// Pooling then scores; ws holds the two pooled-mean arrays (2 * pooled_bytes).
int launch_block_scores(const recap_desc* d, const void* q, const void* k, float sm_scale,
                        float* probs, void* ws, hipStream_t st) {
  const int M = num_blocks(d);
  float* qbar = (float*)ws;
  float* kbar = (float*)((char*)ws + pooled_bytes(d));
  hipError_t e = launch_pool((const bf16_t*)q, (const bf16_t*)k, strides_of(d), d->batch,
                             d->heads, d->seq, d->head_dim, d->block, qbar, kbar, st);
  if (e == hipSuccess)
    e = launch_scores(qbar, kbar, d->batch * d->heads, M, d->head_dim,
                      (float)((double)sm_scale * 1.4426950408889634), probs, st);
  return launched(e);
}

}  // namespace

extern "C" {

int recap_abi_version(void) { return RECAP_ABI_VERSION; }

const char* recap_status_string(int status) {
  switch (status) {
    case RECAP_OK: return "ok";
    case RECAP_E_NULL: return "a required pointer is NULL";
    case RECAP_E_SHAPE: return "unsupported shape (batch, heads, seq, head_dim or block)";
    case RECAP_E_STRIDE: return "invalid strides (positive multiples of 8, non-overlapping)";
    case RECAP_E_ALIGN: return "a base pointer is not 16-byte aligned (workspace: 256-byte)";
    case RECAP_E_VALUE: return "a scalar or per-head value is out of range";
    case RECAP_E_WORKSPACE: return "workspace missing or too small (no-alloc calls: the fixed scratch is too small)";
    case RECAP_E_DEVICE: return "no current gfx950 HIP device";
    case RECAP_E_LAUNCH: return "kernel launch failed";
    default: return "unknown status";
  }
}

int recap_workspace_size(int op, const recap_desc* d, size_t* bytes) {
  if (bytes == nullptr) return RECAP_E_NULL;
  const int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (op < RECAP_OP_BLOCK_SCORES || op > RECAP_OP_SPARSE_FP8) return RECAP_E_VALUE;
  *bytes = workspace_for(op, d);
  return RECAP_OK;
}

int recap_block_scores(const recap_desc* d, const void* q, const void* k, float sm_scale,
                       float* probs, void* ws, size_t ws_bytes, void* stream) {
  int s = validate_block_scores(d, q, k, sm_scale, probs);
  if (s != RECAP_OK) return s;
  if ((s = check_workspace(RECAP_OP_BLOCK_SCORES, d, ws, ws_bytes)) != RECAP_OK) return s;
  if ((s = check_device()) != RECAP_OK) return s;
  return launch_block_scores(d, q, k, sm_scale, probs, ws, (hipStream_t)stream);
}

int recap_block_scores_noalloc(const recap_desc* d, const void* q, const void* k,
                               float sm_scale, float* probs, void* stream) {
  int s = validate_block_scores(d, q, k, sm_scale, probs);
  if (s != RECAP_OK) return s;
  if (workspace_for(RECAP_OP_BLOCK_SCORES, d) > (size_t)RECAP_NOALLOC_SCRATCH_BYTES)
    return RECAP_E_WORKSPACE;
  if ((s = check_device()) != RECAP_OK) return s;
  void* ws = nullptr;
  if ((s = scratch_address(&ws)) != RECAP_OK) return s;
  // the pooling kernel writes every mean the score kernel reads: nothing to clear
  return launch_block_scores(d, q, k, sm_scale, probs, ws, (hipStream_t)stream);
}

int recap_topp_mask(const recap_desc* d, const float* probs, const float* top_p_host,
                    int32_t* kept_count, int32_t* kept_idx, uint8_t* mask_opt,
                    float* kept_mass_opt, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (probs == nullptr || top_p_host == nullptr || kept_count == nullptr || kept_idx == nullptr)
    return RECAP_E_NULL;
  if (!aligned16(probs) || !aligned16(kept_count) || !aligned16(kept_idx) ||
      (mask_opt && !aligned16(mask_opt)) || (kept_mass_opt && !aligned16(kept_mass_opt)))
    return RECAP_E_ALIGN;
  HeadScalars tp;
  memset(&tp, 0, sizeof(tp));
  for (int h = 0; h < d->heads; ++h) {
    const float p = top_p_host[h];
    if (!(p >= 0.f && p <= 1.f)) return RECAP_E_VALUE;  // also rejects NaN
    tp.v[h] = p;
  }
  if ((s = check_device()) != RECAP_OK) return s;
  return launched(launch_topp(probs, d->batch, d->heads, num_blocks(d), tp, nullptr, nullptr,
                              kept_count, kept_idx, mask_opt, kept_mass_opt,
                              (hipStream_t)stream));
}

}  // extern "C"

namespace {

int sparse_impl(const recap_desc* d, const void* q, const void* k, const void* v,
                const int32_t* kept_count, const int32_t* kept_idx, float sm_scale,
                const void* residual_opt, const float* res_scale_host, void* out,
                float* lse_out, void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || kept_count == nullptr ||
      kept_idx == nullptr || out == nullptr)
    return RECAP_E_NULL;
  if (residual_opt != nullptr && res_scale_host == nullptr) return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(kept_count) || !aligned16(kept_idx) ||
      (residual_opt != nullptr && !aligned16(residual_opt)))
    return RECAP_E_ALIGN;
  if (lse_out != nullptr && !aligned16(lse_out)) return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  if (out == q || out == k || out == v || (residual_opt != nullptr && out == residual_opt))
    return RECAP_E_VALUE;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  if (residual_opt != nullptr) {
    for (int h = 0; h < d->heads; ++h) {
      if (!isfinite(res_scale_host[h])) return RECAP_E_VALUE;
      p.res_scale.v[h] = res_scale_host[h];
    }
  }
  if ((s = check_workspace(RECAP_OP_SPARSE, d, ws, ws_bytes)) != RECAP_OK) return s;
  if ((s = check_device()) != RECAP_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  const int M = num_blocks(d);
  const int npad = M * d->block;
  p.q = (const bf16_t*)q;
  p.k = (const bf16_t*)k;
  p.v = (const bf16_t*)v;
  p.st = strides_of(d);
  p.H = d->heads;
  p.N = d->seq;
  p.M = M;
  p.block = d->block;
  p.npad = npad;
  p.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  p.count = kept_count;
  p.idx = kept_idx;
  p.res = (const bf16_t*)residual_opt;
  p.out = (bf16_t*)out;
  p.lse_out = lse_out;
  // the grid's last tiles run longest walk first (their order written to the workspace)
  const int g = sparse_end_order_tiles(d->batch, d->heads, M, d->block);
  if (g > 0) {
    hipError_t e = launch_end_order(kept_count, d->batch, d->heads, M, g, (int32_t*)ws, st);
    if (e != hipSuccess) return launched(e);
    p.end_order = (const int32_t*)ws;
    p.end_order_g = g;
  }
  return launched(launch_attention(p, d->batch, d->head_dim, kSparse, st));
}

int dense_impl(const recap_desc* d, const void* q, const void* k, const void* v,
               float sm_scale, const int32_t* kept_count_opt, const int32_t* kept_idx_opt,
               void* out, void* residual_out_opt, float* lse_out, float* kmass_out,
               void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || out == nullptr) return RECAP_E_NULL;
  // the kept-block accumulation runs for the residual and for the kept-mass output
  const bool capture = residual_out_opt != nullptr || kmass_out != nullptr;
  if (capture && (kept_count_opt == nullptr || kept_idx_opt == nullptr)) return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      (residual_out_opt != nullptr && !aligned16(residual_out_opt)) ||
      (capture && (!aligned16(kept_count_opt) || !aligned16(kept_idx_opt))) ||
      (lse_out != nullptr && !aligned16(lse_out)) ||
      (kmass_out != nullptr && !aligned16(kmass_out)))
    return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  if (out == q || out == k || out == v ||
      (residual_out_opt != nullptr && (residual_out_opt == out || residual_out_opt == q ||
                                       residual_out_opt == k || residual_out_opt == v)))
    return RECAP_E_VALUE;
  const int op = capture ? RECAP_OP_DENSE_CAPTURE : RECAP_OP_DENSE;
  if ((s = check_workspace(op, d, ws, ws_bytes)) != RECAP_OK) return s;
  if ((s = check_device()) != RECAP_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  const int M = num_blocks(d);
  const int npad = M * d->block;
  AttnParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const bf16_t*)q;
  p.k = (const bf16_t*)k;
  p.v = (const bf16_t*)v;
  p.st = strides_of(d);
  p.H = d->heads;
  p.N = d->seq;
  p.M = M;
  p.block = d->block;
  p.npad = npad;
  p.scale_log2 = (float)((double)sm_scale * 1.4426950408889634);
  p.count = kept_count_opt;
  p.idx = kept_idx_opt;
  p.out = (bf16_t*)out;
  p.res_out = (bf16_t*)residual_out_opt;
  p.od_ws = capture ? (float*)ws : nullptr;
  p.flags = capture ? (uint8_t*)ws + snapshot_bytes(d) : nullptr;
  p.lse_out = lse_out;
  p.kmass_out = kmass_out;
  // capture: the dense pass also accumulates the kept blocks and writes R; the residual pass
  // only recomputes query blocks the dense pass flagged (kept mass underflow), others exit
  hipError_t e = launch_attention(p, d->batch, d->head_dim, capture ? kDenseCapture : kDense, st);
  if (e == hipSuccess && residual_out_opt != nullptr)
    e = launch_attention(p, d->batch, d->head_dim, kCaptureR, st);
  return launched(e);
}

}  // namespace

extern "C" {

int recap_block_means(const recap_desc* d, const void* q, const void* k, float* qbar,
                      float* kbar, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || qbar == nullptr || kbar == nullptr) return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(qbar) || !aligned16(kbar)) return RECAP_E_ALIGN;
  if (qbar == kbar) return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;
  return launched(launch_pool((const bf16_t*)q, (const bf16_t*)k, strides_of(d), d->batch,
                              d->heads, d->seq, d->head_dim, d->block, qbar, kbar,
                              (hipStream_t)stream));
}

int recap_scores_from_means(const recap_desc* d, const float* qbar, const float* kbar,
                            float sm_scale, const int32_t* cand_count_opt,
                            const int32_t* cand_idx_opt, float* probs, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (qbar == nullptr || kbar == nullptr || probs == nullptr) return RECAP_E_NULL;
  if ((cand_count_opt == nullptr) != (cand_idx_opt == nullptr)) return RECAP_E_NULL;
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(probs) ||
      (cand_count_opt != nullptr && (!aligned16(cand_count_opt) || !aligned16(cand_idx_opt))))
    return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;
  const float sl2 = (float)((double)sm_scale * 1.4426950408889634);
  const int BH = d->batch * d->heads, M = num_blocks(d);
  hipStream_t st = (hipStream_t)stream;
  if (cand_count_opt == nullptr)
    return launched(launch_scores(qbar, kbar, BH, M, d->head_dim, sl2, probs, st));
  return launched(launch_scores_cand(qbar, kbar, BH, M, d->head_dim, sl2, cand_count_opt,
                                     cand_idx_opt, probs, st));
}

int recap_topp_mask_cand(const recap_desc* d, const float* probs, const int32_t* cand_count,
                         const int32_t* cand_idx, const float* top_p_host, int32_t* kept_count,
                         int32_t* kept_idx, uint8_t* mask_opt, float* kept_mass_opt,
                         void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (probs == nullptr || cand_count == nullptr || cand_idx == nullptr ||
      top_p_host == nullptr || kept_count == nullptr || kept_idx == nullptr)
    return RECAP_E_NULL;
  if (!aligned16(probs) || !aligned16(cand_count) || !aligned16(cand_idx) ||
      !aligned16(kept_count) || !aligned16(kept_idx) || (mask_opt && !aligned16(mask_opt)) ||
      (kept_mass_opt && !aligned16(kept_mass_opt)))
    return RECAP_E_ALIGN;
  if (kept_idx == cand_idx || kept_count == cand_count) return RECAP_E_VALUE;
  HeadScalars tp;
  memset(&tp, 0, sizeof(tp));
  for (int h = 0; h < d->heads; ++h) {
    const float p = top_p_host[h];
    if (!(p >= 0.f && p <= 1.f)) return RECAP_E_VALUE;
    tp.v[h] = p;
  }
  if ((s = check_device()) != RECAP_OK) return s;
  return launched(launch_topp(probs, d->batch, d->heads, num_blocks(d), tp, cand_count,
                              cand_idx, kept_count, kept_idx, mask_opt, kept_mass_opt,
                              (hipStream_t)stream));
}

int recap_mean_drift(const recap_desc* d, const float* qbar, const float* kbar,
                     const float* qbar_ref, const float* kbar_ref, float* drift, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (qbar == nullptr || kbar == nullptr || qbar_ref == nullptr || kbar_ref == nullptr ||
      drift == nullptr)
    return RECAP_E_NULL;
  if (!aligned16(qbar) || !aligned16(kbar) || !aligned16(qbar_ref) || !aligned16(kbar_ref) ||
      !aligned16(drift))
    return RECAP_E_ALIGN;
  if ((s = check_device()) != RECAP_OK) return s;
  return launched(launch_mean_drift(qbar, kbar, qbar_ref, kbar_ref, d->batch * d->heads,
                                    num_blocks(d), d->head_dim, drift, (hipStream_t)stream));
}

int recap_block_sparse_attn(const recap_desc* d, const void* q, const void* k, const void* v,
                            const int32_t* kept_count, const int32_t* kept_idx, float sm_scale,
                            const void* residual_opt, const float* res_scale_host, void* out,
                            void* ws, size_t ws_bytes, void* stream) {
  return sparse_impl(d, q, k, v, kept_count, kept_idx, sm_scale, residual_opt, res_scale_host,
                     out, nullptr, ws, ws_bytes, stream);
}

int recap_block_sparse_attn_stats(const recap_desc* d, const void* q, const void* k,
                                  const void* v, const int32_t* kept_count,
                                  const int32_t* kept_idx, float sm_scale,
                                  const void* residual_opt, const float* res_scale_host,
                                  void* out, float* lse_out, void* ws, size_t ws_bytes,
                                  void* stream) {
  if (lse_out == nullptr) return RECAP_E_NULL;
  return sparse_impl(d, q, k, v, kept_count, kept_idx, sm_scale, residual_opt, res_scale_host,
                     out, lse_out, ws, ws_bytes, stream);
}

int recap_dense_attn(const recap_desc* d, const void* q, const void* k, const void* v,
                     float sm_scale, const int32_t* kept_count_opt, const int32_t* kept_idx_opt,
                     void* out, void* residual_out_opt, void* ws, size_t ws_bytes,
                     void* stream) {
  return dense_impl(d, q, k, v, sm_scale, kept_count_opt, kept_idx_opt, out, residual_out_opt,
                    nullptr, nullptr, ws, ws_bytes, stream);
}

int recap_dense_attn_stats(const recap_desc* d, const void* q, const void* k, const void* v,
                           float sm_scale, const int32_t* kept_count_opt,
                           const int32_t* kept_idx_opt, void* out, void* residual_out_opt,
                           float* lse_out, float* kept_mass_out_opt, void* ws,
                           size_t ws_bytes, void* stream) {
  if (lse_out == nullptr) return RECAP_E_NULL;
  return dense_impl(d, q, k, v, sm_scale, kept_count_opt, kept_idx_opt, out, residual_out_opt,
                    lse_out, kept_mass_out_opt, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

constexpr double kLog2eD = 1.4426950408889634;

// Coarse tail over each query block's omitted key blocks (log-mass c_lse [B*H][N], output c_o
// [B*H][N][D], fp32) from the block means of k and v; tws: tail_estimate_bytes(d) of workspace.
hipError_t coarse_tail(const recap_desc* d, const void* q, const void* k, const void* v,
                       const int32_t* count, const int32_t* idx, float sm_scale, bool moments,
                       float* c_lse, float* c_o, void* tws, hipStream_t st) {
  const int M = num_blocks(d), mpad = pooled_pad(d), H = d->heads, D = d->head_dim;
  char* w = (char*)tws;
  float* kbar = (float*)w;
  float* vbar = (float*)(w + pooled_bytes(d));
  char* w16 = w + 2 * pooled_bytes(d);
  bf16_t* kb_hi = (bf16_t*)w16;
  bf16_t* kb_lo = (bf16_t*)(w16 + pooled16_bytes(d));
  bf16_t* vb16 = (bf16_t*)(w16 + 2 * pooled16_bytes(d));
  char* wm = w16 + 3 * pooled16_bytes(d);
  uint32_t* bits = (uint32_t*)wm;
  float* var = (float*)(wm + bits_bytes(d));
  bf16_t* sv16 = (bf16_t*)(wm + bits_bytes(d) + pooled_bytes(d));
  float* cov_part = (float*)(wm + bits_bytes(d) + pooled_bytes(d) + pooled16_bytes(d));
  bf16_t* cov16 = (bf16_t*)((char*)cov_part + cov_part_bytes(d));
  hipError_t e = launch_pool((const bf16_t*)k, (const bf16_t*)v, strides_of(d), d->batch, H,
                             d->seq, D, d->block, kbar, vbar, st);
  if (e == hipSuccess && moments)
    e = launch_tail_stats((const bf16_t*)k, (const bf16_t*)v, strides_of(d), d->batch, H,
                          d->seq, D, d->block, kbar, vbar, var, cov_part,
                          (float)((double)sm_scale / d->seq), cov16, st);
  if (e == hipSuccess)
    e = launch_tail_keys(kbar, vbar, moments ? var : nullptr, 0.5f * sm_scale, d->batch * H, M,
                         D, mpad, kb_hi, kb_lo, vb16, sv16, st);
  if (e == hipSuccess)
    e = launch_kept_bits(count, idx, d->batch * H * M, M, bit_words(d), bits, st);
  if (e != hipSuccess) return e;
  TailParams p;
  memset(&p, 0, sizeof(p));
  p.q = (const bf16_t*)q;
  p.st = strides_of(d);
  p.kb = kb_hi;
  p.kb_lo = kb_lo;
  p.vb = vb16;
  p.H = H;
  p.N = d->seq;
  p.M = M;
  p.block = d->block;
  p.mpad = mpad;
  p.scale_log2 = (float)((double)sm_scale * kLog2eD);
  const int n_last = d->seq - (M - 1) * d->block;
  p.last_bias = (float)log2((double)n_last / d->block);
  p.ln_block = (float)log((double)d->block);
  p.bits = bits;
  p.wbits = bit_words(d);
  p.tail_lse = c_lse;
  p.tail_o = c_o;
  p.sv = moments ? sv16 : nullptr;
  p.cov = moments ? cov16 : nullptr;
  p.BH = d->batch * H;
  return launch_tail(p, d->batch, D, st);
}

// Shared validation of the tail entry points: q, k, v, kept lists, scale, flags, workspace.
int check_tail_args(int op, const recap_desc* d, const void* q, const void* k, const void* v,
                    const int32_t* count, const int32_t* idx, float sm_scale, int flags,
                    const void* ws, size_t ws_bytes) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || count == nullptr || idx == nullptr)
    return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(count) || !aligned16(idx))
    return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  if ((flags & ~RECAP_TAIL_MOMENTS) != 0) return RECAP_E_VALUE;
  return check_workspace(op, d, ws, ws_bytes);
}

// Workspace carving shared by the dense and sparse tail calls (tail_merge_bytes).
struct TailWs {
  float *a_lse, *a_o, *c_lse, *c_o;
  void* est;
};
TailWs carve_tail_ws(const recap_desc* d, void* ws) {
  char* w = (char*)ws;
  TailWs t;
  t.a_lse = (float*)w;
  w += row_bytes(d);
  t.a_o = (float*)w;
  w += row_d_bytes(d);
  t.c_lse = (float*)w;
  w += row_bytes(d);
  t.c_o = (float*)w;
  w += row_d_bytes(d);
  t.est = w;
  return t;
}

void fill_attn(AttnParams& p, const recap_desc* d, const void* q, const void* k,
               const void* v, float sm_scale, const int32_t* count, const int32_t* idx) {
  memset(&p, 0, sizeof(p));
  p.q = (const bf16_t*)q;
  p.k = (const bf16_t*)k;
  p.v = (const bf16_t*)v;
  p.st = strides_of(d);
  p.H = d->heads;
  p.N = d->seq;
  p.M = num_blocks(d);
  p.block = d->block;
  p.npad = p.M * d->block;
  p.scale_log2 = (float)((double)sm_scale * kLog2eD);
  p.count = count;
  p.idx = idx;
}

}  // namespace

extern "C" {

int recap_tail_estimate(const recap_desc* d, const void* q, const void* k, const void* v,
                        const int32_t* kept_count, const int32_t* kept_idx, float sm_scale,
                        int flags, float* tail_lse, float* tail_out, void* ws, size_t ws_bytes,
                        void* stream) {
  int s = check_tail_args(RECAP_OP_TAIL, d, q, k, v, kept_count, kept_idx, sm_scale, flags, ws,
                          ws_bytes);
  if (s != RECAP_OK) return s;
  if (tail_lse == nullptr || tail_out == nullptr) return RECAP_E_NULL;
  if (!aligned16(tail_lse) || !aligned16(tail_out)) return RECAP_E_ALIGN;
  if ((void*)tail_lse == (void*)tail_out) return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;
  return launched(coarse_tail(d, q, k, v, kept_count, kept_idx, sm_scale,
                              (flags & RECAP_TAIL_MOMENTS) != 0, tail_lse, tail_out, ws,
                              (hipStream_t)stream));
}

int recap_dense_attn_tail(const recap_desc* d, const void* q, const void* k, const void* v,
                          float sm_scale, int flags, const int32_t* kept_count,
                          const int32_t* kept_idx, void* out, float* tail_dlse,
                          float* tail_dout, void* ws, size_t ws_bytes, void* stream) {
  int s = check_tail_args(RECAP_OP_DENSE_TAIL, d, q, k, v, kept_count, kept_idx, sm_scale,
                          flags, ws, ws_bytes);
  if (s != RECAP_OK) return s;
  if (out == nullptr || tail_dlse == nullptr || tail_dout == nullptr) return RECAP_E_NULL;
  if (!aligned16(out) || !aligned16(tail_dlse) || !aligned16(tail_dout)) return RECAP_E_ALIGN;
  if (out == q || out == k || out == v || (void*)tail_dout == out ||
      (void*)tail_dout == (void*)tail_dlse)
    return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  const TailWs t = carve_tail_ws(d, ws);
  // dense pass with the kept-block accumulator: the exact tail is the dense sums minus the
  // kept ones (no residual, so no snapshot or flags)
  AttnParams p;
  fill_attn(p, d, q, k, v, sm_scale, kept_count, kept_idx);
  p.out = (bf16_t*)out;
  p.tail_lse = t.a_lse;
  p.tail_o = t.a_o;
  hipError_t e = launch_attention(p, d->batch, d->head_dim, kDenseTail, st);
  if (e == hipSuccess)
    e = coarse_tail(d, q, k, v, kept_count, kept_idx, sm_scale,
                    (flags & RECAP_TAIL_MOMENTS) != 0, t.c_lse, t.c_o, t.est, st);
  if (e == hipSuccess)
    e = launch_tail_combine(0, d->batch, d->heads, d->seq, d->head_dim, strides_of(d), t.a_lse,
                            t.a_o, t.c_lse, t.c_o, nullptr, nullptr, tail_dlse, tail_dout,
                            nullptr, st);
  return launched(e);
}

int recap_block_sparse_attn_tail(const recap_desc* d, const void* q, const void* k,
                                 const void* v, const int32_t* kept_count,
                                 const int32_t* kept_idx, float sm_scale, int flags,
                                 const float* tail_dlse_opt, const float* tail_dout_opt,
                                 void* out, void* ws, size_t ws_bytes, void* stream) {
  int s = check_tail_args(RECAP_OP_SPARSE_TAIL, d, q, k, v, kept_count, kept_idx, sm_scale,
                          flags, ws, ws_bytes);
  if (s != RECAP_OK) return s;
  if (out == nullptr) return RECAP_E_NULL;
  if ((tail_dlse_opt == nullptr) != (tail_dout_opt == nullptr)) return RECAP_E_NULL;
  if (!aligned16(out) || (tail_dlse_opt != nullptr && (!aligned16(tail_dlse_opt) ||
                                                       !aligned16(tail_dout_opt))))
    return RECAP_E_ALIGN;
  if (out == q || out == k || out == v ||
      (tail_dout_opt != nullptr && (const void*)tail_dout_opt == (const void*)out))
    return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  const TailWs t = carve_tail_ws(d, ws);
  AttnParams p;
  fill_attn(p, d, q, k, v, sm_scale, kept_count, kept_idx);
  p.out = (bf16_t*)out;  // not written: the fp32 output goes to the merge
  p.o32_out = t.a_o;
  p.lse_out = t.a_lse;
  hipError_t e = launch_attention(p, d->batch, d->head_dim, kSparse, st);
  if (e == hipSuccess)
    e = coarse_tail(d, q, k, v, kept_count, kept_idx, sm_scale,
                    (flags & RECAP_TAIL_MOMENTS) != 0, t.c_lse, t.c_o, t.est, st);
  if (e == hipSuccess)
    e = launch_tail_combine(1, d->batch, d->heads, d->seq, d->head_dim, strides_of(d), t.a_lse,
                            t.a_o, t.c_lse, t.c_o, tail_dlse_opt, tail_dout_opt, nullptr,
                            nullptr, (bf16_t*)out, st);
  return launched(e);
}

}  // extern "C"

extern "C" {

int recap_mx_quantize(const recap_desc* d, const void* x, int along_tokens, uint8_t* codes,
                      uint8_t* scales, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (x == nullptr || codes == nullptr || scales == nullptr) return RECAP_E_NULL;
  if (!aligned16(x) || !aligned16(codes)) return RECAP_E_ALIGN;
  if (along_tokens != 0 && along_tokens != 1) return RECAP_E_VALUE;
  if ((const void*)codes == x || (const void*)scales == x || (void*)codes == (void*)scales)
    return RECAP_E_VALUE;
  if ((s = check_device()) != RECAP_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  if (along_tokens == 0)
    return launched(launch_mx_rows((const bf16_t*)x, strides_of(d), d->batch, d->heads, d->seq,
                                   d->head_dim, codes, scales, st));
  return launched(launch_mx_cols((const bf16_t*)x, strides_of(d), d->batch, d->heads, d->seq,
                                 d->head_dim, codes, scales, st));
}

int recap_block_sparse_attn_fp8(const recap_desc* d, const void* q, const void* k, const void* v,
                                const int32_t* kept_count, const int32_t* kept_idx,
                                float sm_scale, const void* residual_opt,
                                const float* res_scale_host, void* out, float* lse_out_opt,
                                void* ws, size_t ws_bytes, void* stream) {
  int s = validate_desc(d);
  if (s != RECAP_OK) return s;
  if (q == nullptr || k == nullptr || v == nullptr || kept_count == nullptr ||
      kept_idx == nullptr || out == nullptr)
    return RECAP_E_NULL;
  if (residual_opt != nullptr && res_scale_host == nullptr) return RECAP_E_NULL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) ||
      !aligned16(kept_count) || !aligned16(kept_idx) ||
      (residual_opt != nullptr && !aligned16(residual_opt)) ||
      (lse_out_opt != nullptr && !aligned16(lse_out_opt)))
    return RECAP_E_ALIGN;
  if (!isfinite(sm_scale) || !(sm_scale > 0.f)) return RECAP_E_VALUE;
  if (out == q || out == k || out == v || (residual_opt != nullptr && out == residual_opt))
    return RECAP_E_VALUE;
  MxParams p;
  memset(&p, 0, sizeof(p));
  if (residual_opt != nullptr) {
    for (int h = 0; h < d->heads; ++h) {
      if (!isfinite(res_scale_host[h])) return RECAP_E_VALUE;
      p.res_scale.v[h] = res_scale_host[h];
    }
  }
  if ((s = check_workspace(RECAP_OP_SPARSE_FP8, d, ws, ws_bytes)) != RECAP_OK) return s;
  if ((s = check_device()) != RECAP_OK) return s;

  hipStream_t st = (hipStream_t)stream;
  char* w = (char*)ws;
  uint8_t* q8 = (uint8_t*)w;
  uint8_t* qs = (uint8_t*)(w + fp8_q_bytes(d));
  uint8_t* kt = (uint8_t*)(w + fp8_q_bytes(d) + fp8_qs_bytes(d));
  uint8_t* vt = kt + fp8_tile_bytes(d);
  const int ntile = num_blocks(d) * d->block / 64;
  hipError_t e = launch_mx_rows((const bf16_t*)q, strides_of(d), d->batch, d->heads, d->seq,
                                d->head_dim, q8, qs, st);
  if (e == hipSuccess)
    e = launch_mx_kv_tiles((const bf16_t*)k, (const bf16_t*)v, strides_of(d), d->batch,
                           d->heads, d->seq, d->head_dim, ntile, kt, vt, st);
  if (e != hipSuccess) return launched(e);
  p.q8 = q8;
  p.qs = qs;
  p.kt = kt;
  p.vt = vt;
  p.st = strides_of(d);
  p.H = d->heads;
  p.N = d->seq;
  p.M = num_blocks(d);
  p.block = d->block;
  p.ntile = ntile;
  p.scale_log2 = (float)((double)sm_scale * kLog2eD);
  p.count = kept_count;
  p.idx = kept_idx;
  p.res = (const bf16_t*)residual_opt;
  p.out = (bf16_t*)out;
  p.lse_out = lse_out_opt;
  return launched(launch_attention_mx(p, d->batch, d->head_dim, st));
}

}  // extern "C"
