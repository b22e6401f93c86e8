// Host-side driver for the sanitizer build of the C ABI (AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code only): walks every entry point's validation with
// fake device addresses (never dereferenced: every call below fails validation, or reaches the
// device check and returns RECAP_E_DEVICE where no GPU is present), the descriptor checks
// (stride / overlap arithmetic with extreme values), the workspace sizing of every op at the
// largest accepted shapes, and the status strings. Prints "OK" and exits 0 when every status is
// the expected one.
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "recap.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got_ = (call);                                                            \
    if (got_ != (want)) {                                                               \
      printf("line %d: %s returned %d, expected %d\n", __LINE__, #call, got_, (want));  \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

static void* P(uintptr_t off = 0) { return (void*)(uintptr_t)(0x100000 + off); }

static recap_desc desc(int B = 1, int H = 2, int N = 4096, int D = 64, int blk = 64) {
  recap_desc d;
  memset(&d, 0, sizeof(d));
  d.batch = B;
  d.heads = H;
  d.seq = N;
  d.head_dim = D;
  d.block = blk;
  d.stride_n = D;
  d.stride_h = (int64_t)N * D;
  d.stride_b = (int64_t)H * N * D;
  return d;
}

int main() {
  EXPECT(recap_abi_version(), RECAP_ABI_VERSION);
  for (int s = -20; s <= 2; ++s)
    if (recap_status_string(s) == nullptr || strlen(recap_status_string(s)) == 0) ++failures;

  // descriptors: shapes, strides, overlap arithmetic with extreme values
  size_t n = 0;
  recap_desc d = desc();
  EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &d, &n), RECAP_OK);
  EXPECT(recap_workspace_size(RECAP_OP_SPARSE, nullptr, &n), RECAP_E_NULL);
  EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &d, nullptr), RECAP_E_NULL);
  EXPECT(recap_workspace_size(99, &d, &n), RECAP_E_VALUE);
  EXPECT(recap_workspace_size(-1, &d, &n), RECAP_E_VALUE);
  const int64_t big[] = {INT64_MAX, INT64_MAX - 7, (int64_t)1 << 62, (int64_t)1 << 40, -8, 0, 8,
                         128, 1 << 20, 1 << 24};
  for (int64_t sb : big)
    for (int64_t sh : big)
      for (int64_t sn : big) {
        recap_desc e = desc(3, 5, 1000, 128, 128);
        e.stride_b = sb;
        e.stride_h = sh;
        e.stride_n = sn;
        const int st = recap_workspace_size(RECAP_OP_DENSE_CAPTURE, &e, &n);
        if (st != RECAP_OK && st != RECAP_E_STRIDE) {
          printf("strides %lld %lld %lld: status %d\n", (long long)sb, (long long)sh,
                 (long long)sn, st);
          ++failures;
        }
      }
  const int32_t bad_int[] = {0, -1, INT32_MIN, INT32_MAX};
  for (int32_t x : bad_int) {
    recap_desc e = desc();
    e.batch = x;
    if (x != INT32_MAX) EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
    e = desc();
    e.seq = x;
    if (x != INT32_MAX) EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
    e = desc();
    e.heads = x;
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
    e = desc();
    e.head_dim = x;
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
  }
  {  // B = INT32_MAX: B * H * M beyond the grid limit (no overflow in the product)
    recap_desc e = desc(INT32_MAX, 128, 4096, 64, 64);
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
  }
  {  // N = INT32_MAX: M far beyond the block limit
    recap_desc e = desc(1, 1, INT32_MAX, 64, 64);
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &e, &n), RECAP_E_SHAPE);
  }
  // largest accepted shapes: every op's workspace size computes without overflow
  {
    recap_desc e = desc(1, 128, 8192 * 128, 128, 128);
    for (int op = RECAP_OP_BLOCK_SCORES; op <= RECAP_OP_SPARSE_FP8; ++op) {
      EXPECT(recap_workspace_size(op, &e, &n), RECAP_OK);
      // top-p, sparse (128-token blocks: no end-order table) and plain dense attention need
      // no workspace; every other op does
      const bool none = op == RECAP_OP_TOPP || op == RECAP_OP_SPARSE || op == RECAP_OP_DENSE;
      if (none != (n == 0)) ++failures;
    }
    recap_desc f = desc(1024, 128, 8192 * 64, 64, 64);  // B * H * M = 2^30: accepted
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &f, &n), RECAP_OK);
    f.batch = 1025;
    EXPECT(recap_workspace_size(RECAP_OP_SPARSE, &f, &n), RECAP_E_SHAPE);
  }

  // every entry point: NULL, alignment, value checks, then the device check
  d = desc();
  size_t ws_sc = 0, ws_sp = 0, ws_dc = 0, ws_t = 0, ws_m = 0, ws_8 = 0;
  recap_workspace_size(RECAP_OP_BLOCK_SCORES, &d, &ws_sc);
  recap_workspace_size(RECAP_OP_SPARSE, &d, &ws_sp);
  recap_workspace_size(RECAP_OP_DENSE_CAPTURE, &d, &ws_dc);
  recap_workspace_size(RECAP_OP_TAIL, &d, &ws_t);
  recap_workspace_size(RECAP_OP_SPARSE_TAIL, &d, &ws_m);
  recap_workspace_size(RECAP_OP_SPARSE_FP8, &d, &ws_8);
  const float pp[2] = {0.9f, 0.5f}, bad_p[2] = {0.9f, NAN}, cc[2] = {1.0f, INFINITY};
  EXPECT(recap_block_scores(&d, P(), P(4096), 0.125f, (float*)P(8192), P(1 << 20), ws_sc, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_block_scores(&d, P(2), P(4096), 0.125f, (float*)P(8192), P(1 << 20), ws_sc, nullptr),
         RECAP_E_ALIGN);
  EXPECT(recap_block_scores(&d, P(), P(4096), NAN, (float*)P(8192), P(1 << 20), ws_sc, nullptr),
         RECAP_E_VALUE);
  EXPECT(recap_block_scores(&d, P(), P(4096), 0.125f, (float*)P(8192), P(1 << 20), ws_sc - 1,
                            nullptr),
         RECAP_E_WORKSPACE);
  EXPECT(recap_block_scores_noalloc(&d, P(), P(4096), 0.125f, (float*)P(8192), nullptr),
         RECAP_E_DEVICE);
  {
    recap_desc e = desc(1, 64, 75600, 128, 64);  // pooled means beyond the fixed scratch
    EXPECT(recap_block_scores_noalloc(&e, P(), P(4096), 0.125f, (float*)P(8192), nullptr),
           RECAP_E_WORKSPACE);
  }
  EXPECT(recap_topp_mask(&d, (float*)P(), pp, (int32_t*)P(4096), (int32_t*)P(8192), nullptr,
                         nullptr, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_topp_mask(&d, (float*)P(), bad_p, (int32_t*)P(4096), (int32_t*)P(8192), nullptr,
                         nullptr, nullptr),
         RECAP_E_VALUE);
  EXPECT(recap_topp_mask(&d, (float*)P(), nullptr, (int32_t*)P(4096), (int32_t*)P(8192), nullptr,
                         nullptr, nullptr),
         RECAP_E_NULL);
  EXPECT(recap_block_sparse_attn(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                 (int32_t*)P(16384), 0.125f, P(20480), pp, P(24576), P(1 << 20),
                                 ws_sp, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_block_sparse_attn(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                 (int32_t*)P(16384), 0.125f, P(20480), cc, P(24576), P(1 << 20),
                                 ws_sp, nullptr),
         RECAP_E_VALUE);
  EXPECT(recap_block_sparse_attn(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                 (int32_t*)P(16384), 0.125f, nullptr, nullptr, P(), P(1 << 20),
                                 ws_sp, nullptr),
         RECAP_E_VALUE);  // out aliases q
  EXPECT(recap_block_sparse_attn_stats(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                       (int32_t*)P(16384), 0.125f, nullptr, nullptr, P(24576),
                                       (float*)P(28672), P(1 << 20), ws_sp, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_dense_attn(&d, P(), P(4096), P(8192), 0.125f, (int32_t*)P(12288),
                          (int32_t*)P(16384), P(24576), P(28672), P(1 << 20), ws_dc, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_dense_attn(&d, P(), P(4096), P(8192), 0.125f, nullptr, nullptr, P(24576),
                          P(28672), P(1 << 20), ws_dc, nullptr),
         RECAP_E_NULL);  // capture needs the lists
  EXPECT(recap_dense_attn_stats(&d, P(), P(4096), P(8192), 0.125f, (int32_t*)P(12288),
                                (int32_t*)P(16384), P(24576), nullptr, (float*)P(28672),
                                (float*)P(32768), P(1 << 20), ws_dc, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_block_means(&d, P(), P(4096), (float*)P(8192), (float*)P(12288), nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_scores_from_means(&d, (float*)P(), (float*)P(4096), 0.125f, nullptr, nullptr,
                                 (float*)P(8192), nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_topp_mask_cand(&d, (float*)P(), (int32_t*)P(4096), (int32_t*)P(8192), pp,
                              (int32_t*)P(12288), (int32_t*)P(16384), nullptr, nullptr, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_mean_drift(&d, (float*)P(), (float*)P(4096), (float*)P(8192), (float*)P(12288),
                          (float*)P(16384), nullptr),
         RECAP_E_DEVICE);
  for (int fl : {0, RECAP_TAIL_MOMENTS, 2, -1}) {
    const int want = (fl == 0 || fl == RECAP_TAIL_MOMENTS) ? RECAP_E_DEVICE : RECAP_E_VALUE;
    EXPECT(recap_tail_estimate(&d, P(), P(4096), P(8192), (int32_t*)P(12288), (int32_t*)P(16384),
                               0.125f, fl, (float*)P(20480), (float*)P(24576), P(1 << 20), ws_t,
                               nullptr),
           want);
    EXPECT(recap_dense_attn_tail(&d, P(), P(4096), P(8192), 0.125f, fl, (int32_t*)P(12288),
                                 (int32_t*)P(16384), P(20480), (float*)P(24576), (float*)P(28672),
                                 P(1 << 20), ws_m, nullptr),
           want);
    EXPECT(recap_block_sparse_attn_tail(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                        (int32_t*)P(16384), 0.125f, fl, nullptr, nullptr,
                                        P(20480), P(1 << 20), ws_m, nullptr),
           want);
  }
  EXPECT(recap_block_sparse_attn_fp8(&d, P(), P(4096), P(8192), (int32_t*)P(12288),
                                     (int32_t*)P(16384), 0.125f, nullptr, nullptr, P(20480),
                                     nullptr, P(1 << 20), ws_8, nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_mx_quantize(&d, P(), 0, (uint8_t*)P(4096), (uint8_t*)P(8192), nullptr),
         RECAP_E_DEVICE);
  EXPECT(recap_mx_quantize(&d, P(), 2, (uint8_t*)P(4096), (uint8_t*)P(8192), nullptr),
         RECAP_E_VALUE);

  if (failures) {
    printf("FAILED %d\n", failures);
    return 1;
  }
  printf("OK\n");
  return 0;
}
