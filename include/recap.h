/*
 * recap.h -- C ABI of the block-sparse top-p attention library for MI355X (gfx950).
 *
 * The library implements the attention-layer hot path of training-free block-sparse
 * attention for video diffusion transformers, with a RECAP-style cached-residual epilogue:
 *
 *   1. recap_block_scores  mean-pool Q and K over token blocks and score every block pair
 *                          with a row softmax (mask prediction);
 *   2. recap_topp_mask     keep, per query block, the fewest key blocks whose probability
 *                          mass reaches the head's threshold p_h (top-p);
 *   3. recap_block_sparse_attn
 *                          online-softmax attention over the kept blocks only, with an
 *                          optional fused epilogue  O' = O + c_h * R;
 *   4. recap_dense_attn    dense refresh over all keys, optionally capturing the residual
 *                          R = O_dense - O_sparse on a given kept set.
 * Beside them: row statistics (*_stats), mask reuse across steps, RECAP's tail
 * reconstruction (*_tail: a coarse estimate of the omitted attention from block means plus a
 * discrepancy cached at the dense refresh, merged with the sparse part by log-mass), and an
 * FP8 variant of the sparse attention products (*_fp8, MXFP8).
 *
 * Sources (page title, section / figure):
 *   RECAP: Reciprocal Sparse Attention and Hierarchical Caching for Efficient Video Diffusion
 *     (paperpeel.com/paper/2610.26244): Sec. 3.2 (block means as coarse estimates; cached
 *     dense refinement added to the fresh estimate, error d_h - d_t vanishing at the refresh
 *     step; state kept per layer and head), Sec. 4.1 (dense refreshes vs. block-sparse
 *     "selected interactions"), Sec. 1 and 5 (fresh sparse statistics regulate how strongly
 *     the aging refinement is applied), Sec. 2 (dense-minus-window residuals).
 *   The same title at thelatestinai.com/papers/2610.26244: first abstract (online top-p mask
 *     prediction with per-head thresholds), third abstract (top-p selection).
 *   CalibAtt (thelatestinai.com/papers/2603.05503): Fig. 5 (threshold the top key blocks of
 *     each query block), Table S6 and Fig. S14 (query x key block sizes).
 *
 * Conventions shared by every entry point
 *   - Tensors q, k, v, out, residual are bf16 device arrays addressed as
 *       base + b*stride_b + h*stride_h + n*stride_n + d      (element strides, d contiguous),
 *     so both [B,H,N,D] and [B,N,H,D] storage work. Bases must be 16-byte aligned, every
 *     stride a positive multiple of 8 elements, stride_n below 2^24 elements (the kernels
 *     address one key tile's rows as 32-bit byte offsets), and no two (b, h, n) rows may
 *     overlap.
 *   - Blocks: b = desc.block; M = ceil(N / b). Block j holds tokens [j*b, min(N,(j+1)*b)); the
 *     same partition is used for queries and keys. The last block may be short: it is pooled
 *     over its valid tokens, padded keys carry no weight, padded query rows are not written.
 *   - probs is fp32 [B,H,M,M] contiguous; kept_count int32 [B,H,M]; kept_idx int32 [B,H,M,M]
 *     (row r holds kept_count[r] key-block indices, ascending; later entries unspecified);
 *     mask uint8 [B,H,M,M] (1 = kept); kept_mass fp32 [B,H,M].
 *   - Host arrays (top_p_host, res_scale_host) have H entries and are copied into the kernel
 *     arguments before the call returns.
 *   - Ownership: the caller owns every buffer. The library allocates no device memory;
 *     scratch comes from the caller's workspace (size from recap_workspace_size), which must
 *     stay untouched until the stream has run the call. No pointer is kept after returning.
 *   - Streams: `stream` is a hipStream_t passed as void* (NULL = the null stream). Calls are
 *     asynchronous and never synchronise the host.
 *   - Errors: every argument is validated before the first HIP call; on a validation error
 *     nothing is launched and no buffer is written. RECAP_E_DEVICE means no usable gfx950
 *     device is current; RECAP_E_LAUNCH means a kernel launch failed (outputs undefined).
 *   - Thread safety: calls may come from several host threads; the only global state is a
 *     per-device property cache filled once.
 */
#ifndef RECAP_H
#define RECAP_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RECAP_ABI_VERSION 7 /* 2: *_stats; 3: mask reuse; 4: coarse tail; 5: FP8; 6: no-alloc scores;
                             7: tail flags (moment refinements) */
#define RECAP_MAX_HEADS 128   /* per-head host arrays are passed by value to the kernels */
#define RECAP_MAX_BLOCKS 8192 /* M = ceil(N / block) upper bound (top-p sorts a row in LDS) */
/* Size of the fixed device scratch of recap_block_scores_noalloc (64 MiB per device): the
 * call needs 2 * B * H * M * D * 4 bytes (each of the two rounded up to 256 bytes). */
#define RECAP_NOALLOC_SCRATCH_BYTES (64u << 20)

typedef struct recap_desc {
  int32_t batch;    /* B >= 1 */
  int32_t heads;    /* 1 <= H <= RECAP_MAX_HEADS */
  int32_t seq;      /* N >= 1 tokens; queries and keys share it (self-attention) */
  int32_t head_dim; /* D in {64, 128} */
  int32_t block;    /* b in {64, 128}; M = ceil(N / b) <= RECAP_MAX_BLOCKS */
  int32_t reserved; /* must be 0 */
  int64_t stride_b; /* element strides of q, k, v, out and residual (all share them) */
  int64_t stride_h;
  int64_t stride_n;
} recap_desc;

enum recap_status {
  RECAP_OK = 0,
  RECAP_E_NULL = -1,      /* a required pointer is NULL */
  RECAP_E_SHAPE = -2,     /* B, H, N, D or block out of the supported set */
  RECAP_E_STRIDE = -3,    /* a stride is not a positive multiple of 8, >= 2^24 (stride_n), or overlaps */
  RECAP_E_ALIGN = -4,     /* a base pointer is not 16-byte aligned */
  RECAP_E_VALUE = -5,     /* a scalar or host-array value is out of range (NaN, p not in [0,1]) */
  RECAP_E_WORKSPACE = -6, /* workspace missing or smaller than recap_workspace_size */
  RECAP_E_DEVICE = -7,    /* no current HIP device, or it is not gfx950 */
  RECAP_E_LAUNCH = -8     /* a kernel launch failed */
};

enum recap_op {
  RECAP_OP_BLOCK_SCORES = 0,
  RECAP_OP_TOPP = 1,
  RECAP_OP_SPARSE = 2,
  RECAP_OP_DENSE = 3,         /* dense refresh without capture */
  RECAP_OP_DENSE_CAPTURE = 4, /* dense refresh that also writes the residual */
  RECAP_OP_TAIL = 5,          /* recap_tail_estimate */
  RECAP_OP_DENSE_TAIL = 6,    /* recap_dense_attn_tail */
  RECAP_OP_SPARSE_TAIL = 7,   /* recap_block_sparse_attn_tail */
  RECAP_OP_SPARSE_FP8 = 8     /* recap_block_sparse_attn_fp8 */
};

/* Version of this ABI (RECAP_ABI_VERSION of the built library). */
int recap_abi_version(void);

/* Static English text for a status code; never NULL. */
const char* recap_status_string(int status);

/* Bytes of device workspace that entry point `op` needs for descriptor `d`, written to
 * *bytes; zero (top-p, plain dense attention, sparse attention with 128-token blocks) means
 * the call uses none and ws may be NULL. Sparse attention with 64-token blocks needs at most
 * 4 KB. Returns RECAP_OK, RECAP_E_NULL or the descriptor's validation error. Pure host
 * computation: makes no HIP call. */
int recap_workspace_size(int op, const recap_desc* d, size_t* bytes);

/* Mask prediction, part 1 (RECAP Sec. 3.2 block means; first abstract of the RECAP page at
 * thelatestinai.com: online top-p mask prediction).
 *   Q̄_i = mean of the valid query tokens of block i, K̄_j likewise (fp32 accumulation);
 *   probs[b,h,i,:] = softmax_j(sm_scale * Q̄_i . K̄_j) in fp32.
 * q, k: bf16 device tensors (layout above). sm_scale: finite and > 0 (1/sqrt(D) typical).
 * probs: fp32 device [B,H,M,M], written in full. ws: device workspace of at least
 * recap_workspace_size(RECAP_OP_BLOCK_SCORES) bytes, 256-byte aligned. */
int recap_block_scores(const recap_desc* d, const void* q, const void* k, float sm_scale,
                       float* probs, void* ws, size_t ws_bytes, void* stream);

/* recap_block_scores for callers that cannot allocate device memory or pass a workspace
 * (code recorded in a HIP graph, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as recap_block_scores, bit for bit; the pooled means go
 * to a fixed device scratch array of RECAP_NOALLOC_SCRATCH_BYTES that the library holds on
 * each device it runs on, from the library's load until the process ends. The call allocates
 * nothing (no hipMalloc, hipFree or allocating library routine); its first call on a device
 * looks up that device's scratch address.
 * Errors: as recap_block_scores, and RECAP_E_WORKSPACE when the call would need more than
 * RECAP_NOALLOC_SCRATCH_BYTES (2 * B*H*M*D*4 bytes; 48.4 MB at B=1, H=40, M=1182, D=128).
 * All calls on one device share its scratch, and every call rewrites what it reads: calls
 * whose execution overlaps on one device (concurrent streams, or host threads on different
 * streams) race on the scratch and give undefined results. Calls on one stream are ordered
 * and safe. */
int recap_block_scores_noalloc(const recap_desc* d, const void* q, const void* k,
                               float sm_scale, float* probs, void* stream);

/* Mask prediction, part 2: top-p selection per query-block row (thelatestinai.com RECAP page,
 * first and third abstracts; CalibAtt Fig. 5). Key blocks are ordered by probability,
 * descending, equal values by lower index first; k* is the smallest k whose running mass
 * reaches p_h (inclusive), or M when p_h >= 1 or when no prefix reaches p_h; the first k*
 * ordered blocks are kept. The selection is the one an fp64 running mass over the fp32 probs
 * gives (fp32 sums decide where they are farther from p than their error bound, fp64 sums
 * elsewhere). probs: fp32 device [B,H,M,M]. top_p_host: host array of H values in [0, 1].
 * kept_count, kept_idx: int32 device outputs (kept indices ascending). mask_opt (uint8
 * [B,H,M,M]) and kept_mass_opt (fp32 [B,H,M], mass of the kept set, summed in fp32 or fp64
 * in an unspecified order) may be NULL. */
int recap_topp_mask(const recap_desc* d, const float* probs, const float* top_p_host,
                    int32_t* kept_count, int32_t* kept_idx, uint8_t* mask_opt,
                    float* kept_mass_opt, void* stream);

/* Block-sparse attention over the kept blocks (RECAP Sec. 4.1 "selected interactions") with
 * an optional fused residual epilogue (RECAP Sec. 3.2):
 *   O_t = sum_u softmax_u(sm_scale * Q_t . K_u) V_u over the valid tokens u of the kept key
 *         blocks of t's query block; then O_t += c_h * R_t when residual_opt is given.
 * fp32 online softmax, bf16 MFMA products, fp32 accumulation, bf16 (RNE) output.
 * kept_count/kept_idx: int32 device lists as written by recap_topp_mask (indices outside
 * [0, M) are clamped; a row with count 0 outputs zeros before the epilogue).
 * residual_opt: bf16 device tensor in the q/out layout, or NULL. res_scale_host: host array
 * of H finite scales c_h, required iff residual_opt is not NULL. out: bf16 device tensor,
 * must not alias q, k, v or the residual. ws: recap_workspace_size(RECAP_OP_SPARSE) bytes
 * (with 64-token blocks, pairs of query blocks share work-groups and the call first writes
 * there the order in which the launch's last work-groups take their pairs: the longest kept
 * lists first, so that the launch does not end on long walks). */
int recap_block_sparse_attn(const recap_desc* d, const void* q, const void* k, const void* v,
                            const int32_t* kept_count, const int32_t* kept_idx, float sm_scale,
                            const void* residual_opt, const float* res_scale_host, void* out,
                            void* ws, size_t ws_bytes, void* stream);

/* Dense refresh (RECAP Sec. 4.1) over all N keys, written to out. When residual_out_opt is
 * given, the kept lists are required and the call also writes the residual
 *   R = O_dense - O_sparse
 * with O_sparse the block-sparse output on the same inputs and kept set (RECAP Sec. 3.2:
 * the discrepancy cached at the refresh step; Sec. 2: dense-minus-window residuals), in bf16.
 * The kept blocks' products are also summed on their own, under the running max of the dense
 * pass; a query block whose kept weights underflow against that max (sum below 2^-64) has
 * its sparse output recomputed over its kept list alone. With every block kept R is exactly
 * zero. ws: recap_workspace_size(RECAP_OP_DENSE) bytes, or RECAP_OP_DENSE_CAPTURE when
 * capturing. */
int recap_dense_attn(const recap_desc* d, const void* q, const void* k, const void* v,
                     float sm_scale, const int32_t* kept_count_opt, const int32_t* kept_idx_opt,
                     void* out, void* residual_out_opt, void* ws, size_t ws_bytes,
                     void* stream);

/* Row statistics of the attention computed above, written from the softmax state of the same
 * pass (the GSRS abstract on the RECAP page at thelatestinai.com: exact attention weights
 * obtained inside the flash-attention computation; the DFSAttn page "Ride the Wave":
 * attention recall of a block-sparse mask). Both outputs are fp32 device arrays indexed
 * [b, h, t] (contiguous [B,H,N], 16-byte aligned), one value per query token t < N:
 *   lse_out[b,h,t]       = ln sum_u exp(sm_scale * Q_t . K_u) over the keys u the call attends
 *                          (kept key blocks for the sparse call, all N keys for the dense
 *                          call); -inf for a row with an empty kept list;
 *   kept_mass_out[b,h,t] = sum over the kept keys u of softmax_u(sm_scale * Q_t . K_u) taken
 *                          over all N keys: the share of the dense attention mass the kept set
 *                          holds, exp(lse_kept - lse_dense), in [0, 1].
 * The weights behind both are the bf16-rounded ones the products use.
 * recap_block_sparse_attn_stats: as recap_block_sparse_attn, plus lse_out (required).
 * recap_dense_attn_stats: as recap_dense_attn, plus lse_out (required) and kept_mass_out
 * (optional; needs the kept lists, and then the RECAP_OP_DENSE_CAPTURE workspace even
 * without residual_out). */
int recap_block_sparse_attn_stats(const recap_desc* d, const void* q, const void* k,
                                  const void* v, const int32_t* kept_count,
                                  const int32_t* kept_idx, float sm_scale,
                                  const void* residual_opt, const float* res_scale_host,
                                  void* out, float* lse_out, void* ws, size_t ws_bytes,
                                  void* stream);
int recap_dense_attn_stats(const recap_desc* d, const void* q, const void* k, const void* v,
                           float sm_scale, const int32_t* kept_count_opt,
                           const int32_t* kept_idx_opt, void* out, void* residual_out_opt,
                           float* lse_out, float* kept_mass_out_opt, void* ws,
                           size_t ws_bytes, void* stream);

/* Mask reuse across steps (the GSRS abstract on the RECAP page at thelatestinai.com: blocks
 * selected early keep most of the attention weight at later steps, so later searches can be
 * restricted to an earlier candidate set; RECAP Sec. 2, related work: early-step block indices
 * reused at later denoising steps). Four building blocks; the caller owns the policy.
 *
 * recap_block_means: the block means of recap_block_scores part 1 (RECAP Sec. 3.2) written to
 *   qbar, kbar: fp32 device [B,H,M,D], contiguous, distinct.
 * recap_scores_from_means: recap_block_scores part 2 from given means. Without candidate lists
 *   it writes the full rows of probs [B,H,M,M]. With them (int32 [B,H,M] counts and
 *   [B,H,M,M] lists of ascending key-block indices, as recap_topp_mask writes; both or neither)
 *   row i holds the softmax over its n_i candidates only,
 *     probs[b,h,i,r] = softmax_r(sm_scale * Q̄_i . K̄_{cand[r]}),  r < n_i,
 *   at the candidate positions r; entries past n_i are unspecified.
 * recap_topp_mask_cand: top-p (as recap_topp_mask) over each row's candidate distribution
 *   (positions r < n_i of probs); the kept lists hold block indices cand[r] (ascending), the
 *   optional mask is over blocks (0 outside the kept set), kept_mass is the candidate mass kept.
 *   Ties: lower position = lower block index first. kept lists must not alias the candidates.
 * recap_mean_drift: drift[b,h,0] = ||Q̄ - Q̄_ref||_F / ||Q̄_ref||_F and drift[b,h,1] likewise
 *   for K̄, fp32 device [B,H,2] (sums in fp64; +inf when the reference is zero and the means
 *   are not). */
int recap_block_means(const recap_desc* d, const void* q, const void* k, float* qbar,
                      float* kbar, void* stream);
int recap_scores_from_means(const recap_desc* d, const float* qbar, const float* kbar,
                            float sm_scale, const int32_t* cand_count_opt,
                            const int32_t* cand_idx_opt, float* probs, void* stream);
int recap_topp_mask_cand(const recap_desc* d, const float* probs, const int32_t* cand_count,
                         const int32_t* cand_idx, const float* top_p_host, int32_t* kept_count,
                         int32_t* kept_idx, uint8_t* mask_opt, float* kept_mass_opt,
                         void* stream);
int recap_mean_drift(const recap_desc* d, const float* qbar, const float* kbar,
                     const float* qbar_ref, const float* kbar_ref, float* drift, void* stream);

/* RECAP's attention-level reconstruction of the omitted tail (paperpeel.com RECAP Sec. 3.2):
 * a fresh coarse estimate of the attention over the key blocks a query block omits, from block
 * means, plus the discrepancy d the estimate leaves, taken exactly at a dense refresh and
 * cached; at a sparse step the tail is estimated again and d added (y = coarse + d, whose
 * error d_h - d_t vanishes at the refresh step), and the result is merged with the sparse
 * attention by log-mass. `flags` selects the estimate: 0 for the zeroth-order block-mean one,
 * RECAP_TAIL_MOMENTS for the page's two moment refinements (key variance refines the
 * log-mass at second order, after COBS; the pooled value-key covariance refines the value at
 * first order, after PISA's shared first-order value compensation; Sec. 3.2 and Sec. 2). The
 * page gives no formulas; the reading implemented (cumulant expansion about the block mean):
 *   block log-mass  ln n_j + sm_scale Q_t.K̄_j + (sm_scale^2 / 2) sum_d Q_{t,d}^2 Var_j(k_d)
 *     with Var_j the per-dimension variance of the block's keys (population form, the diagonal
 *     of the block's key covariance);
 *   output          sum_j w_tj V̄_j / sum_j w_tj + sm_scale C Q_t
 *     with C = (1/N) sum_j sum_{u in j} (v_u - V̄_j)(k_u - K̄_j)^T the pooled within-block
 *     value-key covariance of the head (rows: value dimension), one matrix for every block.
 * On the GPU the variance term is one more product per pooled-key tile, of bf16(Q^2) with
 * bf16((sm_scale / 2) Var) (relative error within 2^-8 of the term), and C Q is a bf16 product
 * of bf16((sm_scale / N) C) with Q (fp32 statistics and sums). Other flag bits:
 * RECAP_E_VALUE. A refresh and the sparse steps that use its discrepancy must pass the same
 * flags.
 *
 * Coarse tail of query token t in query block i, over the key blocks j outside i's kept set,
 * with n_j the token count of block j and K̄_j, V̄_j block means (fp32 pooling; K̄ then held
 * as a bf16 pair hi + lo, about 16 significant bits, V̄ as bf16):
 *   lse_bar_t = ln sum_j n_j exp(sm_scale * Q_t . K̄_j)           (-inf when i keeps all blocks)
 *   o_bar_t   = sum_j n_j exp(sm_scale * Q_t . K̄_j) V̄_j / sum_j n_j exp(...)   (0 when empty)
 * computed like attention over the pooled keys (bf16 products, fp32 sums).
 * Exact tail at a refresh: lse_T_t = ln sum_u exp(sm_scale * Q_t . K_u) and o_T_t the softmax
 * attention output over the tokens u of those blocks, taken from the dense pass as its sums
 * minus the kept blocks' sums (same running maximum).
 * Discrepancy: d_lse = lse_T - lse_bar (0 when both are -inf), d_o = o_T - o_bar.
 * Merge at a sparse step with the block-sparse output O_s of log-sum-exp lse_s:
 *   l = lse_bar + d_lse, o = o_bar + d_o (d omitted: coarse alone),
 *   out = w O_s + (1 - w) o,  w = 1 / (1 + exp(l - lse_s))  (w = 1 when l = -inf).
 *
 * recap_tail_estimate: the coarse tail alone. tail_lse fp32 [B,H,N], tail_out fp32 [B,H,N,D]
 *   (contiguous, distinct). ws: recap_workspace_size(RECAP_OP_TAIL).
 * recap_dense_attn_tail: dense refresh (out as recap_dense_attn) that also writes the
 *   discrepancy on the given kept set: tail_dlse fp32 [B,H,N] and tail_dout fp32 [B,H,N,D]
 *   (contiguous; fp32 because d_o is a difference of tail outputs, as large as the values, and
 *   its rounding would enter every later merge; neither may alias out). ws: RECAP_OP_DENSE_TAIL.
 * recap_block_sparse_attn_tail: block-sparse attention merged with the coarse tail plus the
 *   cached discrepancy (tail_dlse_opt and tail_dout_opt, both or neither), out bf16.
 *   ws: RECAP_OP_SPARSE_TAIL. With the refresh's inputs and kept lists it reproduces the
 *   dense output (up to rounding).
 * Kept lists as for recap_block_sparse_attn (indices clamped into [0, M)). */
#define RECAP_TAIL_MOMENTS 1 /* flags of the tail entry points: the moment refinements */
int recap_tail_estimate(const recap_desc* d, const void* q, const void* k, const void* v,
                        const int32_t* kept_count, const int32_t* kept_idx, float sm_scale,
                        int flags, float* tail_lse, float* tail_out, void* ws, size_t ws_bytes,
                        void* stream);
int recap_dense_attn_tail(const recap_desc* d, const void* q, const void* k, const void* v,
                          float sm_scale, int flags, const int32_t* kept_count,
                          const int32_t* kept_idx, void* out, float* tail_dlse,
                          float* tail_dout, void* ws, size_t ws_bytes, void* stream);
int recap_block_sparse_attn_tail(const recap_desc* d, const void* q, const void* k,
                                 const void* v, const int32_t* kept_count,
                                 const int32_t* kept_idx, float sm_scale, int flags,
                                 const float* tail_dlse_opt, const float* tail_dout_opt,
                                 void* out, void* ws, size_t ws_bytes, void* stream);

/* FP8 variant of the block-sparse attention products (the RECAP page at thelatestinai.com,
 * second abstract: FP8 quantisation with fused kernels; the format is not given there). Format
 * (OCP microscaling, MXFP8): E4M3 elements (1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits; largest finite 448) and one E8M0 scale 2^E per block of 32 consecutive elements along
 * a product's contraction dimension, E = floor(log2(max |x|)) - 7 clamped to [-127, 127]
 * (-127 for an all-zero block), elements = round-to-nearest-even of x / 2^E.
 *
 * recap_block_sparse_attn_fp8: recap_block_sparse_attn (and recap_block_sparse_attn_stats
 *   when lse_out_opt is given) with Q and K quantised per token in blocks of 32 head dims, V per
 *   channel in blocks of 32 tokens counted from token 0, the attention weights per row in
 *   blocks of 32 keys with the block's exponent chosen from its largest weight, and both
 *   products on the FP8 matrix cores with fp32 accumulation; the row sum adds the rounded
 *   weights. The inputs stay bf16; the library writes the FP8 copies to the workspace
 *   (recap_workspace_size(RECAP_OP_SPARSE_FP8)) on every call. Same arguments, layouts and
 *   errors as recap_block_sparse_attn; the result is within FP8 rounding of attention on the
 *   quantised Q, K, V.
 * recap_mx_quantize: the MXFP8 encoding of a bf16 tensor x (q/k/v layout) alone. along_tokens
 *   = 0: blocks of 32 head dims per token, scales uint8 [B,H,N,D/32]; along_tokens = 1: blocks
 *   of 32 tokens per channel, scales uint8 [B,H,ceil(N/32),D]. codes: uint8 [B,H,N,D]
 *   contiguous (E4M3 bit patterns), 16-byte aligned; scale bytes are E + 127. */
int recap_block_sparse_attn_fp8(const recap_desc* d, const void* q, const void* k, const void* v,
                                const int32_t* kept_count, const int32_t* kept_idx,
                                float sm_scale, const void* residual_opt,
                                const float* res_scale_host, void* out, float* lse_out_opt,
                                void* ws, size_t ws_bytes, void* stream);
int recap_mx_quantize(const recap_desc* d, const void* x, int along_tokens, uint8_t* codes,
                      uint8_t* scales, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RECAP_H */
