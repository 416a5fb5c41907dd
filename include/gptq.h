/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer quantizer, libgptq.so.
 *
 * The library quantizes the weights of one linear layer W [d_out x d_in] with
 * GPTQ: a Hessian from calibration activations, damping of its diagonal, an
 * optional column order by descending diag(H), the upper Cholesky factor of
 * H^-1, and a column-by-column min-max group quantization whose rounding
 * error is pushed onto the columns not yet quantized, 128 columns at a time
 * with one lazy update of the rest.
 *
 * Sources: the GPTQ practice page at m.lqnn.cn/news/117696, section 2.1 (the
 * OBQ step and the Hessian from calibration activations), section 2.2 (fixed
 * order, lazy batch updates, Cholesky of H^-1), section 3.3 (bits,
 * group_size, desc_act, damp_percent); the tutorial page "大模型压缩量化技术：
 * GPTQ 与 AWQ 原理详解 + Python 实战教程", section 二 (the min-max grid).
 *
 * Conventions shared by every call:
 *  - Pointers are device pointers owned by the caller, except out_host in
 *    gptq_layer_error, which is host memory.  The library allocates no device
 *    memory; scratch memory comes in through ws/ws_bytes, sized by the
 *    matching *_workspace_size query.  Workspaces need 256-byte alignment
 *    (any hipMalloc / torch allocation satisfies this).
 *  - The library keeps no state between calls (no handles, no globals) and
 *    reads no environment variables: every option is an argument.  The one
 *    exception is gptq_hessian_accumulate_noalloc, which keeps per device the
 *    address of its static scratch array.
 *  - All work is enqueued on stream s, in stream order: it starts after the
 *    work already on s and is complete, as seen from s, before anything
 *    enqueued on s later.  Only gptq_prepare_hinv and gptq_layer_error
 *    synchronize s (to read one device flag or scalar).
 *  - Argument errors return GPTQ_ERR_INVALID_ARG (or GPTQ_ERR_WORKSPACE)
 *    before anything is enqueued.  HIP failures return GPTQ_ERR_HIP.
 *  - Layouts are row-major.  Columns of W are input channels.  X is
 *    token-major [n_tokens x d_in].
 *  - Calls on distinct buffers and streams are independent (reentrant).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GPTQ_F32 = 0, GPTQ_F16 = 1, GPTQ_BF16 = 2 } gptq_dtype;

typedef enum {
  GPTQ_OK = 0,
  GPTQ_ERR_INVALID_ARG = -1,
  GPTQ_ERR_NOT_PD = -2,      /* damped Hessian not positive definite: raise damp_percent */
  GPTQ_ERR_HIP = -3,
  GPTQ_ERR_WORKSPACE = -4,   /* workspace missing or smaller than the query returns */
  GPTQ_ERR_UNSUPPORTED = -5  /* a valid option this library does not implement */
} gptq_status;

/* The quantizer's options, as the pages' config objects name them
 * (practice page section 3.3; the ms-swift review page's GptqConfig).
 *  bits          2..8 (the code range is [0, 2^bits - 1])
 *  group_size    columns sharing one scale/zero (consecutive in processing
 *                order); -1 = one group per row.  Must divide block_size, or
 *                be a multiple of it, or be -1; in-block groups must be a
 *                multiple of 4.
 *  block_size    lazy-batch width; this library supports 128 only.
 *  damp_percent  lambda = damp_percent * mean(diag H) is added to diag(H).
 *  desc_act      0/1: process columns by descending diag(H).
 *  sym           0 = asymmetric min-max grid: scale = (max - min)/maxq,
 *                zero = rint(-min/scale).  1 = symmetric grid (the ms-swift
 *                review page's sym=True; no formula is given, the plainest
 *                reading is used): m = max(|min|, |max|), scale = 2m/maxq,
 *                zero = (maxq + 1)/2 (scale 1 for an all-zero group).
 *  per_block_steps  0 (default): with groups inside the block, each block's
 *                column loop runs in the same launch as the previous block's
 *                lazy update of the later columns.  1: one launch per step
 *                (column loop, then lazy update).  The results are the same
 *                bit for bit; 1 exists to show that. */
typedef struct {
  int32_t bits;
  int32_t group_size;
  int32_t block_size;
  float damp_percent;
  int32_t desc_act;
  int32_t sym;
  int32_t per_block_steps;
} gptq_config;

/* ---------------------------------------------------------------- Hessian
 * H += 2 * X^T X over n_tokens calibration tokens (practice page 2.1: the
 * Hessian is built from the layer's input activations).
 *  H        [d_in x d_in] fp32, full symmetric, accumulated into (the caller
 *           zero-fills it once; further calls add more tokens).
 *  hdiag    [d_in] fp64, nullable, accumulated like H: diag(H) summed in fp64
 *           (the squares of bf16/fp16 values are exact).  gptq_prepare_hinv
 *           orders columns by these keys when given, so the desc_act order is
 *           the exact one and does not depend on fp32 accumulation rounding.
 *           NULL: the 16-bit kernels do none of this work (H is the same).
 *  X        [n_tokens x d_in], token-major, of x_dtype (bf16/fp16 multiply
 *           exactly in fp32 on MFMA; fp32 inputs use the fp32 MFMA), 16-byte
 *           aligned (the kernels load 16 bytes at a time; INVALID_ARG else).
 *  d_in     1..65536, multiple of 8.  n_tokens >= 0 (0 leaves H unchanged).
 *  ws       scratch of gptq_hessian_workspace_size(n_tokens, d_in) bytes
 *           (partial sums of the split token range; the result does not
 *           depend on timing: every partial is reduced in a fixed order). */
size_t gptq_hessian_workspace_size(int64_t n_tokens, int32_t d_in);
int gptq_hessian_accumulate(float* H, double* hdiag, const void* X, gptq_dtype x_dtype,
                            int64_t n_tokens, int32_t d_in, void* ws, size_t ws_bytes,
                            hipStream_t s);

/* gptq_hessian_accumulate for callers that cannot allocate device memory
 * (code under HIP graph capture, tight calibration loops, harnesses that forbid
 * hipMalloc): the same H and hdiag (same kernels; H within fp32 accumulation
 * order of the other call, since the token range may be split differently),
 * with the partial sums in a static device array of
 * gptq_hessian_noalloc_scratch_bytes() = 256 MiB that each GPU the library
 * runs on holds until the process ends.  It calls no allocator.
 *  d_in up to 11,264 (one token split's partial tiles must fit the array);
 *  larger d_in returns GPTQ_ERR_WORKSPACE before anything is enqueued.
 *  The first call on a device looks up the array's device address (kept per
 *  device).  Every call on one GPU shares its array, so calls that overlap on
 *  one GPU (different streams, or host threads) race: order them on one
 *  stream.  Nothing in the array needs clearing (every partial is written
 *  before it is read). */
size_t gptq_hessian_noalloc_scratch_bytes(void);
int gptq_hessian_accumulate_noalloc(float* H, double* hdiag, const void* X, gptq_dtype x_dtype,
                                    int64_t n_tokens, int32_t d_in, hipStream_t s);

/* ---------------------------------------------------------------- H^-1 factor
 * From H (undamped, as accumulated): lambda = damp_percent * mean(diag H);
 * perm = processing order -> original column (identity, or stable descending
 * diag(H) when desc_act); U [d_in x d_in] fp32 upper triangular (zeros below)
 * with U^T U = (H[perm][:,perm] + lambda I)^-1 -- the triangular factor of the
 * inverse Hessian of practice page section 2.2 ("third").  The page calls it
 * lower-triangular; that factor is U^T.
 *  H        [d_in x d_in] fp32 input, unchanged.
 *  hdiag    [d_in] fp64 diagonal keys from gptq_hessian_accumulate, or NULL
 *           to take diag(H): used for lambda and for the desc_act order.
 *  U        [d_in x d_in] fp32 output.  perm [d_in] int32 output.
 *  ws       scratch of gptq_prepare_hinv_workspace_size(d_in) bytes.
 * Synchronizes s.  Returns GPTQ_ERR_NOT_PD when a pivot of the factorization
 * is <= 0 or NaN (the pages' remedy: a larger damp_percent); U is then
 * undefined. */
size_t gptq_prepare_hinv_workspace_size(int32_t d_in);
int gptq_prepare_hinv(const float* H, const double* hdiag, int32_t d_in, float damp_percent,
                      int32_t desc_act, float* U, int32_t* perm, void* ws, size_t ws_bytes,
                      hipStream_t s);

/* ---------------------------------------------------------------- quantize
 * GPTQ column loop (practice page 2.1 / 2.2; min-max grid of the tutorial
 * page section 二).  In processing order k (column perm[k]) and per row r:
 * at each group start, scale = (max - min)/maxq and zero = rint(-min/scale)
 * over the group's current (already compensated) weights; code =
 * clamp(rint(w/scale) + zero, 0, maxq); q = scale*(code - zero);
 * e = (w - q)/U[k][k]; the later columns of the 128-column block take
 * w -= e * U[k][.] at once, the columns after the block take one lazy update
 * W -= Err * U[block rows][after] at the block's end.  The block's running
 * weights, the grid and every integer decision (zero point, code) are fp64;
 * the work copy of W, U and the lazy update are fp32.  scales are the fp64
 * scales rounded to fp32.
 *  W       [d_out x d_in] of w_dtype, original column order, unchanged.
 *  U, perm as produced by gptq_prepare_hinv (processing order).
 *  codes   [d_out x d_in] uint8 output, original column order.
 *  scales  [d_out x n_groups] fp32, zeros [d_out x n_groups] int32 outputs,
 *          indexed by processing-order group; n_groups = ceil(d_in / G).
 *  g_idx   [d_in] int32 output: original column -> group.
 *  Q       [d_out x d_in] fp32 dequantized weights, original order; may be NULL.
 *  ws      scratch of gptq_quantize_workspace_size(d_out, d_in, cfg) bytes (cfg
 *          NULL: a size that suffices for every configuration at this shape).
 *  d_out >= 1, d_in >= 1 (any width; packing needs d_in % 8 == 0). */
size_t gptq_quantize_workspace_size(int32_t d_out, int32_t d_in, const gptq_config* cfg);
int gptq_quantize_layer(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                        const float* U, const int32_t* perm, const gptq_config* cfg,
                        uint8_t* codes, float* scales, int32_t* zeros, int32_t* g_idx,
                        float* Q, void* ws, size_t ws_bytes, hipStream_t s);

/* ---------------------------------------------------------------- pack
 * Eight 4-bit codes per uint32 (practice page section 1.1: half a byte per
 * weight at 4 bits): packed[r][m] = sum_k (codes[r][8m+k] & 15) << 4k.
 *  codes [rows x cols] uint8, packed [rows x cols/8] uint32; cols % 8 == 0.
 *  3-bit codes are stored as nibbles too. */
int gptq_pack_int4(const uint8_t* codes, int64_t rows, int64_t cols, uint32_t* packed,
                   hipStream_t s);

/* Dense packing for 2, 3, 4 or 8 bits (practice page section 1.1 counts
 * bits/8 byte per weight): each row is one bit stream, code k at bits
 * [k*bits, (k+1)*bits) from the least significant bit of the row's word 0; a
 * 3-bit code may straddle two words.  At 4 bits the layout equals
 * gptq_pack_int4's.  Each code is masked to its low `bits` bits.
 *  codes [rows x cols] uint8, packed [rows x cols*bits/32] uint32.
 *  INVALID_ARG: bits not in {2, 3, 4, 8}, (cols * bits) % 32 != 0, null
 *  pointers, negative sizes. */
int gptq_pack_dense(const uint8_t* codes, int64_t rows, int64_t cols, int32_t bits,
                    uint32_t* packed, hipStream_t s);

/* ---------------------------------------------------------------- using the packed layer
 * Y = X W^T with W dequantized from the packed 4-bit layer (practice page
 * section 4.3: at inference the 4-bit weights are dequantized to a 16-bit type,
 * then multiplied).  W[r][c] = round16(scales[r][g] * (code[r][c] - zeros[r][g])),
 * the product taken in fp32 and rounded (ties to even) to x_dtype, with
 * code[r][c] = (packed[r][c/8] >> 4(c%8)) & 15 and g = g_idx[c] (clamped to
 * [0, n_groups)), or, with g_idx NULL, g = c / group_size (group_size a
 * multiple of 8, or -1 for one group per row).  Products accumulate in fp32;
 * Y is rounded once to y_dtype.
 *  X [m x d_in] f16/bf16 row-major, 16-byte aligned; packed [d_out x d_in/8]
 *  uint32; scales [d_out x n_groups] fp32; zeros [d_out x n_groups] int32;
 *  Y [m x d_out] of y_dtype (F32, F16 or BF16).  d_in % 8 == 0.
 *  INVALID_ARG: null pointers, bad sizes or dtypes, misaligned X, with g_idx
 *  NULL a group size that is not a multiple of 8 or an n_groups that does not
 *  match it. */
int gptq_w4a16_gemm(const void* X, gptq_dtype x_dtype, int64_t m, int32_t d_in,
                    const uint32_t* packed, const float* scales, const int32_t* zeros,
                    const int32_t* g_idx, int32_t group_size, int32_t n_groups, int32_t d_out,
                    void* Y, gptq_dtype y_dtype, hipStream_t s);

/* ---------------------------------------------------------------- layer error
 * out_host[0] = ||(W - Q) X^T||_F^2 = 1/2 tr((W - Q) H (W - Q)^T) with the
 * undamped H (practice page section 5.5: measure the loss, do not eyeball it).
 * fp32 products, fp64 final sum.  Synchronizes s.
 *  H [d_in x d_in] fp32, W [d_out x d_in] of w_dtype, Q [d_out x d_in] fp32.
 *  ws: gptq_layer_error_workspace_size(d_out, d_in) bytes. */
size_t gptq_layer_error_workspace_size(int32_t d_out, int32_t d_in);
int gptq_layer_error(const float* H, const void* W, gptq_dtype w_dtype, const float* Q,
                     int32_t d_out, int32_t d_in, double* out_host, void* ws, size_t ws_bytes,
                     hipStream_t s);

/* ---------------------------------------------------------------- AWQ
 * Activation-aware weight quantization, the second method of the pages
 * ("GPTQ/AWQ量化导出：让大模型在消费级显卡上跑起来", its AWQ steps: per-channel RMS
 * of the calibration activations, the top 5 % of channels get a larger factor,
 * the factor is undone at inference; "大模型压缩量化技术：GPTQ 与 AWQ 原理详解 +
 * Python 实战教程" section 四: weights of the large-activation channels times
 * s > 1, quantize, activations divided by s, the best factor chosen; no
 * Hessian).  The grid is the asymmetric min-max grid of the GPTQ calls, with
 * correctly rounded fp32 divisions. */

/* a[j] += sum_t X[t][j]^2 in fp64 (exact squares; the token splits are added
 * in a fixed order), the square of the RMS times n_tokens.  Accumulates, like
 * the Hessian: zero a before the first chunk.
 *  a   [d_in] fp64 (device).  X [n_tokens x d_in] of x_dtype.
 *  ws  scratch of gptq_awq_sumsq_workspace_size(n_tokens, d_in) bytes.
 *  n_tokens == 0 leaves a untouched. */
size_t gptq_awq_sumsq_workspace_size(int64_t n_tokens, int32_t d_in);
int gptq_awq_act_sumsq(double* a, const void* X, gptq_dtype x_dtype, int64_t n_tokens,
                       int32_t d_in, void* ws, size_t ws_bytes, hipStream_t s);

/* The factor search.  Salient channels: the k = floor(top_frac * d_in + 0.5)
 * channels with the largest a[j] (ties to the lower index).  For each
 * candidate sigma = grid[i]: s_j = sigma on salient channels, 1 elsewhere;
 * per group of group_size consecutive columns (-1: the whole row) the grid of
 * fp32(W[r][j] * s_j); Qhat = scale * (code - zero) / s_j (fp64); and
 * scores[i] = sum_j a[j] sum_r (W[r][j] - Qhat[r][j])^2 (fp64, rows added in a
 * fixed order).  The first smallest score wins: s_out[j] = its sigma on
 * salient channels, 1 elsewhere; *best = its index (best may be NULL).
 *  W [d_out x d_in] of w_dtype; a [d_in] fp64 from gptq_awq_act_sumsq;
 *  grid: HOST array of n_grid (1..32) finite factors > 0;
 *  s_out [d_in] fp32, scores [n_grid] fp64, best [1] int32 (device).
 *  ws  scratch of gptq_awq_search_workspace_size(d_out, d_in, group_size) bytes.
 *  INVALID_ARG: bits outside 2..8, group_size 0 or < -1, top_frac outside
 *  [0, 1], a bad grid, null pointers, non-positive sizes. */
size_t gptq_awq_search_workspace_size(int32_t d_out, int32_t d_in, int32_t group_size);
int gptq_awq_search(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                    const double* a, int32_t bits, int32_t group_size, float top_frac,
                    const float* grid, int32_t n_grid, float* s_out, double* scores,
                    int32_t* best, void* ws, size_t ws_bytes, hipStream_t s);

/* Quantize with given channel factors: per group the grid of
 * fp32(W[r][j] * s[j]); codes [d_out x d_in] uint8; scales/zeros
 * [d_out x n_groups] fp32/int32 (the grid of the scaled weights; at inference
 * the activations are divided by s); Qhat (may be NULL) [d_out x d_in] fp32,
 * the effective weights scale * (code - zero) / s[j] rounded from fp64. */
int gptq_awq_quantize(const void* W, gptq_dtype w_dtype, int32_t d_out, int32_t d_in,
                      const float* s, int32_t bits, int32_t group_size, uint8_t* codes,
                      float* scales, int32_t* zeros, float* Qhat, hipStream_t s_stream);

/* ---------------------------------------------------------------- one decoder block
 * The forward pieces that layer-by-layer quantization needs between the
 * sub-layers of a Llama decoder block ("GPTQ/AWQ量化导出：让大模型在消费级显卡上
 * 跑起来": a calibration forward pass collects each layer's inputs and the
 * layers are quantized one after another; "大模型压缩量化技术：GPTQ 与 AWQ 原理
 * 详解 + Python 实战教程": one layer at a time, its curvature from running the
 * calibration data through it).  fp32 throughout; token-major [T x d]. */

/* Y[t] = X[t] / sqrt(mean_j X[t][j]^2 + eps) * gamma (gamma NULL: 1).
 *  X [n_tokens x d] of x_dtype; Y [n_tokens x d] fp32. */
int gptq_rmsnorm(const void* X, gptq_dtype x_dtype, int64_t n_tokens, int32_t d,
                 const float* gamma, float eps, float* Y, hipStream_t s);

/* Y = X W^T (+ R): X [n_tokens x d_in], W [d_out x d_in] (e.g. the dequantized
 * Q of gptq_quantize_layer), R and Y [n_tokens x d_out]; R may be NULL or
 * equal to Y (then Y is accumulated into).  n_tokens <= INT_MAX.
 *  ws  scratch of gptq_linear_workspace_size(d_out, d_in) bytes (W^T). */
size_t gptq_linear_workspace_size(int32_t d_out, int32_t d_in);
int gptq_linear(const float* X, int64_t n_tokens, int32_t d_in, const float* W, int32_t d_out,
                const float* R, float* Y, void* ws, size_t ws_bytes, hipStream_t s);

/* Causal self-attention of the block: q = x1 Wq^T, k = x1 Wk^T, v = x1 Wv^T
 * ([d x d] each); q and k rotated per head (pairs (i, i + hd/2) by
 * p * rope_base^(-2i/hd), p = t % seq_len); per sequence of seq_len tokens and
 * per head: softmax(q_h k_h^T / sqrt(hd)) over positions <= the query's,
 * times v_h; out [n_tokens x d] is the heads side by side (the o projection's
 * input).  hd = d / n_heads must be even; n_tokens a multiple of seq_len and
 * at most 65535 * 32.
 *  ws  scratch of gptq_block_attention_workspace_size(...) bytes (W^T, q, k,
 *      v, k^T, one sequence's scores per head, the rotation table). */
size_t gptq_block_attention_workspace_size(int64_t n_tokens, int32_t d, int32_t n_heads,
                                           int32_t seq_len);
int gptq_block_attention(const float* x1, int64_t n_tokens, int32_t d, int32_t n_heads,
                         int32_t seq_len, const float* Wq, const float* Wk, const float* Wv,
                         float rope_base, float* out, void* ws, size_t ws_bytes, hipStream_t s);

/* M = silu(G) * U elementwise, silu(x) = x / (1 + exp(-x)); n elements. */
int gptq_swiglu(const float* G, const float* U, int64_t n, float* M, hipStream_t s);

/* ---------------------------------------------------------------- misc */
const char* gptq_status_string(int status);
int gptq_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* GPTQ_MI355X_H */
