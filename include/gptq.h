/*
 * gptq.h -- C ABI of libgptq_mi355x.so: GPTQ's per-layer quantization hot path
 * on AMD MI355X (gfx950).
 *
 * Sources, cited by page title and section:
 *   [P1] "GPTQ：基于近似二阶信息的大模型权重量化"  (GPTQ tutorial)
 *   [P4] "GPTQ: практическое квантование языковых моделей без потери смысла"
 *   [P5] "GPTQ/AWQ量化中Group Size的精确含义与计算"  (group-size explainer)
 *
 * Conventions shared by every call
 *   - Every pointer argument is a DEVICE pointer owned by the caller, unless
 *     marked "host".  The library allocates no memory and keeps no state
 *     between calls; scratch space is passed in as `ws` of `ws_bytes` bytes,
 *     sized by the matching *_workspace() query (pass ws = NULL when the
 *     query returns 0).  `ws` must be 256-byte aligned.
 *   - Matrices are row-major and dense unless a leading dimension is given.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the
 *     null stream) and returns at once.  Results are valid once the stream
 *     has been synchronised.
 *   - Argument errors are reported synchronously, before anything is
 *     enqueued, as GPTQ_EINVAL / GPTQ_EUNSUPPORTED; a failed launch returns
 *     GPTQ_EHIP.  A factorization breakdown is only known on the device and
 *     is written to `dev_status` (see gptq_prepare_hinv).
 *   - NaN/Inf inputs are not detected; their outputs are unspecified.
 *   - Calls that share a workspace or an output buffer must not overlap in
 *     time (use one stream, or synchronise between them).
 */
#ifndef GPTQ_MI355X_H
#define GPTQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GPTQ_OK = 0,
  GPTQ_EINVAL = 1,       /* bad pointer, size or parameter */
  GPTQ_EUNSUPPORTED = 2, /* valid for the method but not implemented here */
  GPTQ_EHIP = 3,         /* a HIP launch or runtime call failed */
  GPTQ_ENOTSPD = 4       /* the damped Hessian is not positive definite */
} gptq_status;

typedef enum { GPTQ_BF16 = 0, GPTQ_F32 = 1 } gptq_dtype;

/* hipStream_t, kept opaque so this header needs no HIP include. */
typedef void* gptq_stream;

/* ---------------------------------------------------------------------------
 * Hessian accumulation.  [P1] 阶段一: the layer's Hessian is H = 2 X^T X over
 * the calibration tokens X [n x d_in].
 *
 *   H += 2 * X^T X
 *
 * H        [d x d] float32, row-major.  Only the lower triangle (diagonal
 *          included) is read and written; the strict upper triangle is left
 *          untouched.  Zero it before the first call; call again on further
 *          token chunks to accumulate (a saved H is a complete resume point).
 * X        [n_tokens x ldx] elements of x_dtype, row-major; columns 0..d-1
 *          are used.  bf16 values are widened exactly; products are formed
 *          exactly in float32 and summed in float32.
 * n_tokens >= 0 (0 is a no-op); ldx >= d; d >= 1.
 * ws       device scratch of gptq_hessian_workspace(d, n_tokens, x_dtype) bytes,
 *          256-byte aligned; its contents on entry do not matter (it holds the
 *          split-K partial tiles, which depend on d, n_tokens and x_dtype).
 * The result is deterministic: the same inputs give the same bits.
 * ------------------------------------------------------------------------- */
int gptq_hessian_accumulate(float* H, int64_t d, const void* X, int x_dtype,
                            int64_t n_tokens, int64_t ldx, void* ws, size_t ws_bytes,
                            gptq_stream stream);
size_t gptq_hessian_workspace(int64_t d, int64_t n_tokens, int x_dtype);

/* ---------------------------------------------------------------------------
 * gptq_hessian_accumulate without a workspace argument, for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * or calibration loops, harnesses that forbid allocation): the same
 * H += 2 X^T X with the same arguments, but the split-K partial tiles live in
 * a fixed array of gptq_noalloc_scratch_bytes() (64 MiB) that the library
 * holds on each GPU it runs on, from its load until the process ends.  This
 * call allocates and frees nothing.
 *
 * The number of token splits is capped so that the partials fit the array:
 * with bf16 X (256 x 256 tiles) d <= 5632, with fp32 X (64 x 64 tiles)
 * d <= 5760; larger d returns GPTQ_EUNSUPPORTED before anything is enqueued.
 * When the cap does not bind (small d or few tokens) the split count, and so
 * the result, is bit-identical to gptq_hessian_accumulate's; otherwise the
 * same sums are formed in another split order.
 * Every call on one GPU uses that GPU's one array: calls that overlap in time
 * on the same GPU (different streams, or different host threads without
 * ordering) race on it and give wrong results.  Calls on one stream are
 * ordered and safe; every partial tile is rewritten by each call, so nothing
 * carries over from the previous call.
 * ------------------------------------------------------------------------- */
int gptq_hessian_accumulate_noalloc(float* H, int64_t d, const void* X, int x_dtype,
                                    int64_t n_tokens, int64_t ldx, gptq_stream stream);
size_t gptq_noalloc_scratch_bytes(void);

/* ---------------------------------------------------------------------------
 * Damping, Cholesky and the upper factor of the inverse.  [P1] 阶段一 (H ~
 * 2X^T X + lambda I, then a Cholesky factorization whose triangular factor is
 * used row by row instead of a full inverse).
 *
 * In place on H (lower triangle read):
 *   1. dead[i] = (H_ii == 0); for dead i, H_ii = 1 (such an input channel is
 *      always zero; its weights are then quantized as 0);
 *   2. H += lambda I with lambda = damp * mean(diag H)   (damp = 0.01 usual);
 *   3. the strict upper triangle is overwritten with the mirror of the lower.
 * Then U [d x d] float32 is written: the upper triangular matrix with positive
 * diagonal and U^T U = H^{-1} (the strict lower triangle of U is set to 0).
 * It is computed as U = V^{-1} where H = V V^T with V upper triangular, which
 * is the same unique factor as chol(H^{-1}); arithmetic is fp32 with fused
 * multiply-adds (the lambda shift is formed in float64).  The factorization
 * is blocked in panels of 256 columns, each run by one launch whose
 * workgroups hand results to each other through flags in `ws`; every such
 * wait is bounded.
 *
 * dead       [d] uint8 out, may be NULL.
 * dev_status [1] int32 out (device): 0 on success; > 0: 1 + the index (in
 *            H's numbering) of the first diagonal element found non-positive
 *            (the elimination runs from index d-1 down to 0); -1: a bounded
 *            wait between workgroups expired and the factorization did not
 *            complete (not expected in normal operation; the environment
 *            variable GPTQ_SYNC_SPIN_LIMIT, read once per process, sets the
 *            number of polls, default 2^20).  U is unspecified when
 *            dev_status != 0.
 * ws         scratch of gptq_prepare_workspace(d) bytes (three d x d float32
 *            matrices plus O(d) more); its contents on entry do not matter.
 * ------------------------------------------------------------------------- */
int gptq_prepare_hinv(float* H, int64_t d, double damp, float* U, uint8_t* dead,
                      int32_t* dev_status, void* ws, size_t ws_bytes, gptq_stream stream);
size_t gptq_prepare_workspace(int64_t d);

/* ---------------------------------------------------------------------------
 * Greedy column-by-column quantization with error feedback.  [P1] 阶段二
 * (fixed ascending column order, lazy batched updates), 对称与仿射量化
 * (q = round(x/s) + z), 量化误差与补偿; [P4] rows are independent; [P5] group
 * sizes, the 0..2^b-1 grid and the zero point.
 *
 * For each row independently, columns j = 0..d_in-1 in order:
 *   at a group's first column (every group_size columns; only column 0 when
 *   group_size = -1, the whole row being one group) the group's CURRENT
 *   values v (after all feedback so far) give
 *     asymmetric: lo = min(0, min v), hi = max(0, max v),
 *                 scale = fp16((hi - lo)/maxq), zero = clamp(round(-lo/scale), 0, maxq)
 *     symmetric:  scale = fp16(2 max|v| / maxq), zero = (maxq + 1)/2
 *     (fp16 = one rounding of the float64 quotient to binary16, nearest-even;
 *      a zero range, or a scale that rounds to 0, gives scale = 1)
 *   q_j = clamp(round(w_j/scale) + zero, 0, maxq)   (round: nearest integer
 *         of the exact quotient, ties to even);  w_hat_j = scale (q_j - zero)
 *   delta_j = (w_j - w_hat_j) / U_jj;  w_k -= delta_j U_jk for all k > j.
 * The feedback to columns past the current block of `block` columns is
 * applied once per block as one matrix product (lazy batching); in exact
 * arithmetic this equals the column-by-column form.
 *
 * W        [d_out x d_in] of w_dtype (bf16 or float32), read only.
 * U        [d_in x d_in] float32 from gptq_prepare_hinv (upper triangle read).
 * dead     [d_in] uint8 or NULL; columns with dead[i] != 0 are zeroed first.
 * bits     2, 3 or 4 (maxq = 2^bits - 1).
 * group_size  32, 64, 128, or -1 (one group per row).  Must divide d_in.
 * sym      0 asymmetric, 1 symmetric.
 * block    128 (the only supported value).
 * codes    [d_out x d_in] uint8 out.
 * scales   [d_out x n_groups] float32 out (values exact in binary16);
 *          n_groups = d_in / group_size, or 1 when group_size = -1.
 * zeros    [d_out x n_groups] float32 out (integers).
 * loss_rows [d_out] float32 out or NULL: sum_j delta_j^2 per row, which
 *          equals (w - w_hat) H (w - w_hat)^T for the damped H.
 * ws       scratch of gptq_quantize_workspace(d_out, d_in, block) bytes.
 * d_out may be 0 (no-op).
 * ------------------------------------------------------------------------- */
int gptq_quantize_layer(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                        const float* U, const uint8_t* dead, int bits, int group_size,
                        int sym, int block, uint8_t* codes, float* scales, float* zeros,
                        float* loss_rows, void* ws, size_t ws_bytes, gptq_stream stream);
size_t gptq_quantize_workspace(int64_t d_out, int64_t d_in, int block);

/* ---------------------------------------------------------------------------
 * Packing.  [P5] 存储代价 gives the bit budget (b-bit codes, 16-bit scale and
 * a zero point per group; no zero when symmetric) but no layout; the layout
 * here is: the codes of a row form a little-endian bit stream, code j in bits
 * [b*j, b*j + b), cut into uint32 words, ceil(d_in*b/32) words per row
 * (3-bit codes straddle words: 32 codes per 3 words).
 *
 * codes      [d_out x d_in] uint8, each < 2^bits.
 * scales     [d_out x n_groups] float32 (binary16-exact), zeros likewise.
 * qweight    [d_out x ceil(d_in*bits/32)] uint32 out.
 * scales_f16 [d_out x n_groups] uint16 out: IEEE binary16 bits of scales.
 * zeros_f16  [d_out x n_groups] uint16 out: binary16 bits of zeros; not
 *            written when sym != 0 (may then be NULL).
 * ------------------------------------------------------------------------- */
int gptq_pack(const uint8_t* codes, const float* scales, const float* zeros, int64_t d_out,
              int64_t d_in, int bits, int group_size, int sym, uint32_t* qweight,
              uint16_t* scales_f16, uint16_t* zeros_f16, gptq_stream stream);

/* ---------------------------------------------------------------------------
 * Activation ordering and static groups.  "GPTQ：基于近似二阶信息的大模型权重量化",
 * GPTQ 的高级技巧: 激活排序（desc_act） (columns reordered by the summed
 * absolute input activations, the least influential quantized first, so the
 * error feedback lands on the more sensitive ones) and 静态与动态分组.
 *
 * gptq_act_order: perm[k] = the k-th column to quantize, in ascending order
 *   of a_c = sum_t |X[t][c]| (float64), ties by column index.
 *   X          [n_tokens x ldx] bf16 or fp32 (x_dtype), row-major, d used
 *              columns (as for gptq_hessian_accumulate); n_tokens may be 0
 *              (natural order).
 *   perm       [d] int32 out.
 *   act_sum    [d] float64 out: a_c (may be NULL).
 *   ws         gptq_act_order_workspace(d, n_tokens) bytes.
 *   NaN inputs leave perm unspecified.
 *
 * gptq_prepare_hinv_perm: gptq_prepare_hinv for the permuted matrix
 *   H[perm][:, perm]: H is damped and mirrored in place in natural order as
 *   before, dead[] is in natural order, U [d x d] is the upper factor of the
 *   permuted damped matrix's inverse.  perm NULL = natural order (then
 *   identical to gptq_prepare_hinv).  Workspace: gptq_prepare_workspace(d).
 *
 * gptq_quantize_layer_perm: gptq_quantize_layer with the columns processed
 *   in the order perm (NULL = natural), U from gptq_prepare_hinv_perm with the
 *   same perm, dead[] in natural order.  codes come back in natural column
 *   order.  Groups:
 *     static_groups = 0: a group is a run of group_size consecutive columns
 *       in processing order, its parameters set at its first column from the
 *       current (compensated) values; scales/zeros [d_out x n_groups] are
 *       indexed by that group number.
 *     static_groups = 1: the natural runs of group_size columns, parameters
 *       from the original weights before any feedback; column c uses group
 *       c / group_size.
 *   g_idx      [d_in] int32 out (may be NULL): the group of each natural column
 *              (dynamic: g_idx[perm[k]] = k / group_size; static: c /
 *              group_size; group_size -1: 0).
 *   ws         gptq_quantize_perm_workspace(d_out, d_in, block) bytes.
 *   perm must be a permutation of 0..d-1 (d = d_in); entries outside that
 *   range are clamped (results then unspecified, memory stays in bounds).
 * ------------------------------------------------------------------------- */
int gptq_act_order(const void* X, int x_dtype, int64_t n_tokens, int64_t ldx, int64_t d,
                   int32_t* perm, double* act_sum, void* ws, size_t ws_bytes, gptq_stream stream);
size_t gptq_act_order_workspace(int64_t d, int64_t n_tokens);
int gptq_prepare_hinv_perm(float* H, int64_t d, double damp, const int32_t* perm, float* U,
                           uint8_t* dead, int32_t* dev_status, void* ws, size_t ws_bytes,
                           gptq_stream stream);
int gptq_quantize_layer_perm(const void* W, int w_dtype, int64_t d_out, int64_t d_in,
                             const float* U, const uint8_t* dead, const int32_t* perm,
                             int static_groups, int bits, int group_size, int sym, int block,
                             uint8_t* codes, float* scales, float* zeros, int32_t* g_idx,
                             float* loss_rows, void* ws, size_t ws_bytes, gptq_stream stream);
size_t gptq_quantize_perm_workspace(int64_t d_out, int64_t d_in, int block);

/* ---------------------------------------------------------------------------
 * Several layers that share one Hessian (their inputs are the same
 * activations, e.g. the query/key/value projections, or the gate and up
 * projections of a feed-forward block), quantized in one call:
 * gptq_quantize_layer on the row-wise stack of the matrices.  Rows are
 * independent given U, so each layer's results are bit-identical to its own
 * gptq_quantize_layer call.
 *
 * W_list       HOST array of count device pointers, matrix i [d_out_list[i] x d_in]
 *              (all of dtype w_dtype).
 * d_out_list   HOST array of count row counts (0 allowed).
 * codes, scales, zeros, loss_rows: stacked outputs over all rows, matrix 0
 *              first ([sum d_out x d_in] codes, [sum d_out x n_groups]
 *              scales/zeros, [sum d_out] losses; loss_rows may be NULL).
 * ws           gptq_quantize_workspace(sum d_out, d_in, block) bytes.
 * Other arguments and errors as gptq_quantize_layer; 1 <= count <= 64.
 * ------------------------------------------------------------------------- */
int gptq_quantize_layers(const void* const* W_list, const int64_t* d_out_list, int count,
                         int w_dtype, int64_t d_in, const float* U, const uint8_t* dead, int bits,
                         int group_size, int sym, int block, uint8_t* codes, float* scales,
                         float* zeros, float* loss_rows, void* ws, size_t ws_bytes,
                         gptq_stream stream);

/* ---------------------------------------------------------------------------
 * Dequantized product with the packed 4-bit weights (W4A16).
 * "GPTQ：基于近似二阶信息的大模型权重量化", 阶段三 (inference on the integer codes
 * with their group scale and zero) and "GPTQ/AWQ量化中Group Size的精确含义与计算",
 * 存储代价 (a 16-bit scale and a zero per group of g columns).
 *
 *   Y[i][n] = sum_k X[i][k] W_hat[n][k],
 *   W_hat[n][k] = s[n][k/g] (q[n][k] - z[n][k/g])   (g = d_in when group_size = -1)
 *
 * X           [m x ldx] bf16, row-major, d_in used columns; 16-byte aligned,
 *             ldx a multiple of 8.
 * qweight     [d_out x d_in/8] uint32: gptq_pack's 4-bit layout (code k of a
 *             row in bits 4(k%8) .. 4(k%8)+3 of word k/8).
 * scales_f16, zeros_f16  [d_out x n_groups] binary16 bits as gptq_pack writes
 *             them; with sym = 1 zeros_f16 is not read and z = 8.
 * Y           [m x d_out] float32 out.
 * d_in must be a multiple of 128 (GPTQ_EUNSUPPORTED otherwise); group_size
 * 32, 64, 128 or -1.  Groups are the natural runs of g columns (the plain
 * path, or static groups with activation ordering).  Every product
 * x (q - z) is exact in fp32; each group's sum is scaled by s in fp32, so
 * only fp32 accumulation rounds.
 * ------------------------------------------------------------------------- */
int gptq_w4a16_matmul(const void* X, int64_t m, int64_t ldx, const uint32_t* qweight,
                      const uint16_t* scales_f16, const uint16_t* zeros_f16, int64_t d_out,
                      int64_t d_in, int group_size, int sym, float* Y, gptq_stream stream);

/* ---------------------------------------------------------------------------
 * Two-sided adaptive rounding.  "GPTQ-2D: 三次时间复杂度的双侧自适应舍入",
 * 方法 steps 1-3 (anti-diagonal order, entries of one anti-diagonal in
 * parallel, errors carried through the two bases' triangular factors) and
 * 核心洞察 (the same output as nearest-plane rounding on the vectorized,
 * Kronecker-structured problem, in O(n^3) instead of O(n^4)).
 *
 * Rounds Y to the integer matrix Z, coordinate by coordinate with error
 * feedback, under the metric || R_L (Y - Z) R_R^T ||_F^2 (scale 1, no clamp):
 * anti-diagonals i + j = s from s = 2n-2 down to 0; for entry (i, j),
 *   S = sum_{k>=i} R_L[i][k] P[k][j],  Z[i][j] = rint(Y[i][j] + S / (R_L[i][i] R_R[j][j])),
 * then row i of the running array P gets (Y[i][j] - Z[i][j]) R_R[0..j][j].
 * rint rounds half to even.  All arithmetic is float64.
 *
 * Y            [n x n] float64, row-major.
 * left_basis   [n x n] float64 R_L, row-major; only the upper triangle
 *              (diagonal included) is read.  Its diagonal must be positive.
 * right_basis  [n x n] float64 R_R, likewise.
 * Z            [n x n] float64 out: integer values.
 * ws           gptq2d_workspace(n) bytes: the running array and a transposed
 *              copy of R_R.
 * n            1 .. GPTQ2D_MAX_N (0 is a no-op); larger n gives
 *              GPTQ_EUNSUPPORTED.  For n <= 1024 one persistent launch
 *              (a wave per row; rows hand values to each other through
 *              the workspace, and through LDS inside a workgroup, with
 *              bounded waits); beyond, 2n-1 dependent launches, one per
 *              anti-diagonal.  Both give the same Z.
 * A bounded wait that gives up (environment GPTQ_SYNC_SPIN_LIMIT polls,
 * default 2^20; not reached in a normal run) leaves NaN in every entry of Z
 * that depends on the missing value; the call still completes.
 * A non-positive diagonal entry in a basis is not detected: Z is then
 * unspecified.
 * ------------------------------------------------------------------------- */
#define GPTQ2D_MAX_N 32768
int gptq2d_round(const double* Y, const double* left_basis, const double* right_basis, int64_t n,
                 double* Z, void* ws, size_t ws_bytes, gptq_stream stream);
size_t gptq2d_workspace(int64_t n);

/* Host: static description of a status code. */
const char* gptq_strerror(int status);

/* Host: ABI version (major * 100 + minor). */
int gptq_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
