/*
 * gptq.h -- C ABI of the MI355X (gfx950) GPTQ layer-quantization library
 * (libgptq_mi355x.so).
 *
 * The method: for one linear layer with weights W [m, d] and calibration
 * activations X [N, d], form H = 2 X^T X, damp it, take the upper Cholesky
 * factor U of H^-1, then round the columns of W one by one in natural order,
 * pushing each column's error (w_i - q_i) / U_ii onto the columns not yet
 * rounded, with the updates applied lazily in blocks of 128 columns.
 * Sources: "GPTQ: Accurate Post-Training Quantization for Generative
 * Pre-trained Transformers", breakdown by FDE Interviews -- section 01 "The
 * paper in one minute" and the figure "Quantize a column, correct the rest",
 * steps 1-4; "[Paper Review] GPTQ ..." (nubint), "Proposed method".
 *
 * Conventions for every entry point
 *  - Pointers named d_* / H / X / U / W / outputs are DEVICE pointers (HIP
 *    global memory of the current device); `cfg` and `info_host` style
 *    arguments are host pointers where stated. The caller owns every buffer;
 *    the library never allocates or frees device memory. Scratch memory comes
 *    only from `workspace`, sized with gptq_workspace_bytes().
 *  - `stream` is a hipStream_t passed as void* (NULL = the null stream). Every
 *    call validates its arguments on the host, enqueues its kernels on
 *    `stream` and returns; outputs are valid once the stream has synchronized.
 *    Calls on distinct streams with distinct buffers are independent.
 *  - Matrices are row-major with a leading dimension (elements) `ld*`.
 *  - Errors: host-detectable problems (null pointer, size <= 0, bad ld,
 *    unsupported option, workspace too small) return a status synchronously and
 *    enqueue nothing. A failed launch returns GPTQ_ERR_HIP. Numerical failure
 *    (H_d not positive definite) is reported through the device int `*info`.
 *    No C++ exception crosses this interface.
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
  GPTQ_ERR_INVALID_ARG = 1,
  GPTQ_ERR_WORKSPACE = 2,
  GPTQ_ERR_HIP = 3,
  GPTQ_ERR_UNSUPPORTED = 4
} gptq_status_t;

typedef enum { GPTQ_GRID_ASYM_MINMAX = 0, GPTQ_GRID_TERNARY = 1, GPTQ_GRID_SYM_MINMAX = 2 } gptq_grid_t;

typedef enum { GPTQ_F16 = 0, GPTQ_F32 = 1, GPTQ_F64 = 2 } gptq_dtype_t;

/* Which factor of the damped Hessian H_d the quantizer is given. */
typedef enum {
  GPTQ_FACTOR_HINV_CHOL = 0, /* U, upper, U^T U = H_d^-1 (gptq_prepare_hinv) */
  GPTQ_FACTOR_H_CHOL = 1     /* R, upper, R R^T = H_d, R = U^-1 (gptq_prepare_hchol) */
} gptq_factor_t;

/* Quantizer configuration (host struct).
 *  bits       2, 3, 4 or 8 (ternary: 2; codes 0, 1, 2 stand for -s, 0, +s).
 *  grid       gptq_grid_t. Asymmetric min-max: lo = min(min v, 0),
 *             hi = max(max v, 0) (both 0 -> -1, +1), s = (hi - lo) / (2^b - 1),
 *             z = rint(-lo / s). Ternary: s = max|v| (0 -> 1), z = 1.
 *             Symmetric min-max: a = max|v| (0 -> 1), s = 2a / (2^b - 1),
 *             z = 2^(b-1) (code z is exactly 0).
 *             The pages only name "3/4-bit grids", grouping, 2-bit and ternary
 *             levels and compatibility with various grids (nubint review, "Key
 *             findings"); these fits are the readings the library implements.
 *  group_size 0 = one grid per output row, fitted on the original row;
 *             16, 32, 64 or 128 = a grid per group of columns, fitted at the
 *             group's first column on the current (error-updated) weights;
 *             any other multiple of 32 dividing d (96, 192, 256, 1024, ...) =
 *             the same, fitted over the whole group with every earlier update
 *             applied (the lazy blocks are then also cut at group starts).
 *             Other sizes: GPTQ_ERR_UNSUPPORTED; not dividing d: INVALID_ARG.
 *  block_size must be 128 (the lazy-update block of the figure's step 4).
 *  factor     gptq_factor_t: the matrix passed as `U` to the quantize calls.
 *             GPTQ_FACTOR_H_CHOL takes R = U^-1 and never forms U: since the
 *             errors are e = (w - q) R for the original weights w, the pushes of
 *             earlier blocks sum to A = sum_l (w_l - q_l) R[l, .], and a block's
 *             true state is w + A_blk (R_bb)^-1 with R_bb its diagonal block;
 *             the steps inside the block are the figure's, with (R_bb)^-1.
 *             Group sizes other than 16, 32, 64 and 128 need
 *             GPTQ_FACTOR_HINV_CHOL unless the groups are static. */
typedef struct {
  int32_t bits;
  int32_t grid;
  int32_t group_size;
  int32_t block_size;
  int32_t factor;
} gptq_qcfg_t;

/* Which call a workspace is sized for. */
enum { GPTQ_WS_ACCUMULATE_HESSIAN = 0, GPTQ_WS_PREPARE_HINV = 1, GPTQ_WS_QUANTIZE_LAYER = 2 };

/* ABI version of this header (incremented on incompatible changes; 2 added the
 * `factor` field of gptq_qcfg_t and gptq_prepare_hchol). */
int32_t gptq_abi_version(void);

/* Human-readable text for a status code (static storage, never NULL). */
const char* gptq_status_string(int32_t status);

/* Bytes of workspace the named call needs for these sizes (0 = none).
 *  which = GPTQ_WS_ACCUMULATE_HESSIAN: uses d and n (tokens per call): the
 *          split-K partial tiles, then for d >= 12288 a feature-major copy
 *          of the call's tokens (d x n fp16, at most d x 65536 when the call
 *          is cut into launches). A smaller workspace (even NULL / 0) is accepted: without
 *          room for the copy X is read token-major (a slower form of the same
 *          sum), without room for the partials the token-split parallelism
 *          goes too.
 *  which = GPTQ_WS_PREPARE_HINV: uses d.
 *  which = GPTQ_WS_QUANTIZE_LAYER: uses m, d and cfg (host pointer, may be NULL
 *          for the defaults). */
size_t gptq_workspace_bytes(int32_t which, int64_t m, int64_t d, int64_t n, const gptq_qcfg_t* cfg);

/* Hessian accumulation: H[i][j] = (accumulate ? H[i][j] : 0) + 2 sum_t X[t][i] X[t][j]
 * for i >= j (lower triangle; the strictly upper triangle is not touched).
 * FDE breakdown, section 01: the curvature of the layer-wise least-squares
 * problem is H = 2XX^T from the calibration inputs (X = [d, N] there; here X is
 * token-major [N, d], the same matrix).
 *  H        device, [d][ldh], h_dtype GPTQ_F64 (recommended) or GPTQ_F32.
 *  X        device, fp16, token-major [n][ldx]; 16-byte aligned, ldx % 8 == 0.
 *  d        features, d % 32 == 0. n tokens in this call, n >= 0 (n = 0 with
 *           accumulate = 0 zeroes the lower triangle).
 *  Products are exact fp16 x fp16 -> fp32 on the matrix cores. Each window of
 *  W tokens is summed in fp32 (W/16 matrix steps, one rounding each) and
 *  folded into a compensated running sum, combined in fp64 at the end: the
 *  error does not grow with n beyond the windows' own roundings, each entry
 *  within (W/8) 2^-24 sum_t 2|x_ti x_tj|; in Frobenius norm it scales as
 *  W / sqrt(n) (1.1e-8 relative measured at n = 262144, W = 1024). W follows
 *  this call's n: 1024 from 262144 tokens, 512 from 65536, 256 below.
 *  Call it once per chunk of tokens with accumulate = 1 after the first. */
gptq_status_t gptq_accumulate_hessian(void* H, int32_t h_dtype, int64_t d, int64_t ldh,
                                      const void* X, int64_t n, int64_t ldx, int32_t accumulate,
                                      void* workspace, size_t ws_bytes, void* stream);

/* gptq_accumulate_hessian for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results, with the split-K partial tiles in a static device
 * array of the library (192 MiB, one per GPU it runs on, held until the process
 * ends) instead of a workspace. The call allocates nothing: no hipMalloc, no
 * hipFree, no event (a trace active on the thread is paused for the call).
 * Arguments, layout and errors as gptq_accumulate_hessian, plus
 * GPTQ_ERR_WORKSPACE when (d, n) would need more partial tiles than the array
 * holds (gptq_workspace_bytes(GPTQ_WS_ACCUMULATE_HESSIAN, 0, d, n, NULL) >
 * 192 MiB; no call of up to 262144 tokens with d <= 65536 does). Every call
 * on one GPU shares that GPU's array and leaves its contents behind; the
 * kernels write every partial they read, so nothing needs clearing. Calls that
 * overlap on one GPU (other streams, other host threads) race on the array:
 * serialize them. */
gptq_status_t gptq_accumulate_hessian_noalloc(void* H, int32_t h_dtype, int64_t d, int64_t ldh,
                                              const void* X, int64_t n, int64_t ldx, int32_t accumulate,
                                              void* stream);

/* Inverse-Hessian factor: U (upper, row-major, zeros below the diagonal) with
 * U^T U = (H + lambda I)^-1, lambda = damp * mean(diag H).
 * FDE breakdown, figure step 2: U = chol(H^-1); section 01: the rows of the
 * inverse Hessian come from a Cholesky decomposition for numerical stability;
 * nubint review, "Proposed method": Cholesky reformulation and dampening.
 * Computed in fp64 as U = J inv(L) J with L L^T = J H_d J (J the reversal
 * permutation), the same unique factor in half the flops of
 * Cholesky -> inverse -> Cholesky.
 *  H        device [d][ldh] (lower triangle read), h_dtype GPTQ_F32 | GPTQ_F64.
 *  U        device [d][ldu], u_dtype GPTQ_F32 | GPTQ_F64. May alias H (H is
 *           read into the workspace before U is written).
 *  damp     relative dampening (0.01 in the pages' defaults), >= 0.
 *  info     device int32: 0 = success, k > 0 = the reversed leading minor of
 *           order k is not positive definite (U is then undefined).
 *  lambda_out device double, may be NULL: receives lambda.
 *  workspace gptq_workspace_bytes(GPTQ_WS_PREPARE_HINV, 0, d, 0, NULL) bytes. */
gptq_status_t gptq_prepare_hinv(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, double damp,
                                void* U, int32_t u_dtype, int64_t ldu, int32_t* info,
                                double* lambda_out, void* workspace, size_t ws_bytes, void* stream);

/* The Cholesky factor of the damped Hessian itself: R (upper, row-major, zeros
 * below the diagonal) with R R^T = H + lambda I, lambda as gptq_prepare_hinv;
 * R = U^-1 for the U that gptq_prepare_hinv returns. FDE breakdown, section 01:
 * the inverse Hessian's rows are taken from a Cholesky decomposition (figure
 * step 2: U = chol(H^-1)); the quantize calls take R with cfg->factor =
 * GPTQ_FACTOR_H_CHOL and apply U = R^-1 without forming it (see gptq_qcfg_t).
 * Computed in fp64 as R = J L J with L L^T = J H_d J (J the reversal), the
 * Cholesky alone: d^3 / 3 flops, half of gptq_prepare_hinv's.
 * Arguments, workspace, info and errors as gptq_prepare_hinv (R in place of U;
 * R may alias H). For the quantize calls R should be GPTQ_F64: they invert R's
 * 128 x 128 diagonal blocks from it. */
gptq_status_t gptq_prepare_hchol(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, double damp,
                                 void* R, int32_t r_dtype, int64_t ldr, int32_t* info,
                                 double* lambda_out, void* workspace, size_t ws_bytes, void* stream);

/* Column-by-column quantization in natural order with lazy 128-column blocks.
 * FDE breakdown, figure steps 1-4, for column i: round w_i to the grid (q_i);
 * err = (w_i - q_i) / U_ii; W[:, i+1:] -= err x U[i, i+1:]; updates applied in
 * blocks of 128 columns. Section 01: one column order shared by every row.
 *  W        device [m][ldw], w_dtype GPTQ_F16 | GPTQ_F32. Read only (the library
 *           works on an fp32 copy in the workspace).
 *  U        device [d][ldu] upper factor from gptq_prepare_hinv, u_dtype
 *           GPTQ_F32 | GPTQ_F64 (GPTQ_F64 is converted to fp32 per block); with
 *           cfg->factor = GPTQ_FACTOR_H_CHOL, R from gptq_prepare_hchol instead.
 *  cfg      host pointer to the quantizer configuration.
 *  qcodes   device uint32 [m][d * bits / 32]: row-wise LSB-first bitstream,
 *           code j at bits [j*bits, (j+1)*bits) of its row. d * bits % 32 == 0.
 *  scales   device float [m][ngroups], ngroups = group_size ? d / group_size : 1.
 *  zeros    device uint8 [m][ngroups] (integer zero points).
 *  W_hat    device float [m][d] = s * (code - z), may be NULL.
 *  err_sq   device float [m]: sum over the row of err^2 / 2 (the optimal-brain-
 *           surgeon loss increments), may be NULL.
 *  Sizes: m >= 1, d % 32 == 0, group_size dividing d. */
gptq_status_t gptq_quantize_layer(const void* W, int32_t w_dtype, int64_t m, int64_t d, int64_t ldw,
                                  const void* U, int32_t u_dtype, int64_t ldu, const gptq_qcfg_t* cfg,
                                  uint32_t* qcodes, float* scales, uint8_t* zeros, float* W_hat,
                                  float* err_sq, void* workspace, size_t ws_bytes, void* stream);

/* Act-order (desc_act): the order in which to quantize the columns, largest
 * activations first. The zhiliyouxian blog ("实践指南", "超参数选择") passes
 * desc_act, which sorts the columns by their activations (off by default);
 * the CSDN page "GPTQ量化参数搜索工具" lists --desc_act and --static_groups. The
 * pages say no more; this library reads the size of column j's activations as
 * H_jj = 2 sum_t x_tj^2.
 *  H        device [d][ldh] (only the diagonal is read), h_dtype GPTQ_F32 | GPTQ_F64.
 *  perm     device int32 [d], out: perm[j] = the column with the j-th largest
 *           H_jj, equal values in index order (+0 = -0; a NaN sorts first).
 *  d        1 <= d <= INT32_MAX. */
gptq_status_t gptq_act_order(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, int32_t* perm, void* stream);

/* The Hessian in the order perm: Hp[i][j] = H[perm[i]][perm[j]] for j <= i
 * (lower triangles; H's lower triangle is read). Pass Hp to gptq_prepare_hinv
 * to get the factor that gptq_quantize_layer_ordered takes.
 *  H, Hp    device [d][ldh] / [d][ldhp], both h_dtype (GPTQ_F32 | GPTQ_F64);
 *           Hp may not alias H.
 *  perm     device int32 [d], a permutation of 0 .. d-1 (entries outside
 *           [0, d) are read as 0: the result is then meaningless, but every
 *           access stays inside H). */
gptq_status_t gptq_permute_hessian(const void* H, int32_t h_dtype, int64_t d, int64_t ldh, const int32_t* perm,
                                   void* Hp, int64_t ldhp, void* stream);

/* gptq_quantize_layer with the columns quantized in the order perm instead of
 * the natural one (act-order). W and every output stay in natural column
 * order; U must be the factor of the Hessian in that order
 * (gptq_permute_hessian, then gptq_prepare_hinv). Same sources as
 * gptq_act_order; the group readings are this library's:
 *  static_groups 0: groups are runs of group_size columns in the order perm,
 *           each fitted at its first column on the current (error-updated)
 *           weights, as in natural order; group k of the outputs is the k-th
 *           such run.
 *  static_groups 1: the grid of every natural group of group_size columns is
 *           fitted on the original W before the loop; each column is rounded on
 *           its natural group's grid wherever the order puts it; group k is
 *           natural columns [k * group_size, (k + 1) * group_size).
 *  With group_size 0 (one grid per row) both give the same result.
 *  perm     device int32 [d], a permutation of 0 .. d-1 (entries outside
 *           [0, d) are read as 0: the result is then meaningless, but every
 *           access stays inside the buffers).
 *  g_idx    device int32 [d], may be NULL: the group number of every natural
 *           column (0 for one grid per row).
 *  Other arguments, sizes and the workspace as gptq_quantize_layer; d <= INT32_MAX. */
gptq_status_t gptq_quantize_layer_ordered(const void* W, int32_t w_dtype, int64_t m, int64_t d, int64_t ldw,
                                          const void* U, int32_t u_dtype, int64_t ldu, const gptq_qcfg_t* cfg,
                                          const int32_t* perm, int32_t static_groups, uint32_t* qcodes,
                                          float* scales, uint8_t* zeros, int32_t* g_idx, float* W_hat,
                                          float* err_sq, void* workspace, size_t ws_bytes, void* stream);

/* Generation with the packed weights: y = W_hat x for one token (batch 1),
 * the weights dequantized on the fly, y[r] = sum_j s[r][g(j)] (c[r][j] - z[r][g(j)]) x[j]
 * with g(j) = j / group_size (0 for one grid per row). FDE breakdown, section
 * 01: an inference kernel reads the 3/4-bit weights and dequantizes them on
 * the fly; nubint review, "Key findings": 3-bit OPT-175B generation speedups.
 *  qcodes   device uint32 [m][d * bits / 32], the bitstream gptq_quantize_layer
 *           writes (4-byte aligned).  scales / zeros: device [m][ngroups] as
 *           written by gptq_quantize_layer.
 *  bits     2, 3, 4 or 8 (ternary codes use bits = 2).
 *  group_size 0, or a multiple of 32 dividing d (natural column groups; for
 *           the g_idx layout of act-order without static groups see
 *           gptq_gemv_prepare_act_order).
 *  x        device fp16 [d], 16-byte aligned.   y device float [m], out.
 *  d % 32 == 0. Sums are carried in fp32: per 32-code chunk sum c x and
 *  sum x, then s (sum c x - z sum x), added over chunks and across a wave. */
gptq_status_t gptq_dequant_gemv(const uint32_t* qcodes, const float* scales, const uint8_t* zeros, int64_t m,
                                int64_t d, int32_t bits, int32_t group_size, const void* x, float* y, void* stream);

/* Act-order codes for the generation product (ordered quantization without
 * static groups: codes in natural column order, g_idx[j] the group of column
 * j). Same sources as gptq_dequant_gemv and gptq_act_order. The group index
 * scatters a row's groups over the columns; this call, made once per layer,
 * sorts the columns by group (ties by column index) into col_perm, so that
 * group k is slots [k group_size, (k + 1) group_size), and rewrites every row's
 * codes in that order. gptq_dequant_gemv_perm then computes the same y as
 * sum_j s[r][g_idx[j]] (c[r][j] - z[r][g_idx[j]]) x[j] from the rewritten codes,
 * the unchanged scales and zeros, and x read in col_perm order.
 *  qcodes   device uint32 [m][d * bits / 32], natural order (4-byte aligned).
 *  g_idx    device int32 [d], as gptq_quantize_layer_ordered writes it.
 *  qcodes_out device uint32 [m][d * bits / 32], out; may not alias qcodes.
 *  col_perm device int32 [d], out.
 *  info     device int32, out: 0 when every group holds exactly group_size
 *           columns and every g_idx lies in [0, d / group_size); otherwise the
 *           number of faults found (col_perm and qcodes_out are then
 *           meaningless, but every access stays in bounds).
 *  bits     2, 3, 4 or 8;  group_size a multiple of 32 dividing d (> 0). */
gptq_status_t gptq_gemv_prepare_act_order(const uint32_t* qcodes, const int32_t* g_idx, int64_t m, int64_t d,
                                          int32_t bits, int32_t group_size, uint32_t* qcodes_out, int32_t* col_perm,
                                          int32_t* info, void* stream);

/* gptq_dequant_gemv for codes in col_perm order (gptq_gemv_prepare_act_order):
 * x_perm[p] = x[col_perm[p]] is gathered into the caller's x_perm (device fp16
 * [d], 16-byte aligned, not aliasing x; its contents are overwritten), then
 * y = W x as gptq_dequant_gemv on (qcodes, scales, zeros, x_perm). Entries of
 * col_perm outside [0, d) read x[0]. Other arguments as gptq_dequant_gemv. */
gptq_status_t gptq_dequant_gemv_perm(const uint32_t* qcodes, const float* scales, const uint8_t* zeros, int64_t m,
                                     int64_t d, int32_t bits, int32_t group_size, const int32_t* col_perm,
                                     const void* x, void* x_perm, float* y, void* stream);

/* Bit packing of integer codes (one byte per code) into the row-wise LSB-first
 * bitstream gptq_quantize_layer writes (which packs in its own epilogue).
 * FDE breakdown, section 01: the output is 3-bit (or 4-bit) weights that an
 * inference kernel dequantizes on the fly; the layout is this library's.
 *  codes    device uint8 [m][d], values < 2^bits.   out device uint32 [m][d*bits/32].
 *  bits     2, 3, 4 or 8; d * bits % 32 == 0. */
gptq_status_t gptq_pack_codes(const uint8_t* codes, int64_t m, int64_t d, int32_t bits,
                              uint32_t* out, void* stream);

/* ---------------------------------------------------------------------------
 * Tracing (instrumentation, not a step of the method): device time per kernel
 * family. While a trace is active on the calling host thread, every kernel the
 * library launches from that thread is bracketed by two HIP events recorded on
 * the stream it is launched on, and the launch's executed work is noted
 * (floating-point operations the matrix cores execute, padding included, for
 * the SYRK and the trailing GEMM; 0 for the others).
 * gptq_trace_start: begins a trace on this thread (GPTQ_ERR_INVALID_ARG if one
 *           is active). Events are created on first use and kept for reuse.
 * gptq_trace_stop: ends it, waits for the last recorded event, and writes, for
 *           the families k < n, launches[k], ms[k] (summed event durations) and
 *           work[k] (any pointer may be NULL). Returns GPTQ_ERR_HIP when an
 *           event could not be created, recorded or read.
 * gptq_trace_family: the name of family k (static storage). */
enum {
  GPTQ_TRACE_SYRK = 0, GPTQ_TRACE_SYRK_REDUCE = 1, GPTQ_TRACE_CHAIN_LOAD = 2, GPTQ_TRACE_CHAIN_PANEL = 3,
  GPTQ_TRACE_CHAIN_UPDATE = 4, GPTQ_TRACE_CHAIN_MERGE = 5, GPTQ_TRACE_CHAIN_STORE = 6, GPTQ_TRACE_QUANT_PREP = 7,
  GPTQ_TRACE_COLLOOP = 8, GPTQ_TRACE_ESPLIT = 9, GPTQ_TRACE_TGEMM = 10, GPTQ_TRACE_PACK = 11,
  GPTQ_TRACE_ORDER = 12, GPTQ_TRACE_GEMV = 13, GPTQ_TRACE_SYRK_TRANSPOSE = 14, GPTQ_TRACE_FAMILIES = 15
};
int32_t gptq_trace_start(void);
int32_t gptq_trace_stop(int64_t* launches, double* ms, double* work, int32_t n);
const char* gptq_trace_family(int32_t k);

#ifdef __cplusplus
}
#endif

#endif /* GPTQ_MI355X_H */
