/*
 * any4.h: C ABI of the MI355X (gfx950) any4 quantizer.
 *
 * The operation is the per-row quantizer of "any4: Learned 4-bit Numeric
 * Representation for LLMs" (arXiv 2507.04610): group-wise asymmetric min/max
 * scaling of each weight row (Section 2.5.1, Eq. 1-2), a LUT of 2^n values per
 * row learned by weighted k-means on the scaled row, with sample weights
 * alpha_{i,j} * E|x_j| (Section 4.1: E-step Eq. 18, M-step Eq. 23; k-means++
 * initialisation per Appendix C.2), and storage as n-bit codes plus an fp16 LUT
 * per row and an fp16 scale and offset per group (Section 2.4.1).
 *
 * Conventions for every entry point:
 *  - All array pointers are DEVICE pointers unless stated otherwise; every call
 *    is asynchronous on `stream` (a hipStream_t; NULL = the null stream).
 *  - The caller allocates and owns every buffer, including the workspace; the
 *    library never allocates device memory and keeps no mutable global state,
 *    so concurrent calls on different streams are safe.
 *  - Argument validation is synchronous and happens before any launch: on a
 *    validation error nothing is launched and no output is written.
 *  - Return value: an ANY4_* status; no C++ exception crosses the ABI.
 *  - Layouts are row-major and contiguous.
 *  - Results are a pure function of (W, act_absmean, params, row_offset,
 *    matrix_index): repeat runs are bit-identical, and quantizing rows
 *    [r0, r0 + n) with row_offset = r0 gives the same bits as those rows of a
 *    whole-matrix call.
 */
#ifndef ANY4_H
#define ANY4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hipStream_t;

/* element type of W */
enum { ANY4_F32 = 0, ANY4_BF16 = 1 };

/* status codes */
enum {
  ANY4_OK = 0,
  ANY4_ERR_INVALID_ARG = 1,  /* bad pointer, size, group, cluster count, ... */
  ANY4_ERR_UNSUPPORTED = 2,  /* valid but outside what the kernels handle (e.g. K > 32768) */
  ANY4_ERR_WORKSPACE = 3,    /* workspace missing or smaller than any4_workspace_bytes() */
  ANY4_ERR_HIP = 4,          /* a HIP launch failed (hipGetLastError) */
  ANY4_ERR_NONFINITE = 5     /* device-detected bad row, read with any4_read_device_status() */
};

/* One weight matrix and its outputs.
 *   w            [n_rows, n_cols] of w_dtype (fp32, or bf16 bits as uint16)
 *   act_absmean  [n_cols] fp32, E|x_j| per input channel (Section 4.1, calibration
 *                statistic); must be finite and >= 0
 *   row_offset   added to the row index in the Philox counter; use it when a
 *                matrix is quantized in row shards
 *   matrix_index a Philox counter word; give each matrix of a batch its own
 *   codes        out [n_rows, n_cols/2] uint8: byte m = q[2m] | q[2m+1] << 4
 *   lut          out [n_rows, n_clusters] IEEE fp16 bits, centroids in draw order
 *   scale        out [n_rows, n_cols/group] fp16 alpha (Eq. 2)
 *   offset       out [n_rows, n_cols/group] fp16 beta = group minimum (Eq. 2)
 *   objective    out [n_rows] fp64 J = sum_j a_j (w_S_j - lut_q_j)^2 with the
 *                fp32 centroids, or NULL
 * A row whose W or E|x| holds a non-finite value, whose E|x| has a negative entry,
 * or whose alpha or sample weight alpha*E|x| is non-finite or above 2^64, gets
 * all-zero codes/lut/scale/offset and a NaN objective, and sets ANY4_ERR_NONFINITE
 * in the workspace status word. */
typedef struct {
  const void* w;
  int32_t w_dtype;
  int32_t matrix_index;
  int64_t n_rows;
  int64_t n_cols;
  const float* act_absmean;
  int64_t row_offset;
  uint8_t* codes;
  uint16_t* lut;
  uint16_t* scale;
  uint16_t* offset;
  double* objective;
} any4_matrix;

/* Method variants (the paper's ablations), OR-ed into any4_params.variant; 0 selects
 * the defaults used everywhere else in the paper. */
enum {
  /* sample weights (Appendix C.1, Table A3): Eq. 23's alpha * E|x| (default), E|x|
   * alone, or none (every weight 1: plain k-means on the scaled weights) */
  ANY4_WEIGHT_ALPHA_ACT = 0, ANY4_WEIGHT_ACT = 1, ANY4_WEIGHT_NONE = 2,
  /* initialization (Appendix C.2, Table A4): k-means++ (default); random: k distinct
   * elements drawn one after another with probability proportional to the sample
   * weight (the same Philox stream); uniform: the integer levels (0..2^n-1, or
   * 1-2^(n-1)..2^(n-1) under symmetric scaling, i.e. int4's -7..8); greedy k-means++
   * (scikit-learn's default form): every centre after the first keeps the best of
   * 2 + floor(ln n_clusters) D^2 candidates (candidate s from Philox counter word
   * t + 16 r + 65536 s), judged by the exact integer potential of the sampling step */
  ANY4_INIT_KMEANSPP = 0, ANY4_INIT_RANDOM = 1 << 2, ANY4_INIT_UNIFORM = 2 << 2,
  ANY4_INIT_GREEDY = 3 << 2,
  /* symmetric scaling (Section 2.5.1, Eq. 3): alpha = max|w| / 2^(n-1), beta = 0 */
  ANY4_SCALE_SYMMETRIC = 1 << 4,
  /* not a method variant: run every one of `iters` Lloyd rounds.  By default a row stops
   * once a round leaves every centroid's bits unchanged, since each later round would
   * give the same assignment, sums and centroids again; the outputs are the same bits
   * either way, only the time differs. */
  ANY4_ALL_ROUNDS = 1 << 5
};
/* restarts (n_init): the whole k-means runs from n initializations (restart r draws
 * from Philox counters t + 16 r) and each row keeps the run with the lowest final
 * objective (the earliest on ties).  n in 1..256; needs the larger workspace that
 * any4_workspace_bytes reports. */
#define ANY4_RESTARTS(n) (((n) - 1) << 8)

/* group:      power of two, 2 <= group, n_cols % group == 0 (Section 2.5.1; 128 is
 *             the paper's default)
 * n_clusters: 2, 4, 8 or 16 (any1..any4; Qmax - Qmin = n_clusters - 1)
 * iters:      Lloyd rounds (E-step then M-step), >= 0, followed by one final E-step
 * variant:    0, or ANY4_WEIGHT_* | ANY4_INIT_* | ANY4_SCALE_SYMMETRIC | ANY4_RESTARTS(n),
 *             optionally with ANY4_ALL_ROUNDS; any other bit is an invalid argument
 * seed:       Philox4x32-10 key for k-means++ and random initialization */
typedef struct {
  int32_t group;
  int32_t n_clusters;
  int32_t iters;
  int32_t variant;
  uint64_t seed;
} any4_params;

/* Size of the workspace any4_quantize needs for this batch: a device status word and
 * padding, plus, with restarts, one candidate set of outputs per matrix (codes, LUT,
 * objectives, centroids, picks).  Validates the arguments like any4_quantize. */
int any4_workspace_bytes(const any4_matrix* mats, int32_t count, const any4_params* params,
                         size_t* bytes_out);

/* Quantize `count` matrices (host array of descriptors) in one call: every row of
 * every matrix is scaled, seeded with k-means++, refined by `iters` Lloyd rounds,
 * finally assigned, and emitted.  Per matrix, n_cols must be even and at most
 * 32768; n_rows may be 0.  The workspace (device, >= any4_workspace_bytes) holds
 * the status word; it is cleared by this call. */
int any4_quantize(const any4_matrix* mats, int32_t count, const any4_params* params,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* Synchronizes `stream`, then returns the status word a previous any4_quantize
 * left in `workspace` (ANY4_OK or ANY4_ERR_NONFINITE), or ANY4_ERR_HIP. */
int any4_read_device_status(const void* workspace, hipStream_t stream);

/* Static English text for a status code. */
const char* any4_status_string(int status);

/* Launch geometry the library uses for rows of n_cols columns: each row is one
 * workgroup of *waves_per_row wave64s, each lane holding *elems_per_lane
 * consecutive columns.  Host-only; returns ANY4_ERR_INVALID_ARG for bad pointers
 * or n_cols outside [2, 32768]. */
int any4_launch_geometry(int64_t n_cols, int32_t* elems_per_lane, int32_t* waves_per_row);

/* ---- stage entry points: the same device code as any4_quantize, stopped after
 * one step, for parity tests against the CPU oracle.  One matrix each; the
 * any4_matrix output fields that a stage does not produce are ignored. ---- */

/* Eq. 1-2 scaling and Eq. 23 sample weights: w_s [N,K] fp32 scaled row,
 * alpha/beta [N, K/group] fp32, a [N,K] fp32 = alpha_{g(j)} * E|x_j|. */
int any4_stage_scale(const any4_matrix* m, const any4_params* params, float* w_s,
                     float* alpha, float* beta, float* a, hipStream_t stream);

/* Scaling then k-means++ (Appendix C.2): c0 [N, n_clusters] fp32 initial
 * centroids in draw order, picks [N, n_clusters] int32 column of each draw
 * (-1 when all sampling weights were 0 and the centre was copied). */
int any4_stage_seed(const any4_matrix* m, const any4_params* params, float* c0,
                    int32_t* picks, hipStream_t stream);

/* Scaling, then ONE Lloyd round from the given centroids c_in [N, n_clusters]:
 * assign [N,K] uint8 E-step result (Eq. 18, lowest index on ties), c_out
 * [N, n_clusters] M-step result (Eq. 23; an empty cluster keeps its value),
 * objective [N] fp64 J at c_in with that assignment (may be NULL). */
int any4_stage_lloyd_step(const any4_matrix* m, const any4_params* params, const float* c_in,
                          uint8_t* assign, float* c_out, double* objective, hipStream_t stream);

/* Sorted-row Lloyd, the Lloyd-Max form of the per-row 1-D clustering (Section 2.5;
 * Lloyd 1982, Max 1960): `params->iters` rounds of Eq. 18 assignment and Eq. 23 update
 * from the centroids c_in [N, n_clusters] fp32, writing c_out [N, n_clusters] fp32.
 * Inputs are the scaled rows w_s [N, K] and sample weights a [N, K] (fp32, as written by
 * any4_stage_scale; device pointers, not modified).  Each row is sorted once with fp64
 * prefix sums of a and a*w_s; a round costs one binary search per switch point and
 * two prefix differences per cluster instead of a pass over the row.  The assignment
 * rule is the same as any4_quantize's, so the fixed points are too; the sums differ
 * only in fp64 rounding order.  Uses m->n_rows and m->n_cols only (other fields
 * ignored); params->group is checked but unused and the symmetric flag of
 * params->variant selects the scaled range.  Rows of at most 16384 columns are sorted
 * in LDS and need no workspace (workspace may be NULL); rows of 16386 to 32768 columns
 * are sorted as two halves and keep their sorted sample weights in `workspace` (device,
 * 16-byte aligned, at least any4_stage_lloyd_sorted_workspace_bytes(N, K) bytes, else
 * ANY4_ERR_WORKSPACE; its contents on entry do not matter and it may be reused once
 * the call has completed on `stream`).  ANY4_ERR_UNSUPPORTED past 32768 columns;
 * ANY4_ERR_INVALID_ARG for a NULL pointer with n_rows > 0, n_cols < 2 or odd, or bad
 * params.  A row holding a non-finite w_s or a (which any4_stage_scale reports through
 * its status) gives unspecified centroids for that row only.  The caller owns every
 * buffer.  Asynchronous on `stream`. */
int any4_stage_lloyd_sorted(const any4_matrix* m, const any4_params* params, const float* w_s,
                            const float* a, const float* c_in, float* c_out, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes any4_stage_lloyd_sorted needs for n_rows rows of n_cols columns, in
 * *bytes_out: 0 up to 16384 columns, n_rows * 3 * 16384 * 4 from 16386 to 32768.
 * Host-only.  ANY4_ERR_INVALID_ARG for a NULL bytes_out, n_rows < 0, or n_cols < 2 or
 * odd; ANY4_ERR_UNSUPPORTED past 32768 columns or 2^31 rows. */
int any4_stage_lloyd_sorted_workspace_bytes(int64_t n_rows, int64_t n_cols, size_t* bytes_out);

/* Emission only: codes, lut, scale, offset of `m` from assign [N,K] uint8,
 * c [N, n_clusters] fp32, alpha/beta [N, K/group] fp32 (Section 2.4.1 layout). */
int any4_stage_pack(const any4_matrix* m, const any4_params* params, const uint8_t* assign,
                    const float* c, const float* alpha, const float* beta, hipStream_t stream);

/* The full path like any4_quantize for one matrix, additionally writing the fp32
 * centroids before the fp16 cast, c_final [N, n_clusters], and the k-means++
 * picks [N, n_clusters] (either may be NULL). */
int any4_stage_full(const any4_matrix* m, const any4_params* params, float* c_final,
                    int32_t* picks, void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The batched path of any4_quantize (the same launches: one per row geometry over
 * every matrix of the batch, longer rows first), additionally writing for each matrix
 * i the fp32 centroids before the fp16 cast, c_final[i] [n_rows_i, n_clusters], and
 * the k-means++ picks, picks[i] [n_rows_i, n_clusters] (of the restart that was kept).
 * c_final and picks are host arrays of `count` device pointers; either array, or any
 * of its entries, may be NULL.  Arguments, workspace and errors as any4_quantize. */
int any4_stage_quantize_batch(const any4_matrix* mats, int32_t count, const any4_params* params,
                              float* const* c_final, int32_t* const* picks, void* workspace,
                              size_t workspace_bytes, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): any4_quantize without a workspace.
 * The status word and, with restarts, the candidate outputs live in a library-owned
 * device array of ANY4_NOALLOC_SCRATCH_BYTES on each device (a static device array,
 * held until the process ends); the call allocates nothing.  The batch may hold at
 * most ANY4_NOALLOC_MAX_MATRICES matrices (else ANY4_ERR_UNSUPPORTED) and need at most
 * ANY4_NOALLOC_SCRATCH_BYTES of workspace as any4_workspace_bytes counts it (else
 * ANY4_ERR_WORKSPACE), both checked before any launch; without restarts every batch
 * fits.  status_out: optional device pointer that receives, in stream order, this
 * call's status word (ANY4_OK or ANY4_ERR_NONFINITE).  The array keeps the last call's
 * contents, and this call clears what it reads; calls that overlap on one GPU (other
 * streams or threads) share it and race, so serialize them.  Otherwise the same as
 * any4_quantize, with the same outputs bit for bit. */
#define ANY4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
#define ANY4_NOALLOC_MAX_MATRICES 64
int any4_quantize_noalloc(const any4_matrix* mats, int32_t count, const any4_params* params,
                          uint32_t* status_out, hipStream_t stream);

/* ---- bookends: the calibration statistic the quantizer consumes and the
 * dequantization of what it emits. ---- */

/* Workspace for any4_act_absmean: fp64 partial sums over token slices (the slice
 * plan depends only on n_tokens and n_cols).  Returns ANY4_ERR_INVALID_ARG for a
 * NULL bytes_out, n_tokens < 1 or n_cols < 1. */
int any4_act_absmean_workspace_bytes(int64_t n_tokens, int64_t n_cols, size_t* bytes_out);

/* E|x_j|, the mean absolute activation of each input channel over a calibration batch
 * (Section 4.1; the sample weights of Eq. 23 are alpha_{i,j} * E|x_j|):
 *   act_absmean[j] = fp32( (sum over t of |x[t, j]|, in fp64) / n_tokens ).
 *   x            [n_tokens, n_cols] row-major activations, fp32 or bf16 bits (x_dtype)
 *   act_absmean  out [n_cols] fp32, ready to pass to any4_quantize
 *   workspace    device, >= any4_act_absmean_workspace_bytes(n_tokens, n_cols)
 * The fp64 sums are taken over fixed token slices and added in slice order, so the
 * result is deterministic; against a sequential fp64 sum it can differ only through
 * the rounding of that sum, i.e. by at most one fp32 ulp.  Inf and NaN inputs
 * propagate to their channel.  Errors: ANY4_ERR_INVALID_ARG (NULL pointer, n_tokens
 * or n_cols < 1, bad dtype), ANY4_ERR_WORKSPACE, ANY4_ERR_HIP. */
int any4_act_absmean(const void* x, int32_t x_dtype, int64_t n_tokens, int64_t n_cols,
                     float* act_absmean, void* workspace, size_t workspace_bytes,
                     hipStream_t stream);

/* Dequantization (Section 2.5.2, Eq. 4: dequant(w_Q) = alpha * w_Q + beta, w_Q the
 * row's LUT entry at the element's code):
 *   w_out[i, j] = fl(fl(alpha_{i,g(j)} * LUT_i[q_ij]) + beta_{i,g(j)})
 * evaluated in fp32 from the fp16 LUT, scale and offset (product and sum rounded
 * separately), written as fp32 (out_dtype ANY4_F32) or as bf16 rounded to nearest
 * even (ANY4_BF16).  Reads the codes, lut, scale and offset fields of `m` (its w,
 * act_absmean and objective are not used); params->group and params->n_clusters must
 * be the ones the codes were made with (iters and seed are ignored).  A code at or
 * above n_clusters gives NaN.  w_out is [n_rows, n_cols], caller-allocated.
 * Errors: ANY4_ERR_INVALID_ARG (NULL pointer, odd n_cols, group not dividing n_cols,
 * bad n_clusters or out_dtype), ANY4_ERR_HIP. */
int any4_dequantize(const any4_matrix* m, const any4_params* params, void* w_out,
                    int32_t out_dtype, hipStream_t stream);

/* The quantized matrix applied to a few tokens without materializing it (the inference
 * consumer; the paper's tinygemm kernels dequantize on the fly before the multiply,
 * Section 4.2): y[t, i] = sum_j x[t, j] * w_hat[i, j], w_hat the Eq. 4 dequantization
 * of any4_dequantize, accumulated in fp32.
 *   m       codes, lut, scale, offset as emitted (w, act_absmean, objective unused)
 *   params  group and n_clusters of the codes (iters, seed, variant ignored)
 *   x       [n_tokens, n_cols] activations, fp32 or bf16 bits (x_dtype)
 *   y       out [n_tokens, n_rows] fp32
 * Each 16-column block is evaluated as alpha * sum x*LUT[q] + beta * sum x; against an
 * exact evaluation of the Eq. 4 definition the error stays within 1e-5 of
 * sum_j |x_j| (|alpha*LUT[q_j]| + |beta|), and the summation order is fixed (repeated calls
 * give identical bits).  Supports 1 <= n_tokens <= 8, n_cols and group multiples of 16,
 * n_rows and n_cols below 2^31, codes 8-byte and x 16-byte aligned (ANY4_ERR_UNSUPPORTED
 * otherwise; use any4_dequantize and a GEMM for larger batches).  A code at or above
 * n_clusters gives NaN.  Errors:
 * ANY4_ERR_INVALID_ARG (NULL pointer, bad sizes or dtype), ANY4_ERR_UNSUPPORTED,
 * ANY4_ERR_HIP. */
int any4_lut_gemv(const any4_matrix* m, const any4_params* params, const void* x, int32_t x_dtype,
                  int64_t n_tokens, float* y, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ANY4_H */
