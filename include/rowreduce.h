/*
 * rowreduce.h -- C ABI of librowreduce.so: row-wise reduce-then-rescale
 * kernels for AMD MI355X (gfx950, CDNA4).
 *
 * Operations (each row of a row-major [M, N] matrix is independent):
 *   rr_rmsnorm            y = x * rsqrt(mean(x^2) + eps) * gamma
 *   rr_fused_add_rmsnorm  residual <- residual + x;  y = rmsnorm(residual) * gamma
 *   rr_layernorm          y = (x - mean) * rsqrt(var + eps) * gamma + beta
 *   rr_softmax_rows       y = exp(x - m) / d with the online normaliser (m, d)
 *   rr_softmax_rows_ex    the same, or log-softmax, optionally under a causal
 *                         rule that does not read masked keys
 *
 * Sources (web pages, cited by title and section):
 *   [P1] "两个融合算子：RMSNorm 与 online softmax" (daleiyang.github.io)
 *   [P2] "GPU Kernel 工程（04）：共享内存与 reduction——softmax、LayerNorm 与
 *        online softmax" (arganzheng.life)
 *   [P4] "Softmax 与归一化" (anrans.github.io ai-infra-handbooks)
 *   [P5] "RMSNorm、Softmax 与在线归约" (notes.kuangjux.top)
 *
 * Conventions shared by every entry point
 *   - Memory: every data pointer is a DEVICE pointer owned by the caller
 *     (allocated on the device that is current when the call is made).  The
 *     library allocates nothing, frees nothing and keeps no per-call state.
 *   - Layout: row-major and contiguous; element (i, j) of an [M, N] matrix is
 *     at offset i * N + j; gamma is a vector of N (or H) elements.  The
 *     *_strided entry points take a row stride per matrix instead.
 *   - dtype: RR_F32 (IEEE binary32) or RR_BF16 (bfloat16).  All arithmetic is
 *     fp32; bf16 inputs widen exactly and outputs round to nearest even once.
 *   - Streams: `stream` is a hipStream_t (NULL = the null stream).  Calls are
 *     asynchronous: they enqueue kernels and return; the caller synchronises.
 *     Same-stream order is the only ordering the library relies on.  The
 *     calls only enqueue kernels (no memsets, copies or host callbacks), so
 *     a caller may capture them into a HIP graph; a captured call reads its
 *     buffers when the graph replays.  (The one-kernel form of the split row
 *     tags its workspace slots from per-row epochs that it reads and
 *     advances on the device, so each replay tags them afresh.)
 *   - Errors: arguments are checked on the host before anything is enqueued;
 *     a failed check returns a non-zero rr_status and enqueues nothing.
 *     M == 0 is a successful no-op.  An empty row (N or H < 1) is the
 *     caller's error ([P1] section "四、数值上到底安不安全": the normaliser is
 *     only defined for a non-empty row).  A failure reported by the HIP
 *     runtime when launching returns RR_ERR_HIP.  rr_last_error_message()
 *     gives the detail for the calling thread.
 *   - Alignment: rows whose pointers are 16-byte aligned and whose width is a
 *     multiple of 4 (fp32) or 8 (bf16) elements use 16-byte vector accesses;
 *     a softmax reading bf16 and writing fp32 reads 4 elements (8 bytes) per
 *     access, so there input rows 8-byte aligned and a width that is a
 *     multiple of 4 suffice.  A call whose input and output rows (and a
 *     fused call's residual rows) start at the same element offset within a
 *     vector (contiguous rows of any width, in place, column slices with
 *     equal strides) is cut into vectors at aligned addresses: whole vectors
 *     inside each row, its first and last vector element by element, nothing
 *     outside the row read or written.  A cut norm may read gamma (and beta)
 *     in whole aligned 16-byte blocks: the bytes that share the blocks
 *     holding their first and last elements may be read, and are ignored.
 *     Anything else runs a scalar path.  Each path gives the same results up
 *     to rounding order.  Any N >= 1 is accepted.
 *   - Determinism: a given (op, M, N, dtypes, alignment) always runs the same
 *     kernel with the same reduction order, so results are bitwise
 *     reproducible run to run; no floating-point atomics are used.
 */
#ifndef ROWREDUCE_H
#define ROWREDUCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum rr_dtype {
  RR_F32 = 0,
  RR_BF16 = 1
} rr_dtype;

typedef enum rr_status {
  RR_OK = 0,
  RR_ERR_INVALID_ARG = 1,  /* null pointer, bad size, unknown dtype, bad aliasing */
  RR_ERR_UNSUPPORTED = 2,  /* valid request the library cannot run (size limits, forced variant) */
  RR_ERR_WORKSPACE = 3,    /* workspace missing or smaller than rr_softmax_rows_workspace_bytes */
  RR_ERR_HIP = 4           /* the HIP runtime reported an error */
} rr_status;

/*
 * rr_rmsnorm -- RMSNorm of each row.
 *   y[i, j] = x[i, j] * r_i * gamma[j],  r_i = 1 / sqrt( (1/H) * sum_j x[i, j]^2 + eps )
 * eps is added to the mean square inside the square root and nothing is
 * subtracted from x ([P5] section "RMSNorm 归约什么"; [P2] sections 二.1 and
 * 八.1; [P4] section "LayerNorm 与 RMSNorm").
 *   y      [M, H] output, dtype `dtype`; may be the same pointer as x (in place)
 *   x      [M, H] input, dtype `dtype`
 *   gamma  [H] scale, dtype `dtype`
 *   M >= 0 rows, H >= 1 elements per row, eps >= 0 finite
 * The sum of squares is accumulated in fp32, so |x| must stay below about
 * 1.8e19 (squares beyond the fp32 range are not supported; the same holds
 * for the spread about the mean in rr_layernorm).  Rows longer than 2^30
 * elements (H or N, every entry point) return RR_ERR_UNSUPPORTED; there is
 * no limit on M beyond memory.  Returns RR_ERR_INVALID_ARG for
 * null pointers (M > 0), M < 0, H < 1, a bad eps, an unknown dtype, or y
 * overlapping x without being equal to it, or gamma overlapping y.
 */
rr_status rr_rmsnorm(void* y, const void* x, const void* gamma, int64_t M, int64_t H,
                     float eps, rr_dtype dtype, void* stream);

/*
 * rr_fused_add_rmsnorm -- residual add followed by RMSNorm, in one pass.
 *   h[i, j]        = round_dtype( x[i, j] + residual[i, j] )   (sum in fp32)
 *   residual[i, j] <- h[i, j]
 *   y[i, j]        = h[i, j] * r_i * gamma[j],  r_i from the stored h
 * ([P4] section "算子融合：fused_add_rms_norm"; [P2] section 八.3: read x and
 * the residual once, write the new residual and the normalised output.)
 * y is computed from the residual as stored, so the result equals an add
 * followed by rr_rmsnorm.
 *   y         [M, H] output; may be the same pointer as x
 *   residual  [M, H] input and output (updated in place)
 *   x         [M, H] input
 *   gamma     [H]
 * All four have dtype `dtype`.  residual must not overlap x, y or gamma;
 * y may equal x but must not partly overlap it.  Other errors as rr_rmsnorm.
 */
rr_status rr_fused_add_rmsnorm(void* y, void* residual, const void* x, const void* gamma,
                               int64_t M, int64_t H, float eps, rr_dtype dtype,
                               void* stream);

/*
 * rr_layernorm -- LayerNorm of each row.
 *   mu_i = (1/H) sum_j x[i, j],   var_i = (1/H) sum_j (x[i, j] - mu_i)^2,
 *   y[i, j] = (x[i, j] - mu_i) / sqrt(var_i + eps) * gamma[j] + beta[j]
 * ([P2] section 八.2; [P4] section "LayerNorm 与 RMSNorm" and its LayerNorm
 * exercise.)  The sums are taken about a shift K, the row's first element:
 * one reduction carries sum(x - K) and sum((x - K)^2), so rows whose mean is
 * far larger than their spread keep their precision.  A row whose first
 * element lies more than two standard deviations from its mean (where that
 * variance would cancel and x - K would be rounded at the scale of the
 * distance) is summed once more about its mean.  Rows up to 65536 elements
 * are held on chip; longer or unaligned rows are read twice (three times for
 * such an outlying first element).
 *   y      [M, H] output, dtype `dtype`; may be the same pointer as x
 *   x      [M, H] input (finite values)
 *   gamma  [H] scale
 *   beta   [H] shift, or NULL for none
 * All in dtype `dtype`.  Errors as rr_rmsnorm (beta must not overlap y).
 */
rr_status rr_layernorm(void* y, const void* x, const void* gamma, const void* beta, int64_t M,
                       int64_t H, float eps, rr_dtype dtype, void* stream);

/*
 * rr_softmax_rows_workspace_bytes -- device workspace rr_softmax_rows needs
 * for this shape (0 when the chosen kernel needs none).  Very long rows with
 * few rows are split over several workgroups; each writes its chunk's
 * (m, d) pair to a 16-byte slot of the workspace and the row's slots are
 * merged ([P4] section "练习", the vocabulary-split exercise): M * S slots
 * (S chunks per row), then one 4-byte epoch per row, padded to a multiple of
 * 16 bytes.  The size covers rows at any address (a row starting inside a
 * vector may take one more chunk).  Host-only; returns 0 for invalid
 * arguments.
 */
size_t rr_softmax_rows_workspace_bytes(int64_t M, int64_t N, rr_dtype in_dtype,
                                       rr_dtype out_dtype);

/*
 * rr_softmax_rows -- softmax of each row.
 *   m_i = max_j x[i, j],  d_i = sum_j exp(x[i, j] - m_i),  y[i, j] = exp(x[i, j] - m_i) / d_i
 * computed with the online normaliser: partial pairs (m, d) over parts of a
 * row combine by (m1,d1) (+) (m2,d2) = (m, d1 e^(m1-m) + d2 e^(m2-m)),
 * m = max(m1, m2), identity (-inf, 0) ([P1] sections "二、递推式怎么来的" and
 * "三、结合律"; [P5] sections "Online Softmax 为什么要重缩放旧的和" and
 * "从逐元素更新到合并两个 tile"; [P2] section 七.3).
 *   y          [M, N] output, dtype out_dtype
 *   x          [M, N] input, dtype in_dtype; entries may be -inf (masked);
 *              +inf and NaN inputs are not supported
 *   workspace  device buffer of at least rr_softmax_rows_workspace_bytes(M, N,
 *              in_dtype, out_dtype) bytes, 16-byte aligned (may be NULL when
 *              that size is 0); contents on entry are ignored (the
 *              one-kernel split tags its slots with per-row epochs kept in
 *              the workspace, which it advances, so any later call of any
 *              shape may reuse it); calls that overlap in time must not
 *              share a workspace
 * Masked entries produce exactly 0; a row whose entries are all -inf
 * produces NaN everywhere (-inf - (-inf)).  Probabilities below 2^-126
 * come out as bf16 subnormals when out_dtype is RR_BF16, and as 0 when it
 * is RR_F32 (an absolute error below 1.2e-38).  In place (y == x) is allowed
 * when in_dtype == out_dtype; otherwise x and y must not overlap.
 * Returns RR_ERR_WORKSPACE when the workspace is needed and missing or too
 * small; other errors as rr_rmsnorm.
 */
rr_status rr_softmax_rows(void* y, const void* x, int64_t M, int64_t N, rr_dtype in_dtype,
                          rr_dtype out_dtype, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Options of rr_softmax_rows_ex.  A NULL options pointer means all zero:
 * plain softmax over every key.
 *   log_output     0: y = exp(x - m) / d (probabilities).
 *                  1: y = (x - m) - log(d), the log of the same quantity
 *                  (PyTorch's softmax forward switches between the two
 *                  with one flag: [P2] section 九, the SoftMax.cu dispatch).
 *   causal         0: every key of a row takes part.
 *                  1: row i keeps the keys j <= (i mod causal_period) +
 *                  causal_offset and masks the rest.  With rows laid out as
 *                  heads x queries and N keys, causal_period = queries and
 *                  causal_offset = N - queries is the attention causal mask
 *                  (the per-layer score softmax of [P1] section
 *                  "二、它们在 Qwen2.5-7B 里的真实位置"; offset 0 when queries
 *                  and keys coincide).  Masked keys are not read: the
 *                  kernel loads only the aligned vectors holding a row's
 *                  kept keys (16 bytes; 8 for a bf16 input written as
 *                  fp32), so only masked keys that share the vector of the
 *                  last kept key are read, and they are discarded; the
 *                  input there may hold anything.
 *   causal_period  >= 1 when causal (ignored otherwise).
 *   causal_offset  >= 0 when causal (ignored otherwise).
 * Masked keys come out as exactly 0 (probabilities) or -inf (log output).
 * Kept keys may themselves be -inf (a further mask in the data); they give 0
 * or -inf the same way ([P2] section 十, the masked entries of the online
 * softmax).  A row whose kept keys are all -inf gives NaN everywhere, as in
 * rr_softmax_rows.
 */
typedef struct rr_softmax_opts {
  int32_t log_output;
  int32_t causal;
  int64_t causal_period;
  int64_t causal_offset;
} rr_softmax_opts;

/*
 * rr_softmax_rows_ex_workspace_bytes -- workspace rr_softmax_rows_ex needs
 * with these options (0 when none: a causal call never splits a row).
 * Host-only; returns 0 for invalid arguments.
 */
size_t rr_softmax_rows_ex_workspace_bytes(int64_t M, int64_t N, rr_dtype in_dtype,
                                          rr_dtype out_dtype, const rr_softmax_opts* opts);

/*
 * rr_softmax_rows_ex -- rr_softmax_rows with options (above).  Arguments,
 * workspace rules, aliasing rules and errors as rr_softmax_rows; in
 * addition RR_ERR_INVALID_ARG for log_output or causal outside {0, 1}, or a
 * causal call with causal_period < 1 or causal_offset < 0.  With opts NULL
 * or all zero it is exactly rr_softmax_rows (same kernels, same bits).
 */
rr_status rr_softmax_rows_ex(void* y, const void* x, int64_t M, int64_t N, rr_dtype in_dtype,
                             rr_dtype out_dtype, const rr_softmax_opts* opts, void* workspace,
                             size_t workspace_bytes, void* stream);

/* ------------------------------------------------------------------------
 * Strided rows.  The same operations on matrices whose rows are not packed
 * back to back: row i of x starts at x + i * ldx elements (likewise y with
 * ldy and the residual with ldr), as when x is a column slice of a wider
 * activation (vLLM's normalisation kernels take such an input stride: [P2]
 * section 九, the fused_add_rms_norm kernel's input_stride).  Every stride is
 * in elements, at least the row width (H or N) and at most 2^40.  Vector
 * accesses need every row start aligned to the access (16 bytes: aligned
 * base pointers and strides that are multiples of 4 fp32 or 8 bf16
 * elements; 8 bytes for the bf16 input of a softmax written as fp32);
 * a call whose x and y (and residual) rows share their offset within a
 * vector is cut at aligned addresses (see above); otherwise the scalar path runs, with the
 * same results up to rounding order.  With every stride equal to the width these are exactly
 * the contiguous entry points above (same kernels, same bits).
 * Aliasing: y may be x itself (same pointer and stride, same dtype); other
 * matrices of a call must not share an element.  Two matrices with the same
 * stride whose column windows are disjoint (two slices of one wider
 * matrix) do not share one; other layouts count as overlapping when their
 * first-to-last-byte spans intersect.  Errors as the contiguous forms, plus
 * RR_ERR_INVALID_ARG for a stride out of range.
 * ------------------------------------------------------------------------ */
rr_status rr_rmsnorm_strided(void* y, int64_t ldy, const void* x, int64_t ldx, const void* gamma,
                             int64_t M, int64_t H, float eps, rr_dtype dtype, void* stream);

rr_status rr_fused_add_rmsnorm_strided(void* y, int64_t ldy, void* residual, int64_t ldr,
                                       const void* x, int64_t ldx, const void* gamma, int64_t M,
                                       int64_t H, float eps, rr_dtype dtype, void* stream);

rr_status rr_layernorm_strided(void* y, int64_t ldy, const void* x, int64_t ldx, const void* gamma,
                               const void* beta, int64_t M, int64_t H, float eps, rr_dtype dtype,
                               void* stream);

/* Workspace: rr_softmax_rows_ex_workspace_bytes(M, N, ...) with the same
 * options (it does not depend on the strides). */
rr_status rr_softmax_rows_strided(void* y, int64_t ldy, const void* x, int64_t ldx, int64_t M,
                                  int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                                  const rr_softmax_opts* opts, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * rr_softmax_rows_strided_noalloc -- rr_softmax_rows_strided for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc).  Same arguments, results
 * (same kernels, same bits), aliasing rules and errors, but no workspace
 * argument: a split row's (m, d) slots live in a static device array of
 * 4 MiB (262144 slots of 16 bytes) that the library holds on each device it
 * runs on until the process ends.  The call allocates nothing and calls no
 * hipMalloc or hipFree; on its first call on a device it looks up that
 * device's copy of the array (hipGetSymbolAddress), which must then be the
 * current device.
 *   - A shape whose split needs more than 4 MiB of slots
 *     (rr_softmax_rows_ex_workspace_bytes > 4194304) returns
 *     RR_ERR_WORKSPACE and enqueues nothing.
 *   - Every call on a device shares that device's array, which keeps the
 *     last call's contents: calls that overlap in time on one device (two
 *     streams, or two threads) race and may produce wrong results; calls on
 *     one stream are ordered and safe.  Nothing in the array needs to start
 *     at zero.
 */
rr_status rr_softmax_rows_strided_noalloc(void* y, int64_t ldy, const void* x, int64_t ldx, int64_t M,
                                          int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                                          const rr_softmax_opts* opts, void* stream);

/* Static English name of a status code ("RR_OK", ...). */
const char* rr_status_string(rr_status status);

/* Detail of the last non-OK status returned on the calling thread ("" if none). */
const char* rr_last_error_message(void);

/* ------------------------------------------------------------------------
 * Dispatch introspection and diagnostics (host-only unless stated).
 * ------------------------------------------------------------------------ */

typedef enum rr_op {
  RR_OP_RMSNORM = 0,
  RR_OP_FUSED_ADD_RMSNORM = 1,
  RR_OP_SOFTMAX = 2,
  RR_OP_LAYERNORM = 3,
  RR_OP_SOFTMAX_CAUSAL = 4 /* rr_softmax_rows_ex with causal = 1 */
} rr_op;

/* Kernel variants, chosen by row length ([P2] section 六; [P4] section
 * "按行长度选择并行方式"):
 *   WAVE  one 64-lane wavefront per row, row held in VGPRs (N <= 2048)
 *   BLOCK one workgroup of up to 16 wavefronts per row, row held in VGPRs,
 *         wavefront totals combined through LDS (N <= 32768)
 *   SPLIT several workgroups per row (softmax, long rows with few rows),
 *         each summarising its chunk as (m, d) into the workspace.  Where the
 *         rows are aligned, a row has at most 64 chunks and the device
 *         holds every workgroup of the grid at once, this is ONE kernel:
 *         each workgroup keeps its chunk in registers, publishes its pair in
 *         a tagged slot, waits (a bounded time, then summarises a missing
 *         chunk itself) for the row's other pairs, merges them and
 *         normalises, so x is read once.
 *         Otherwise two kernels: the summaries, then a second that merges a
 *         row's pairs and normalises, re-reading x (rows of more than 64
 *         chunks get a merge kernel in between that folds each row's pairs
 *         into one, so the cost stays linear in N).  Both forms give the
 *         same bits.  SPLIT_ONE_KERNEL forces the split on aligned rows;
 *         SPLIT_TWO_KERNELS forces the two-kernel form (diagnostics).
 *   LOOP  one workgroup per row streaming the row twice (any N; long rows
 *         with many rows; causal rows too long for BLOCK; rows whose input
 *         and output sit at different offsets within a vector, element by
 *         element)
 *   SUBWAVE short rows (at most 32 vectors, or 32 elements when unaligned):
 *         L lanes per row, 64/L rows per wavefront, reduced inside each
 *         L-lane group ([P4] section "按行长度选择并行方式")
 * For SUBWAVE, rr_plan.waves_per_row holds the lanes per row L. */
typedef enum rr_variant {
  RR_VARIANT_AUTO = 0,
  RR_VARIANT_WAVE = 1,
  RR_VARIANT_BLOCK = 2,
  RR_VARIANT_SPLIT = 3,
  RR_VARIANT_LOOP = 4,
  RR_VARIANT_SPLIT_ONE_KERNEL = 5, /* SPLIT on aligned rows (one kernel where it can) */
  RR_VARIANT_SUBWAVE = 6,          /* short rows, several rows per wavefront */
  RR_VARIANT_SPLIT_TWO_KERNELS = 7 /* SPLIT always as two kernels */
} rr_variant;

typedef struct rr_plan {
  int32_t variant;          /* rr_variant actually used */
  int32_t waves_per_row;    /* wavefronts cooperating on one row */
  int32_t rows_per_group;   /* rows handled by one workgroup per step */
  int32_t vecs_per_lane;    /* vector accesses per lane held in registers */
  int32_t vec_elems;        /* elements per vector access: 4 fp32, 8 bf16 (4 for a bf16
                               softmax written as fp32), 1 scalar */
  int32_t block_threads;    /* workgroup size */
  int64_t chunks_per_row;   /* SPLIT: workgroups per row; otherwise 1 */
  int64_t work_items;       /* workgroup-steps needed (rows / rows_per_group x chunks) */
  size_t workspace_bytes;   /* SPLIT: M * chunks_per_row * 16 + 4 M (to 16); otherwise 0 */
  int32_t row_shift;        /* 1: rows cut into vectors at aligned addresses (WAVE, BLOCK;
                               a softmax also SPLIT, LOOP): a row starting inside a vector, or ending inside one, is
                               accessed whole vectors at a time except its first and last
                               vector, whose elements inside the row are accessed one by one */
} rr_plan;

/*
 * The launch plan the library would use.  aligned16 describes the call's
 * row starts:
 *   1  every row start is aligned for vector access (16 bytes; 8 for the
 *      bf16 input of a softmax written as fp32);
 *   2  row starts anywhere, but each input row and its output row sit at the
 *      same element offset within a vector (contiguous rows of a width that
 *      is not a whole number of vectors, column slices with equal strides):
 *      the call then cuts rows at aligned addresses (row_shift);
 *   0  neither: element-by-element access.
 * Returns RR_ERR_INVALID_ARG / RR_ERR_UNSUPPORTED as the corresponding call
 * would.  (The diagnostics build, rowreduce_diag.h, can force a variant; its
 * plans then follow that override.)
 */
rr_status rr_query_plan(rr_op op, int64_t M, int64_t N, rr_dtype in_dtype, rr_dtype out_dtype,
                        int aligned16, rr_plan* plan);

#ifdef __cplusplus
}
#endif

#endif /* ROWREDUCE_H */
