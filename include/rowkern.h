/*
 * rowkern: fused row-wise reduce-then-normalize kernels for AMD MI355X (gfx950).
 *
 * C ABI of librowkern.so.  Every entry point works on a row-major matrix of M
 * rows and N columns with unit column stride and a row stride (in elements)
 * of ld >= N; rows are independent.  Two storage formats are supported:
 * fp32, and bf16 (storage only: all arithmetic is fp32, outputs are rounded to
 * nearest even).  Input and output have the same format.
 *
 * Pages the operations follow (titles as printed on them):
 *   [TKE] "Triton Kernel 实现练习" (Triton kernel exercises)
 *   [L6]  "第 6 讲：GPU Kernels 与 Triton" (CS336 lecture 6 notes)
 *   [KTN] CS336 Lecture 6 "Kernels, Triton" notes
 *   [FLG] "PyTorch 自定义 CUDA 算子与 Triton 编程从 Python 原型到 GPU 极致性能"
 *
 * Conventions common to all entry points
 *   Ownership   All pointers are device memory owned by the caller.  The
 *               library allocates and frees nothing and is safe to call from
 *               several host threads.  Its only global state is a per-device
 *               count of how many workgroups of each persistent LayerNorm
 *               kernel fit on the chip at once (asked of the occupancy
 *               calculator on first use, kept in atomics) and the fixed
 *               scratch array of rk_online_softmax_noalloc.
 *   Streams     Work is enqueued on `stream` (0 = the null stream) of the
 *               current device and the call returns without synchronizing.
 *               Multi-kernel operations are ordered by the stream alone.
 *   Alignment   Any element-aligned pointer and any ld >= N are accepted.
 *               Rows are read and written with 16-byte vector accesses when
 *               every row of every row operand starts on a 16-byte boundary
 *               (base pointers and row pitches 16-byte aligned), and also
 *               when rows start at other offsets that the input and output
 *               (and residual operands) share row for row: the row is then
 *               covered by aligned vectors whose first and last are masked
 *               (such a load stays inside a 16-byte block that holds an
 *               element of the row).  Weight and bias must be 16-byte
 *               aligned for this.  Other layouts take a slower element-wise
 *               path with the same results.
 *   Aliasing    y may be x exactly (same pointer and same ld: in place);
 *               any other overlap of an output with an input is rejected.
 *   Errors      Arguments are validated before any HIP call; a rejected call
 *               enqueues nothing.  M == 0 is a valid no-op.  A failed kernel
 *               launch returns RK_ERR_HIP.  Nothing is printed and no C++
 *               exception crosses the ABI.
 *   Determinism For fixed arguments the results are bitwise reproducible.
 */
#ifndef ROWKERN_H
#define ROWKERN_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define RK_VERSION 100 /* major * 10000 + minor * 100 + patch */

typedef enum rk_dtype {
    RK_F32 = 0,  /* IEEE binary32 */
    RK_BF16 = 1, /* bfloat16 storage, fp32 arithmetic */
    RK_F16 = 2,  /* IEEE binary16 storage (rk_flash_attention only) */
} rk_dtype;

/* GeLU form ([TKE] §3.4 gives both): the LayerNorm epilogue and rk_gelu. */
typedef enum rk_gelu_kind {
    RK_GELU_TANH = 0, /* 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))) */
    RK_GELU_ERF = 1,  /* 0.5 z (1 + erf(z / sqrt(2))), the exact form */
    RK_GELU_NONE = 2, /* no activation, y = z: the LayerNorm of [TKE] §4.1
                         alone (rk_layernorm_gelu_ex only; rk_gelu rejects it) */
} rk_gelu_kind;

typedef enum rk_status {
    RK_OK = 0,
    RK_ERR_INVALID_ARG = 1, /* a size, stride, pointer, dtype or eps is invalid */
    RK_ERR_UNSUPPORTED = 2, /* valid but beyond what the library handles */
    RK_ERR_WORKSPACE = 3,   /* workspace missing or too small */
    RK_ERR_HIP = 4,         /* the HIP runtime rejected a launch */
    RK_ERR_SCRATCH = 5,     /* more than rk_online_softmax_noalloc's scratch */
} rk_status;

/*
 * Numerically stable row softmax ([TKE] §2.4 "Softmax", stable version;
 * [KTN] "Triton Softmax"):
 *     m_i = max_j x_ij,   y_ij = exp(x_ij - m_i) / sum_k exp(x_ik - m_i).
 *
 * x  [M][ldx] input, y [M][ldy] output, both of `dtype`.
 * Rows that fit on chip (N <= 16384 for fp32, N <= 32768 for bf16; for rows
 * at a shared offset, N + 3 / N + 7 up to those) are held in registers: one
 * HBM read and one HBM write per element.  Longer rows, and rows whose
 * input and output offsets differ, are computed by the online kernels of
 * rk_online_softmax (two reads, one write), with the same result: one
 * workgroup per row, or, for long rows in few rows (the rule of
 * num_splits == 0 there, tightened for the extra launch) when y does not
 * alias x, the split-row form with no workspace: each row's chunk partials
 * are kept in that row's own first output chunk (from its first 8-byte
 * boundary), a second kernel writes every output element but the first
 * vectors of each row, which hold them, and a third, one workgroup per row,
 * reads the partials and then writes those vectors.  The split count is
 * lowered where needed until the first chunk holds them.
 * A row that is all -inf, or holds +inf or NaN, yields NaN (the IEEE value
 * of the definition).
 *
 * Returns RK_ERR_INVALID_ARG if M < 0, N < 1, N > INT32_MAX, ldx < N,
 * ldy < N, x or y is NULL with M > 0, a pointer is not aligned to its
 * element size, dtype is unknown, or x and y overlap other than exactly;
 * RK_ERR_UNSUPPORTED if N > 2^30 or the grid would exceed 2^32 work-items.
 */
rk_status rk_softmax(const void *x, void *y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                     rk_dtype dtype, hipStream_t stream);

/*
 * Online softmax for long rows ([TKE] §2.5 "Online Softmax"; [L6] §7.2
 * "Online Softmax").  Same result as rk_softmax, computed from a running
 * state (m, d) = (max so far, sum of exp(x - m) so far) that is rescaled by
 * exp(m_old - m_new) as each block of the row arrives.
 *
 * num_splits == 1  one kernel; one workgroup streams its row twice: the
 *                  first pass builds (m, d), the second writes
 *                  exp(x - m) / d.  No workspace is used.
 * num_splits >= 2  split-row variant, two kernels on `stream`: the row is
 *                  cut into S = num_splits chunks of whole 16-byte vectors
 *                  (C = ceil(N / S) rounded up to the vector width; trailing
 *                  chunks may be empty), the first kernel writes each chunk's
 *                  partial (m_s, d_s) to `workspace`, the second merges the
 *                  row's S partials with
 *                      (m1,d1)+(m2,d2) = (M, d1 e^(m1-M) + d2 e^(m2-M)),
 *                  M = max(m1, m2), (-inf, 0) the identity,
 *                  and writes its chunk.
 * num_splits == 0  the library picks S from M, N and dtype
 *                  (rk_online_softmax_auto_splits): S = 1 for 256 rows or
 *                  more, or where one workgroup per row streams a row in
 *                  about the time the split kernels take for all rows;
 *                  otherwise chunks of about 16 KiB, at most 2048
 *                  workgroups.
 *
 * workspace  device memory of at least
 *            rk_online_softmax_workspace_bytes(M, N, num_splits, dtype) bytes,
 *            8-byte aligned, owned by the caller; may be NULL when that size
 *            is 0.  Its contents on entry do not matter; on return (stream
 *            order) it holds the partials as float pairs [M][S][2].
 *
 * Returns RK_ERR_INVALID_ARG as rk_softmax, and for num_splits < 0 or
 * num_splits > 65536 or a misaligned workspace; RK_ERR_WORKSPACE if the
 * workspace is NULL or smaller than required.
 */
rk_status rk_online_softmax(const void *x, void *y, int64_t M, int64_t N, int64_t ldx,
                            int64_t ldy, rk_dtype dtype, int32_t num_splits, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes rk_online_softmax needs for these arguments (0 when the
 * streaming kernel is used or the arguments are invalid). */
size_t rk_online_softmax_workspace_bytes(int64_t M, int64_t N, int32_t num_splits,
                                         rk_dtype dtype);

/*
 * rk_online_softmax for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, bit for bit, as
 * rk_online_softmax with the same num_splits, but the split form keeps its
 * partials in a fixed 1 MiB device array inside the library (one per GPU,
 * held until the process ends) instead of a caller's workspace.  The call
 * allocates and frees nothing; the first call on a device looks the array's
 * address up once.
 *
 * Limits and contract
 *   M * S * 8 bytes of partials (S the resolved split count) must fit the
 *   1 MiB scratch (M * S <= 131072), else RK_ERR_SCRATCH and nothing is
 *   enqueued.  S = 1 uses no scratch.  `stream` must belong to the current
 *   device (else RK_ERR_INVALID_ARG).  Every call on a GPU shares that
 *   GPU's scratch: calls on one stream are ordered, but split calls that
 *   overlap in time on one GPU (other streams, other host threads) race on
 *   it and may return wrong results.  Nothing in the scratch needs clearing:
 *   the first kernel writes every partial the second reads.
 * Returns as rk_online_softmax (without the workspace cases), plus
 * RK_ERR_SCRATCH; RK_ERR_HIP if the scratch address cannot be obtained.
 */
rk_status rk_online_softmax_noalloc(const void *x, void *y, int64_t M, int64_t N, int64_t ldx,
                                    int64_t ldy, rk_dtype dtype, int32_t num_splits,
                                    hipStream_t stream);

/* The split count rk_online_softmax uses for num_splits == 0 (1 for invalid
 * arguments). */
int32_t rk_online_softmax_auto_splits(int64_t M, int64_t N, rk_dtype dtype);

/*
 * Fused LayerNorm + affine + tanh-approximation GeLU, one pass over each row
 * ([TKE] §4.1 "LayerNorm" and §3.4 "Approx Activation"; [FLG] section 三
 * "Fused LayerNorm GELU Kernel"):
 *     mu = sum_j x_j / N,  var = sum_j (x_j - mu)^2 / N  (over the N true
 *     columns only), rstd = 1 / sqrt(var + eps),
 *     z_j = (x_j - mu) * rstd * weight_j + bias_j,
 *     y_j = 0.5 z_j (1 + tanh(sqrt(2/pi) (z_j + 0.044715 z_j^3))).
 *
 * x [M][ldx], y [M][ldy], weight [N], bias [N] (contiguous), all of `dtype`.
 * 16-byte aligned rows of up to 14336 (fp32) / 20480 (bf16) columns, and of
 * exactly 16384 (fp32) / 32768 (bf16), stay in registers (one HBM read and
 * write per element), as do rows at a shared offset (see Alignment) with
 * N + 3 (fp32) / N + 7 (bf16) up to the first two limits; other rows take
 * one workgroup per row that reads the row twice (statistics by parts merged
 * as in rk_layernorm_gelu_ex, then the output), which measured faster than a
 * register tile filled well below its capacity.  Long rows in few rows, when
 * y does not alias x, take the split-row form of rk_layernorm_gelu_ex with
 * no workspace, the chunk summaries kept in each row's first output chunk
 * and the vectors holding them written last by a third kernel, as
 * rk_softmax does.
 * Otherwise the same as rk_layernorm_gelu_ex with RK_GELU_TANH and
 * num_splits = 1.
 *
 * Returns RK_ERR_INVALID_ARG as rk_softmax, and when weight or bias is NULL
 * with M > 0, eps is not finite and > 0, or y overlaps weight or bias.
 */
rk_status rk_layernorm_gelu(const void *x, const void *weight, const void *bias, void *y,
                            int64_t M, int64_t N, int64_t ldx, int64_t ldy, float eps,
                            rk_dtype dtype, hipStream_t stream);

/*
 * rk_layernorm_gelu with a choice of activation and of how long rows are
 * split ([TKE] §4.1 "LayerNorm", §3.4 "Approx Activation", and §6.3 on
 * reducing a long dimension in pieces).
 *
 * gelu        RK_GELU_TANH, RK_GELU_ERF, or RK_GELU_NONE for the LayerNorm
 *             alone (y = z, same kernels and statistics).
 * num_splits  1: one workgroup (or register tile) per row, as
 *             rk_layernorm_gelu.  S > 1: each row is cut into S chunks of
 *             C = ceil(N / S) elements (rounded up to whole 16-byte vectors
 *             on the vector path); a first kernel writes a summary of each
 *             chunk to the workspace (its mean, taken relative to the row's
 *             first element K, and M2, the sum of squared deviations from
 *             it) and K itself, a second merges the row's S summaries by
 *             the Chan-Golub-LeVeque pairwise update and writes the chunk,
 *             taking K from the workspace (so y may be x):
 *             2 reads + 1 write per element, all CUs busy even for a few
 *             long rows.  0: rk_layernorm_gelu_auto_splits (S = 1 for rows
 *             a register tile holds, else the rule of
 *             rk_online_softmax_auto_splits with LayerNorm's own rates).
 * workspace   for S > 1: caller-owned device memory of at least
 *             rk_layernorm_gelu_workspace_bytes(M, N, num_splits, dtype)
 *             bytes, 8-byte aligned, not overlapping x, y, weight or bias;
 *             ignored (may be NULL) for S = 1.
 *
 * Returns as rk_layernorm_gelu, plus RK_ERR_INVALID_ARG for an unknown gelu,
 * num_splits outside [0, 65536], a misaligned or overlapping workspace;
 * RK_ERR_WORKSPACE when it is NULL or too small; RK_ERR_UNSUPPORTED when
 * M * S workgroups exceed the launch limits.
 */
rk_status rk_layernorm_gelu_ex(const void *x, const void *weight, const void *bias, void *y,
                               int64_t M, int64_t N, int64_t ldx, int64_t ldy, float eps,
                               rk_dtype dtype, rk_gelu_kind gelu, int32_t num_splits,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes rk_layernorm_gelu_ex needs: M * (S + 1) * 8 for S > 1 (S
 * the resolved split count; per row, S chunk summaries and the shift K as
 * two floats each), 0 for S = 1 or invalid arguments. */
size_t rk_layernorm_gelu_workspace_bytes(int64_t M, int64_t N, int32_t num_splits,
                                         rk_dtype dtype);

/* The split count rk_layernorm_gelu_ex uses for num_splits == 0: 1 when a
 * register tile takes the row (as listed under rk_layernorm_gelu), for 256
 * rows or more, or where one workgroup per row is expected to be as fast;
 * else chunks of about 16 KiB, at most 2048 workgroups (1 for invalid
 * arguments). */
int32_t rk_layernorm_gelu_auto_splits(int64_t M, int64_t N, rk_dtype dtype);

/*
 * RMSNorm ([TKE] §4.2 "RMSNorm"):
 *     inv_rms = 1 / sqrt(sum_j x_j^2 / N + eps),  y_j = x_j * inv_rms * weight_j,
 * with no centring; fp32 accumulation, output in `dtype`.
 *
 * x [M][ldx], y [M][ldy], weight [N] (contiguous), all of `dtype`.  Register
 * resident up to N = 16384 (fp32) / 32768 (bf16), 16-byte aligned or at a
 * shared offset (see Alignment; N + 3 / N + 7 up to those), with one read
 * and one write per element; other rows are read twice by a looping kernel,
 * one workgroup per row, or, for long rows in few rows when y aliases no
 * input, split across workgroups with each chunk's sum of squares kept in
 * the row's first output chunk, the vectors holding them written last by a
 * third kernel (as rk_softmax does).
 *
 * Returns RK_ERR_INVALID_ARG as rk_softmax, and when weight is NULL with
 * M > 0, eps is not finite and > 0, or y overlaps weight.
 */
rk_status rk_rmsnorm(const void *x, const void *weight, void *y, int64_t M, int64_t N,
                     int64_t ldx, int64_t ldy, float eps, rk_dtype dtype, hipStream_t stream);

/*
 * Fused residual add + RMSNorm ([TKE] §4.3 "Fused Residual RMSNorm"), two
 * outputs from one pass:
 *     residual_out = x + residual,
 *     y = residual_out * rsqrt(mean(residual_out^2) + eps) * weight.
 * The sum is formed in fp32 and rounded to `dtype`; the norm is taken of
 * that stored value, so y equals rk_rmsnorm(residual_out) as with an unfused
 * add followed by a norm (identical for fp32).
 *
 * x [M][ldx], residual [M][ldr], y [M][ldy], residual_out [M][ldo],
 * weight [N] (contiguous), all of `dtype`.  Each output may be one of the
 * inputs exactly (same pointer and pitch: e.g. residual_out = residual to
 * update the residual stream in place); y and residual_out must not overlap
 * each other, the weight, or an input other than exactly.
 *
 * Returns RK_ERR_INVALID_ARG for M < 0, N < 1, any pitch < N, a NULL or
 * misaligned pointer with M > 0, an unknown dtype, eps not finite and > 0,
 * or a forbidden overlap; RK_ERR_UNSUPPORTED if N > 2^30.
 */
rk_status rk_residual_rmsnorm(const void *x, const void *residual, const void *weight, void *y,
                              void *residual_out, int64_t M, int64_t N, int64_t ldx,
                              int64_t ldr, int64_t ldy, int64_t ldo, float eps, rk_dtype dtype,
                              hipStream_t stream);

/*
 * Row-wise sum and max ([TKE] §2.2 "Row-wise Sum", §2.3 "Row-wise Max"):
 *     out[i] = sum_j x[i, j]   (fp32 accumulation, rounded to `dtype`),
 *     out[i] = max_j x[i, j]   (exact; NaN if the row holds a NaN).
 *
 * x [M][ldx] and out [M] (contiguous), both of `dtype`.  One HBM read per
 * element.  A row goes to one wave (up to 1024 16-byte vectors), four waves
 * (up to 8192) or sixteen.  The sum's order of addition is fixed: results
 * are reproducible bit for bit.
 *
 * Returns RK_ERR_INVALID_ARG for an unknown dtype, M < 0, N < 1, ldx < N, a
 * NULL or misaligned pointer with M > 0, or out overlapping x;
 * RK_ERR_UNSUPPORTED if N > 2^30.
 */
rk_status rk_row_sum(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                     rk_dtype dtype, hipStream_t stream);
rk_status rk_row_max(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                     rk_dtype dtype, hipStream_t stream);

/*
 * rk_row_sum / rk_row_max with long rows cut into pieces ([TKE] §2.2, §2.3,
 * and §6.3 on reducing a long dimension in pieces).  One workgroup per row
 * leaves most of the chip idle when there are few long rows; the split form
 * spreads every row over many workgroups.
 *
 * num_splits  1: as rk_row_sum / rk_row_max.  S > 1: each row is cut into S
 *             chunks of C = ceil(N / S) elements rounded up to whole 16-byte
 *             vectors (trailing chunks may be empty); a first kernel writes
 *             each chunk's fp32 sum (max) to the workspace as
 *             float [M][S], a second reduces each row's S partials and
 *             writes out[i].  Both add in an order fixed by N and S, so the
 *             results are reproducible bit for bit for a given S (a sum may
 *             differ from S = 1 by rounding; the max is the same).  0:
 *             rk_row_reduce_auto_splits.
 * workspace   for S > 1: caller-owned device memory of at least
 *             rk_row_reduce_workspace_bytes(M, N, num_splits, dtype) bytes,
 *             8-byte aligned, not overlapping x or out; its contents on
 *             entry do not matter.  Ignored (may be NULL) for S = 1.
 *
 * Returns as rk_row_sum, plus RK_ERR_INVALID_ARG for num_splits outside
 * [0, 65536] or a misaligned or overlapping workspace; RK_ERR_WORKSPACE when
 * it is NULL or too small; RK_ERR_UNSUPPORTED when M * S workgroups exceed
 * the launch limits.
 */
rk_status rk_row_sum_ex(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                        rk_dtype dtype, int32_t num_splits, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);
rk_status rk_row_max_ex(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                        rk_dtype dtype, int32_t num_splits, void *workspace,
                        size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes rk_row_sum_ex / rk_row_max_ex need: M * S * 4 for S > 1
 * (S the resolved split count), 0 for S = 1 or invalid arguments. */
size_t rk_row_reduce_workspace_bytes(int64_t M, int64_t N, int32_t num_splits, rk_dtype dtype);

/* The split count of num_splits == 0: 1 for 256 rows or more, or where one
 * workgroup per row is expected to be as fast (by the reductions' own
 * measured rates); else chunks of about 16 KiB, at most 2048 workgroups (1
 * for invalid arguments). */
int32_t rk_row_reduce_auto_splits(int64_t M, int64_t N, rk_dtype dtype);

/*
 * Elementwise GeLU ([TKE] §3.4; [KTN] "Triton GeLU"): y = GeLU(x), the tanh
 * approximation or the exact erf form, fp32 arithmetic.
 *
 * x [M][ldx], y [M][ldy] of `dtype`; a contiguous buffer whose output sits at
 * the same offset past a 16-byte boundary is processed as one flat array.
 * Arguments, aliasing and errors as in rk_softmax, plus RK_ERR_INVALID_ARG
 * for a gelu other than RK_GELU_TANH and RK_GELU_ERF.
 */
rk_status rk_gelu(const void *x, void *y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                  rk_dtype dtype, rk_gelu_kind gelu, hipStream_t stream);

/*
 * Attention forward with the online softmax fused into the value product
 * ([TKE] §5.2 "FlashAttention-style Forward"; [L6] §7.2-7.3 and §8):
 *     o[b,h,i,:] = sum_j softmax_j(scale * q[b,h,i,:] . k[b,h,j,:]) v[b,h,j,:]
 * over keys j < T, or j <= i when `causal` is nonzero.  Neither the T x T
 * scores nor the probabilities are written anywhere: keys and values are
 * scanned in blocks with a running max, sum and output per query row.
 *
 * q, k, v, o  [B][H][T][d] of `dtype` (RK_BF16 or RK_F16), unit stride along
 *             d; `*_strides` = {batch, head, seq} element strides of each, or
 *             NULL for the contiguous layout {H*T*d, T*d, d}.  Base pointers
 *             16-byte aligned and every stride a multiple of 8 elements.
 * d           head dimension, 64 or 128.
 * scale       multiplies the scores (finite and > 0; usually 1 / sqrt(d)).
 * Arithmetic  products on the matrix cores with fp32 accumulation; the
 *             probabilities are rounded to `dtype` for the value product (as
 *             the pages' kernel casts them to the value type); softmax state
 *             and accumulators in fp32; o rounded to nearest even.
 *
 * Returns RK_ERR_INVALID_ARG for negative sizes, d < 1, a NULL pointer with
 * B*H*T > 0, a scale that is not finite and > 0, causal outside {0, 1}, an
 * unknown dtype, a
 * seq stride below d, o overlapping q, k or v, or o's rows overlapping one
 * another; RK_ERR_UNSUPPORTED for RK_F32, d other than 64 or 128,
 * misaligned pointers or strides, or sizes beyond the launch limits.
 * B*H*T == 0 is a no-op.
 */
rk_status rk_flash_attention(const void *q, const void *k, const void *v, void *o, int64_t B,
                             int64_t H, int64_t T, int64_t d, const int64_t *q_strides,
                             const int64_t *k_strides, const int64_t *v_strides,
                             const int64_t *o_strides, float scale, int32_t causal,
                             rk_dtype dtype, hipStream_t stream);

/* Static, NUL-terminated description of a status ("unknown status" for an
 * unknown value). */
const char *rk_status_string(rk_status status);

/* RK_VERSION of the built library. */
int rk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* ROWKERN_H */
