/*
 * rowkern tuning and measurement entry points (librowkern.so).
 *
 * Not needed to use the library.  They expose (a) a plain 16-byte copy
 * kernel, the bandwidth ceiling and counter calibration the kernels are
 * measured against, and (b) each compiled variant of the register-resident
 * ("tile") kernels by index, so that every variant can be tested for parity
 * and timed, and the generic paths can be forced on any input.
 *
 * Ownership, streams, validation and error reporting follow rowkern.h.
 */
#ifndef ROWKERN_TUNE_H
#define ROWKERN_TUNE_H

#include "rowkern.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Copy `bytes` bytes from src to dst with 16-byte non-temporal vector loads
 * and stores (four per thread per step), one HBM read and one write per byte,
 * at most `max_workgroups` workgroups of 256 threads (<= 0: enough to cover
 * the copy once, capped at 65536) striding over the buffer.  src and dst must
 * be 16-byte aligned, bytes a multiple of 16, and the ranges disjoint;
 * otherwise RK_ERR_INVALID_ARG.
 */
rk_status rk_probe_copy(const void *src, void *dst, size_t bytes, int32_t max_workgroups,
                        hipStream_t stream);

/* Operations with tile variants. */
typedef enum rk_op {
    RK_OP_SOFTMAX = 0,
    RK_OP_LAYERNORM_GELU = 1,
    RK_OP_RMSNORM = 2,
    RK_OP_RESIDUAL_RMSNORM = 3,
} rk_op;

/* Number of compiled tile variants of `op` for `dtype` (0 if invalid). */
int32_t rk__variant_count(rk_op op, rk_dtype dtype);

/*
 * Geometry of tile variant `index`: waves cooperating on one row, 16-byte
 * vectors held per lane, waves per workgroup, rows each row-group handles in
 * sequence, the largest N it accepts, whether it is compiled for N == max_n
 * only (every register slot a column: no masks, no padding), and whether it
 * is an alternative (run by index only, never picked).  Any output pointer
 * may be NULL.
 */
rk_status rk__variant_info(rk_op op, rk_dtype dtype, int32_t index, int32_t *waves_per_row,
                           int32_t *vecs_per_lane, int32_t *waves_per_block,
                           int32_t *rows_per_group, int64_t *max_n, int32_t *exact,
                           int32_t *alternative);

/* Index of the variant the entry points pick for N: the first exact variant
 * with max_n == N, else the first general one that holds N, alternatives
 * skipped (-1 when none does and the rows-in-memory path runs). */
int32_t rk__variant_pick(rk_op op, rk_dtype dtype, int64_t N);

/*
 * rk_softmax / rk_layernorm_gelu_ex (one workgroup per row) forced onto one
 * path: variant `index` (RK_ERR_UNSUPPORTED if the data is not 16-byte
 * aligned or the variant does not accept N), or index -1 for the generic path
 * (the streaming kernels: online softmax, LayerNorm statistics by parts),
 * which takes any input.  Arguments otherwise as in rowkern.h.
 */
rk_status rk__softmax_variant(int32_t index, const void *x, void *y, int64_t M, int64_t N,
                              int64_t ldx, int64_t ldy, rk_dtype dtype, hipStream_t stream);
rk_status rk__layernorm_gelu_variant(int32_t index, const void *x, const void *weight,
                                     const void *bias, void *y, int64_t M, int64_t N,
                                     int64_t ldx, int64_t ldy, float eps, rk_dtype dtype,
                                     rk_gelu_kind gelu, hipStream_t stream);

/* rk_rmsnorm / rk_residual_rmsnorm forced onto one path, as above (index -1:
 * the two-pass looping kernel). */
rk_status rk__rmsnorm_variant(int32_t index, const void *x, const void *weight, void *y,
                              int64_t M, int64_t N, int64_t ldx, int64_t ldy, float eps,
                              rk_dtype dtype, hipStream_t stream);
rk_status rk__residual_rmsnorm_variant(int32_t index, const void *x, const void *residual,
                                       const void *weight, void *y, void *residual_out,
                                       int64_t M, int64_t N, int64_t ldx, int64_t ldr,
                                       int64_t ldy, int64_t ldo, float eps, rk_dtype dtype,
                                       hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWKERN_TUNE_H */
