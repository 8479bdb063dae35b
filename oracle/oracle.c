/*
 * CPU oracle for the row-wise kernels -- TEST INFRASTRUCTURE ONLY.
 *
 * Plain, slow, obviously correct reference implementations in IEEE double,
 * one row at a time, single-threaded, no blocking, fusion or reordering
 * beyond what each definition states.  Only the test suite, the smoke check
 * and the benchmark's CPU-baseline leg may load this code; the product path
 * (the HIP library) never does, and this file shares no code with it.
 *
 * Inputs are the exact fp32 / bf16 values the GPU reads, widened to double by
 * the caller; outputs are unrounded doubles.  Every array is row-major and
 * contiguous ([M][N]).
 *
 * Pages cited (titles as printed on them):
 *   [TKE]  "Triton Kernel 实现练习" (Triton kernel exercises)
 *   [L6]   "第 6 讲：GPU Kernels 与 Triton" (CS336 lecture 6 notes)
 *   [KTN]  CS336 Lecture 6 "Kernels, Triton" notes, section "Triton Softmax"
 *   [FLG]  "PyTorch 自定义 CUDA 算子与 Triton 编程从 Python 原型到 GPU 极致性能",
 *          section 三 "Fused LayerNorm GELU Kernel"
 *
 * Parity pins: every function here is pinned by tests under tests/ against
 * closed forms, invariants, library routines (torch float64) and
 * high-precision brute force; none is "parity unpinned".
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

/* ---------------------------------------------------------------------- */
/* Stable softmax: [TKE] §2.4 "Softmax" (stable version m = max(x),        */
/* numerator = exp(x - m), denominator = sum(numerator), out = num / den); */
/* [KTN] "Triton Softmax" (x - max -> exp -> sum -> normalize).            */
/* ---------------------------------------------------------------------- */

/* Maximum of a row; NaN propagates (any NaN makes the row NaN). */
static double row_max(const double *x, int64_t n)
{
    double m = -INFINITY;
    for (int64_t j = 0; j < n; ++j) {
        if (isnan(x[j]))
            return NAN;
        if (x[j] > m)
            m = x[j];
    }
    return m;
}

void oracle_softmax(const double *x, double *y, int64_t M, int64_t N)
{
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double *yr = y + i * N;
        double m = row_max(xr, N);
        double den = 0.0;
        for (int64_t j = 0; j < N; ++j)
            den += exp(xr[j] - m);
        for (int64_t j = 0; j < N; ++j)
            yr[j] = exp(xr[j] - m) / den;
    }
}

/* Row statistics of the stable softmax: m = max(x), d = sum exp(x - m).
 * A part whose every value is -inf has max -inf and contributes nothing to
 * any sum of exp(x - M) with M finite: its state is the empty part's
 * (-inf, 0), the start state of the online recurrence below, and the
 * undefined terms exp(-inf - (-inf)) are never formed. */
void oracle_softmax_stats(const double *x, int64_t N, double *m_out, double *d_out)
{
    double m = row_max(x, N);
    double d = 0.0;
    if (m != -INFINITY)
        for (int64_t j = 0; j < N; ++j)
            d += exp(x[j] - m);
    *m_out = m;
    *d_out = d;
}

/* ---------------------------------------------------------------------- */
/* Online softmax: [TKE] §2.5 "Online Softmax" -- state m (max of the part */
/* scanned so far) and d (sum of exp(x - m) over that part); for each new  */
/* block: m_new = max(m_old, block_max),                                   */
/*        d_new = d_old * exp(m_old - m_new) + sum(exp(block - m_new)).     */
/* [L6] §7.2 "Online Softmax": start from m = -inf, l = 0; the rescale     */
/* factor is exp(m_prev - m_curr).                                         */
/* ---------------------------------------------------------------------- */

/* The rescale factor exp(m_old - m_new).  With m_old = -inf the old sum is
 * empty (d_old = 0), and the factor is taken as 0 so that -inf - (-inf) is
 * never formed. */
static double rescale(double m_old, double m_new)
{
    if (m_old == -INFINITY)
        return 0.0;
    return exp(m_old - m_new);
}

/* Streaming recurrence over blocks of B elements (B >= 1). */
void oracle_online_stats(const double *x, int64_t N, int64_t B, double *m_out, double *d_out)
{
    double m = -INFINITY, d = 0.0;
    for (int64_t s = 0; s < N; s += B) {
        int64_t e = s + B < N ? s + B : N;
        double block_max = row_max(x + s, e - s);
        double m_new = block_max > m ? block_max : m;
        if (isnan(block_max) || isnan(m))
            m_new = NAN;
        /* While every value scanned so far is -inf (m_new = -inf) the
         * state stays the start state (-inf, 0). */
        double block_sum = 0.0;
        if (m_new != -INFINITY)
            for (int64_t j = s; j < e; ++j)
                block_sum += exp(x[j] - m_new);
        d = d * rescale(m, m_new) + block_sum;
        m = m_new;
    }
    *m_out = m;
    *d_out = d;
}

/* Merge of two partial states (m1,d1) and (m2,d2) of disjoint parts of a
 * row: the combined max M and the two sums rescaled to it.  (-inf, 0) is the
 * state of an empty part and is the identity. */
void oracle_merge(double m1, double d1, double m2, double d2, double *m_out, double *d_out)
{
    double M = m1 > m2 ? m1 : m2;
    if (isnan(m1) || isnan(m2))
        M = NAN;
    *m_out = M;
    *d_out = d1 * rescale(m1, M) + d2 * rescale(m2, M);
}

/* Split-row online softmax, [TKE] §2.5 second version: per-chunk partial
 * (m, d), then a reduce of the partials.  The row is cut into S chunks of
 * C = ceil(N / S) elements, chunk s = [s*C, min(N, (s+1)*C)); an empty chunk
 * has the state (-inf, 0).  Partials are written to m_parts/d_parts (length
 * S, may be NULL) and merged left to right. */
void oracle_split_stats(const double *x, int64_t N, int64_t S, double *m_parts, double *d_parts,
                        double *m_out, double *d_out)
{
    int64_t C = (N + S - 1) / S;
    double m = -INFINITY, d = 0.0;
    for (int64_t s = 0; s < S; ++s) {
        int64_t b = s * C, e = (s + 1) * C;
        if (b > N)
            b = N;
        if (e > N)
            e = N;
        double ms = -INFINITY, ds = 0.0;
        if (e > b)
            oracle_softmax_stats(x + b, e - b, &ms, &ds);
        if (m_parts)
            m_parts[s] = ms;
        if (d_parts)
            d_parts[s] = ds;
        oracle_merge(m, d, ms, ds, &m, &d);
    }
    *m_out = m;
    *d_out = d;
}

/* Normalize a row with given statistics: y = exp(x - m) / d. */
void oracle_softmax_apply(const double *x, double *y, int64_t N, double m, double d)
{
    for (int64_t j = 0; j < N; ++j)
        y[j] = exp(x[j] - m) / d;
}

/* Online softmax of M rows: streaming statistics (block B), then the write. */
void oracle_online_softmax(const double *x, double *y, int64_t M, int64_t N, int64_t B)
{
    for (int64_t i = 0; i < M; ++i) {
        double m, d;
        oracle_online_stats(x + i * N, N, B, &m, &d);
        oracle_softmax_apply(x + i * N, y + i * N, N, m, d);
    }
}

/* Split-row online softmax of M rows with S chunks per row. */
void oracle_split_softmax(const double *x, double *y, int64_t M, int64_t N, int64_t S)
{
    for (int64_t i = 0; i < M; ++i) {
        double m, d;
        oracle_split_stats(x + i * N, N, S, 0, 0, &m, &d);
        oracle_softmax_apply(x + i * N, y + i * N, N, m, d);
    }
}

/* ---------------------------------------------------------------------- */
/* GeLU, tanh approximation: [TKE] §3.4 "Approx Activation"               */
/*   gelu_approx(z) = 0.5 z (1 + tanh(sqrt(2/pi) (z + 0.044715 z^3))).     */
/* ---------------------------------------------------------------------- */
double oracle_gelu_tanh(double z)
{
    const double k = sqrt(2.0 / M_PI);
    return 0.5 * z * (1.0 + tanh(k * (z + 0.044715 * z * z * z)));
}

void oracle_gelu_tanh_array(const double *z, double *y, int64_t n)
{
    for (int64_t j = 0; j < n; ++j)
        y[j] = oracle_gelu_tanh(z[j]);
}

/* ---------------------------------------------------------------------- */
/* LayerNorm: [TKE] §4.1 "LayerNorm"                                       */
/*   mean = mean(x); var = mean((x - mean)^2);                             */
/*   out = (x - mean) * rsqrt(var + eps) * weight + bias,                  */
/* statistics over the N true columns only.  [FLG] fuses the affine       */
/* output with the tanh GeLU above in one pass over the row.               */
/* ---------------------------------------------------------------------- */

/* Row statistics: mean, biased variance (divide by N), rstd = 1/sqrt(var+eps). */
void oracle_layernorm_stats(const double *x, int64_t N, double eps, double *mean_out,
                            double *var_out, double *rstd_out)
{
    double s = 0.0;
    for (int64_t j = 0; j < N; ++j)
        s += x[j];
    double mean = s / (double)N;
    double q = 0.0;
    for (int64_t j = 0; j < N; ++j)
        q += (x[j] - mean) * (x[j] - mean);
    double var = q / (double)N;
    *mean_out = mean;
    *var_out = var;
    *rstd_out = 1.0 / sqrt(var + eps);
}

/* Normalized row x_hat = (x - mean) * rstd (before the affine step). */
void oracle_layernorm_normalize(const double *x, double *xhat, int64_t M, int64_t N, double eps)
{
    for (int64_t i = 0; i < M; ++i) {
        double mean, var, rstd;
        oracle_layernorm_stats(x + i * N, N, eps, &mean, &var, &rstd);
        for (int64_t j = 0; j < N; ++j)
            xhat[i * N + j] = (x[i * N + j] - mean) * rstd;
    }
}

/* Fused LayerNorm + affine + tanh GeLU of M rows. */
void oracle_layernorm_gelu(const double *x, const double *w, const double *b, double *y, int64_t M,
                           int64_t N, double eps)
{
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double *yr = y + i * N;
        double mean, var, rstd;
        oracle_layernorm_stats(xr, N, eps, &mean, &var, &rstd);
        for (int64_t j = 0; j < N; ++j) {
            double z = (xr[j] - mean) * rstd * w[j] + b[j];
            yr[j] = oracle_gelu_tanh(z);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* RMSNorm: [TKE] §4.2 "RMSNorm"                                           */
/*   inv_rms = rsqrt(mean(x^2) + eps); out = x * inv_rms * weight,         */
/* no centring (the difference from LayerNorm the page points out).       */
/* ---------------------------------------------------------------------- */

/* Mean square of a row and inv_rms = 1 / sqrt(mean square + eps). */
void oracle_rms_stats(const double *x, int64_t N, double eps, double *ms_out, double *inv_out)
{
    double q = 0.0;
    for (int64_t j = 0; j < N; ++j)
        q += x[j] * x[j];
    double ms = q / (double)N;
    *ms_out = ms;
    *inv_out = 1.0 / sqrt(ms + eps);
}

void oracle_rmsnorm(const double *x, const double *w, double *y, int64_t M, int64_t N, double eps)
{
    for (int64_t i = 0; i < M; ++i) {
        double ms, inv;
        oracle_rms_stats(x + i * N, N, eps, &ms, &inv);
        for (int64_t j = 0; j < N; ++j)
            y[i * N + j] = x[i * N + j] * inv * w[j];
    }
}

/* Fused residual RMSNorm: [TKE] §4.3 "Fused Residual RMSNorm"
 *   residual_out = x + residual;
 *   out = residual_out * rsqrt(mean(residual_out^2) + eps) * weight;
 * both outputs returned.  The sum of two fp32 or bf16 inputs is exact in
 * double. */
void oracle_residual_rmsnorm(const double *x, const double *res, const double *w, double *y,
                             double *r_out, int64_t M, int64_t N, double eps)
{
    for (int64_t i = 0; i < M; ++i) {
        double *rr = r_out + i * N;
        for (int64_t j = 0; j < N; ++j)
            rr[j] = x[i * N + j] + res[i * N + j];
        double ms, inv;
        oracle_rms_stats(rr, N, eps, &ms, &inv);
        for (int64_t j = 0; j < N; ++j)
            y[i * N + j] = rr[j] * inv * w[j];
    }
}

/* ---------------------------------------------------------------------- */
/* Exact GeLU: [TKE] §3.4 "Approx Activation" gives the exact form next to */
/* the tanh approximation:  gelu_exact(z) = 0.5 z (1 + erf(z / sqrt(2))).  */
/* ---------------------------------------------------------------------- */
double oracle_gelu_erf(double z)
{
    return 0.5 * z * (1.0 + erf(z / sqrt(2.0)));
}

void oracle_gelu_erf_array(const double *z, double *y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        y[i] = oracle_gelu_erf(z[i]);
}

/* ---------------------------------------------------------------------- */
/* LayerNorm statistics of long rows by parts.  [TKE] §6.3 "使用 online    */
/* reduction": when the reduced dimension is long, reduce it in pieces     */
/* instead of holding the whole row.  For LayerNorm a piece is summarised  */
/* by (n, mean, M2), M2 = sum of squared deviations from the piece's own   */
/* mean, and two pieces combine by the pairwise update of Chan, Golub and  */
/* LeVeque ("Updating formulae and a pairwise algorithm for computing      */
/* sample variances", 1979):                                               */
/*   n = n1 + n2,  delta = mean2 - mean1,                                  */
/*   mean = mean1 + delta * n2 / n,  M2 = M2_1 + M2_2 + delta^2 n1 n2 / n.  */
/* The row's biased variance is M2 / N.                                    */
/* ---------------------------------------------------------------------- */

/* (mean, M2) of n values by two passes (n >= 1). */
void oracle_chunk_moments(const double *x, int64_t n, double *mean_out, double *m2_out)
{
    double s = 0.0;
    for (int64_t j = 0; j < n; ++j)
        s += x[j];
    double mean = s / (double)n;
    double q = 0.0;
    for (int64_t j = 0; j < n; ++j)
        q += (x[j] - mean) * (x[j] - mean);
    *mean_out = mean;
    *m2_out = q;
}

/* Combine two summaries; a side with n = 0 is empty and is the identity. */
void oracle_chan_merge(double n1, double mean1, double m2_1, double n2, double mean2, double m2_2,
                       double *n_out, double *mean_out, double *m2_out)
{
    if (n1 == 0.0) {
        *n_out = n2, *mean_out = mean2, *m2_out = m2_2;
        return;
    }
    if (n2 == 0.0) {
        *n_out = n1, *mean_out = mean1, *m2_out = m2_1;
        return;
    }
    double n = n1 + n2;
    double delta = mean2 - mean1;
    *n_out = n;
    *mean_out = mean1 + delta * n2 / n;
    *m2_out = m2_1 + m2_2 + delta * delta * n1 * n2 / n;
}

/* Split-row statistics: S chunks of C = ceil(N / S) elements, chunk s =
 * [s*C, min(N, (s+1)*C)) (empty chunks have n = 0); per-chunk summaries go
 * to the *_parts arrays (length S, may be NULL) and are merged left to
 * right.  Returns the row's mean and M2. */
void oracle_split_moments(const double *x, int64_t N, int64_t S, double *n_parts,
                          double *mean_parts, double *m2_parts, double *mean_out, double *m2_out)
{
    int64_t C = (N + S - 1) / S;
    double n = 0.0, mean = 0.0, m2 = 0.0;
    for (int64_t s = 0; s < S; ++s) {
        int64_t lo = s * C;
        int64_t hi = lo + C < N ? lo + C : N;
        double cn = 0.0, cmean = 0.0, cm2 = 0.0;
        if (hi > lo) {
            cn = (double)(hi - lo);
            oracle_chunk_moments(x + lo, hi - lo, &cmean, &cm2);
        }
        if (n_parts)
            n_parts[s] = cn;
        if (mean_parts)
            mean_parts[s] = cmean;
        if (m2_parts)
            m2_parts[s] = cm2;
        oracle_chan_merge(n, mean, m2, cn, cmean, cm2, &n, &mean, &m2);
    }
    *mean_out = mean;
    *m2_out = m2;
}

/* LayerNorm + affine + GeLU with a choice of statistics and activation:
 * S = 0 takes the whole-row two-pass statistics of oracle_layernorm_stats,
 * S >= 1 the split statistics above (rstd = 1 / sqrt(M2 / N + eps));
 * gelu = 0 is the tanh approximation, 1 the exact erf form, 2 no activation
 * (y = z: the LayerNorm of [TKE] §4.1 "LayerNorm" alone). */
void oracle_layernorm_gelu_ex(const double *x, const double *w, const double *b, double *y,
                              int64_t M, int64_t N, double eps, int gelu, int64_t S)
{
    for (int64_t i = 0; i < M; ++i) {
        const double *xr = x + i * N;
        double *yr = y + i * N;
        double mean, var, rstd;
        if (S == 0) {
            oracle_layernorm_stats(xr, N, eps, &mean, &var, &rstd);
        } else {
            double m2;
            oracle_split_moments(xr, N, S, NULL, NULL, NULL, &mean, &m2);
            rstd = 1.0 / sqrt(m2 / (double)N + eps);
        }
        for (int64_t j = 0; j < N; ++j) {
            double z = (xr[j] - mean) * rstd * w[j] + b[j];
            if (gelu == 2)
                yr[j] = z;
            else
                yr[j] = gelu ? oracle_gelu_erf(z) : oracle_gelu_tanh(z);
        }
    }
}

/* ---------------------------------------------------------------------- */
/* Row-wise sum and max: [TKE] §2.2 "Row-wise Sum" (out[i] = sum_j x[i,j])  */
/* and §2.3 "Row-wise Max" (out[i] = max_j x[i,j], padding must be -inf). */
/* ---------------------------------------------------------------------- */
void oracle_row_sum(const double *x, double *out, int64_t M, int64_t N)
{
    for (int64_t i = 0; i < M; ++i) {
        double s = 0.0;
        for (int64_t j = 0; j < N; ++j)
            s += x[i * N + j];
        out[i] = s;
    }
}

/* NaN anywhere in a row makes its max NaN (as row_max above). */
void oracle_row_max(const double *x, double *out, int64_t M, int64_t N)
{
    for (int64_t i = 0; i < M; ++i)
        out[i] = row_max(x + i * N, N);
}

/* ---------------------------------------------------------------------- */
/* Attention: [TKE] §5.1 "Naive Attention" and §5.2 "FlashAttention-style  */
/* Forward"; [L6] §7.1-7.3.  Per (batch, head), with q, k, v, o of shape  */
/* [T][d] (contiguous, one block of T*d per (batch, head)):                */
/*   S = q k^T * scale;  causal: query i sees keys j <= i only;            */
/*   P = softmax(S) over keys;  o = P v.                                   */
/* ---------------------------------------------------------------------- */

/* The definition, row by row: scores of the visible keys, their max, the
 * exp-weights and their sum, then the weighted sum of value rows. */
void oracle_attention(const double *q, const double *k, const double *v, double *o, int64_t BH,
                      int64_t T, int64_t d, int causal, double scale)
{
    double *s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double *w = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int64_t h = 0; h < BH; ++h) {
        const double *qh = q + h * T * d, *kh = k + h * T * d, *vh = v + h * T * d;
        double *oh = o + h * T * d;
        for (int64_t i = 0; i < T; ++i) {
            int64_t n = causal ? i + 1 : T;  /* visible keys 0 .. n-1 */
            for (int64_t j = 0; j < n; ++j) {
                double dot = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    dot += qh[i * d + c] * kh[j * d + c];
                s[j] = dot * scale;
            }
            double m = row_max(s, n);
            double den = 0.0;
            for (int64_t j = 0; j < n; ++j) {
                w[j] = exp(s[j] - m);
                den += w[j];
            }
            for (int64_t c = 0; c < d; ++c) {
                double acc = 0.0;
                for (int64_t j = 0; j < n; ++j)
                    acc += w[j] * vh[j * d + c];
                oh[i * d + c] = acc / den;
            }
        }
    }
    free(s);
    free(w);
}

/* The definition for selected query rows of one (batch, head): row r of q
 * (nq rows of d) is the query at position pos[r] of a sequence of T keys and
 * values; causal: it sees keys j <= pos[r] only.  Each output row is formed
 * exactly as in oracle_attention (scores, max, exp-weights, their sum, the
 * weighted sum of value rows), so sampled rows of a long sequence can be
 * checked without computing the others. */
void oracle_attention_rows(const double *q, const int64_t *pos, int64_t nq, const double *k,
                           const double *v, double *o, int64_t T, int64_t d, int causal,
                           double scale)
{
    double *s = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    double *w = malloc(sizeof(double) * (size_t)(T > 0 ? T : 1));
    for (int64_t r = 0; r < nq; ++r) {
        int64_t n = causal ? pos[r] + 1 : T;  /* visible keys 0 .. n-1 */
        for (int64_t j = 0; j < n; ++j) {
            double dot = 0.0;
            for (int64_t c = 0; c < d; ++c)
                dot += q[r * d + c] * k[j * d + c];
            s[j] = dot * scale;
        }
        double m = row_max(s, n);
        double den = 0.0;
        for (int64_t j = 0; j < n; ++j) {
            w[j] = exp(s[j] - m);
            den += w[j];
        }
        for (int64_t c = 0; c < d; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j)
                acc += w[j] * v[j * d + c];
            o[r * d + c] = acc / den;
        }
    }
    free(s);
    free(w);
}

/* The tiled form ([L6] §7.3, [TKE] §5.2): query blocks of Br rows; for each,
 * key/value blocks of Bc rows are scanned with a per-row state m (max so
 * far), l (sum of exp so far) and acc (exp-weighted sum of value rows so
 * far):  m_new = max(m, rowmax(S_blk)), alpha = exp(m - m_new),
 * P = exp(S_blk - m_new), l = alpha l + rowsum(P), acc = alpha acc + P V_blk;
 * finally o = acc / l.  Causal masking sets the scores of keys j > i to
 * -inf; a block a row cannot see at all leaves its state unchanged. */
void oracle_flash_attention(const double *q, const double *k, const double *v, double *o,
                            int64_t BH, int64_t T, int64_t d, int causal, double scale,
                            int64_t Br, int64_t Bc)
{
    double *acc = malloc(sizeof(double) * (size_t)(Br * d));
    double *m = malloc(sizeof(double) * (size_t)Br);
    double *l = malloc(sizeof(double) * (size_t)Br);
    double *sblk = malloc(sizeof(double) * (size_t)Bc);
    for (int64_t h = 0; h < BH; ++h) {
        const double *qh = q + h * T * d, *kh = k + h * T * d, *vh = v + h * T * d;
        double *oh = o + h * T * d;
        for (int64_t i0 = 0; i0 < T; i0 += Br) {
            int64_t rows = T - i0 < Br ? T - i0 : Br;
            for (int64_t r = 0; r < rows; ++r) {
                m[r] = -INFINITY;
                l[r] = 0.0;
                for (int64_t c = 0; c < d; ++c)
                    acc[r * d + c] = 0.0;
            }
            for (int64_t j0 = 0; j0 < T; j0 += Bc) {
                int64_t cols = T - j0 < Bc ? T - j0 : Bc;
                for (int64_t r = 0; r < rows; ++r) {
                    int64_t i = i0 + r;
                    double bmax = -INFINITY;
                    for (int64_t t = 0; t < cols; ++t) {
                        int64_t j = j0 + t;
                        double dot = 0.0;
                        for (int64_t c = 0; c < d; ++c)
                            dot += qh[i * d + c] * kh[j * d + c];
                        sblk[t] = (causal && j > i) ? -INFINITY : dot * scale;
                        if (sblk[t] > bmax)
                            bmax = sblk[t];
                    }
                    if (bmax == -INFINITY)
                        continue; /* nothing visible in this block */
                    double m_new = m[r] > bmax ? m[r] : bmax;
                    double alpha = m[r] == -INFINITY ? 0.0 : exp(m[r] - m_new);
                    double psum = 0.0;
                    for (int64_t c = 0; c < d; ++c)
                        acc[r * d + c] *= alpha;
                    for (int64_t t = 0; t < cols; ++t) {
                        double p = exp(sblk[t] - m_new);
                        psum += p;
                        for (int64_t c = 0; c < d; ++c)
                            acc[r * d + c] += p * vh[(j0 + t) * d + c];
                    }
                    l[r] = alpha * l[r] + psum;
                    m[r] = m_new;
                }
            }
            for (int64_t r = 0; r < rows; ++r)
                for (int64_t c = 0; c < d; ++c)
                    oh[(i0 + r) * d + c] = acc[r * d + c] / l[r];
        }
    }
    free(acc);
    free(m);
    free(l);
    free(sblk);
}
