// LayerNorm + affine + GeLU for rows held in memory rather than registers:
// rows beyond the register tiles' capacity, rows that are not 16-byte
// aligned, and rows split across workgroups ("Triton Kernel 实现练习" §4.1
// "LayerNorm", and §6.3 on reducing a long dimension in pieces instead of
// loading the whole row at once).
//
// The statistics are gathered by parts: each part is summarised by
// (n, mean, M2), and parts combine by the Chan-Golub-LeVeque update
// (rk::Moments).  A thread's part is one step of U vectors: its mean and M2
// are taken in two passes over registers, then merged into the thread's
// running summary.  var = M2 / N and rstd = 1 / sqrt(var + eps), as in the
// register tiles.
//
// The moments are taken of x - K, K = the row's first element (shifted
// data): M2 does not change, and the means being merged are of the size of
// the spread of the row rather than of its mean, so that a row far from zero
// (mean 100, deviation 1) keeps its centred values to fp32 precision.  The
// output centres the same way, z = ((x - K) - mean_K) rstd w + b, so the
// row mean itself is never rounded.
//
// layernorm_stream    1, 4 or 16 waves per row by the row's length (four
//                     one-wave rows share a workgroup, otherwise one row
//                     each).  Pass 1 gathers the moments (cached loads,
//                     so that pass 2 finds the row in L2 or the
//                     memory-side cache); pass 2 writes GeLU(z).
//                     2 reads + 1 write per element.
// layernorm_partials  split-row, first kernel: one workgroup per
//                     (row, chunk) writes the chunk's (mean, M2) to slot s
//                     of the row's S + 1 slots; chunk 0 also writes the
//                     shift K to slot S.
// layernorm_finish    split-row, second kernel: one workgroup per
//                     (row, chunk) merges the row's S summaries (each lane a
//                     subset, then DPP) and writes its chunk, shifting by
//                     the K of slot S.  With the slots kept in the output
//                     (no workspace), it runs twice: everything but the
//                     first vectors of each row (which hold the slots), then
//                     those vectors.
// Rows are read and written as aligned 16-byte vectors from whatever offset
// they start at (RowSpan), when input and output rows share that offset;
// weight and bias, aligned at column 0, are shifted into each row's phase
// (load_param).  E = 1 (one element per access) serves the rest.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// Summary of one step: v holds U vectors of E elements (already shifted,
// padding 0) at vector indices j0 + u * STRIDE; only row elements below jend
// count.  `full` promises that all of them count.
template <int E, int U, int STRIDE>
__device__ __forceinline__ Moments step_moments(const float (&v)[U][E], int j0, int jend,
                                                RowSpan<E> sp, bool full)
{
    float s = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e)
            s += v[u][e];
    if (full) {
        const float mean = s * (1.0f / (U * E));
        float q = 0.0f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = v[u][e] - mean;
                q = fmaf(d, d, q);
            }
        return Moments{static_cast<float>(U * E), mean, q};
    }
    int cnt = 0;
    bool valid[U][E];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int j = j0 + u * STRIDE;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            valid[u][e] = j < jend && sp.valid(j, e);
            cnt += valid[u][e] ? 1 : 0;
        }
    }
    if (cnt == 0)
        return Moments{0.0f, 0.0f, 0.0f};
    const float n = static_cast<float>(cnt);
    const float mean = s / n;
    float q = 0.0f;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e) {
            const float d = valid[u][e] ? v[u][e] - mean : 0.0f;
            q = fmaf(d, d, q);
        }
    return Moments{n, mean, q};
}

// Moments of vectors [jbeg, jend) of a row (aligned base xb), U vectors per
// thread per step, software-pipelined (the next step's loads are in flight
// while this step is summarised).  Returns the thread's own summary.
template <typename T, int E, int W, int U, int CP>
__device__ __forceinline__ Moments scan_moments(const T *__restrict__ xb, RowSpan<E> sp,
                                                int jbeg, int jend, float K)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    Moments st{0.0f, 0.0f, 0.0f};
    SpanLoad<T, E, U, NT, CP> cur;
    cur.issue(xb, jbeg + tid, jend, full(jbeg));
    for (int base = jbeg; base < jend; base += NT * U) {
        SpanLoad<T, E, U, NT, CP> nxt;
        const int next = base + NT * U;
        if (next < jend)
            nxt.issue(xb, next + tid, jend, full(next));
        const bool f = full(base);
        // padding reads as K (an element of the row, exact in T): 0 once shifted
        float v[U][E];
        cur.finish(v, sp, jend, K, f);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] -= K;
        st = merge(st, step_moments<E, U, NT>(v, base + tid, jend, sp, f));
        cur = nxt;
    }
    return st;
}

// Merge the thread summaries of a workgroup of W waves; every thread returns
// the same summary.  sn/sm/sq are W-entry LDS arrays.
template <int W>
__device__ __forceinline__ Moments ln_block_merge(Moments st, float *sn, float *sm, float *sq)
{
    st = wave_merge(st);
    if constexpr (W > 1) {
        const int wave = threadIdx.x / kWave;
        if (threadIdx.x % kWave == 0) {
            sn[wave] = st.n;
            sm[wave] = st.mean;
            sq[wave] = st.m2;
        }
        __syncthreads();
        st = Moments{sn[0], sm[0], sq[0]};
#pragma unroll
        for (int w = 1; w < W; ++w)
            st = merge(st, Moments{sn[w], sm[w], sq[w]});
    }
    return st;
}

// The row loads of ln_write_range's first step, issued by the caller ahead of
// the merge that forms the statistics, so that they are in flight meanwhile.
template <typename T, int E, int W, int U>
__device__ __forceinline__ SpanLoad<T, E, U, W * kWave> ln_write_first(const T *__restrict__ xb,
                                                                       RowSpan<E> sp, int jbeg,
                                                                       int jend)
{
    constexpr int NT = W * kWave;
    SpanLoad<T, E, U, NT> cur;
    cur.issue(xb, jbeg + static_cast<int>(threadIdx.x % NT), jend,
              sp.step_full(jbeg, jend, NT * U));
    return cur;
}

// y = GeLU(((x - K) - mean_K) rstd w + b) for vectors [jbeg, jend) of a row
// (aligned bases xb, yb; w and b by column); the first step's row loads come
// issued (ln_write_first).
template <typename T, int E, int W, int U, int GK>
__device__ __forceinline__ void ln_write_range(const T *__restrict__ xb,
                                               const T *__restrict__ w, const T *__restrict__ b,
                                               T *__restrict__ yb, RowSpan<E> sp, int jbeg,
                                               int jend, float K, float mean_k, float rstd,
                                               SpanLoad<T, E, U, W * kWave> cur)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    for (int base = jbeg; base < jend; base += NT * U) {
        const bool f = full(base);
        // weight and bias, the next step's row and this step's row are all in
        // flight before the first wait
        ParamLoad<T, E> wl[U], bl[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wl[u].issue(w, base + tid + u * NT, sp.h, sp.n, f);
            bl[u].issue(b, base + tid + u * NT, sp.h, sp.n, f);
        }
        SpanLoad<T, E, U, NT> nxt;
        const int next = base + NT * U;
        if (next < jend)
            nxt.issue(xb, next + tid, jend, full(next));
        float v[U][E], wv[U][E], bv[U][E];
        cur.finish(v, sp, jend, 0.0f, f);
#pragma unroll
        for (int u = 0; u < U; ++u) {
            wl[u].finish(wv[u], base + tid + u * NT, sp.h, sp.n, f);
            bl[u].finish(bv[u], base + tid + u * NT, sp.h, sp.n, f);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = gelu<GK>(fmaf(((v[u][e] - K) - mean_k) * rstd, wv[u][e], bv[u][e]));
        store_span<T, E, U, NT>(yb, base + tid, jend, sp, v, f);
        cur = nxt;
    }
}

// RB rows per workgroup, W waves each; several rows only for W == 1, where
// no barrier is taken and a wave past the last row may leave at once.  PH:
// rows at any offset (else every row starts on a 16-byte boundary).
template <typename T, int E, int W, int U, int GK, int RB, bool PH>
__global__ __launch_bounds__(W *kWave *RB) void layernorm_stream(
    const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b,
    T *__restrict__ y, int64_t M, int N, int64_t ldx, int64_t ldy, float inv_n, float eps)
{
    static_assert(RB == 1 || W == 1, "several rows per workgroup only with one wave each");
    __shared__ float sn[W], sm[W], sq[W];
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RB + threadIdx.x / (W * kWave);
    if (RB > 1 && row >= M)
        return;
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    const int nv = sp.count();
    const float K = Elem<T>::to_f32(xr[0]);
    Moments st = scan_moments<T, E, W, U, kCached>(xb, sp, 0, nv, K);
    const auto first = ln_write_first<T, E, W, U>(xb, sp, 0, nv);
    st = ln_block_merge<W>(st, sn, sm, sq);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(st.m2, inv_n, eps));
    ln_write_range<T, E, W, U, GK>(xb, w, b, y + row * ldy - sp.h, sp, 0, nv, K, st.mean, rstd,
                                   first);
}

template <typename T, int E, int W, int U, bool PH>
__global__ __launch_bounds__(W *kWave) void layernorm_partials(const T *__restrict__ x, int N,
                                                                int64_t ldx, int S, int C,
                                                                char *pbase, int64_t prow)
{
    __shared__ float sn[W], sm[W], sq[W];
    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    // cached: the second kernel reads the chunk again.  Every chunk of a row
    // shifts by the same K, the row's first element.
    const float K = Elem<T>::to_f32(xr[0]);
    Moments st = scan_moments<T, E, W, U, kCached>(xr - sp.h, sp, jbeg, jend, K);
    st = ln_block_merge<W>(st, sn, sm, sq);
    if (threadIdx.x == 0) {
        float2 *pr = row_partials(pbase, prow, row);
        pr[s] = make_float2(st.mean, st.m2);
        // slot S: the shift, for the output kernel (x[r][0] may be gone by
        // then when the output is the input)
        if (s == 0)
            pr[S] = make_float2(K, 0.0f);
    }
}

// Chunk s of row r: workgroup (r, s) of a grid of M S (kAllChunks,
// kAllButFirst) or workgroup r of a grid of M, s = 0 (kFirstOnly), over the
// range output_range gives.  y and pbase may name the same memory (the
// partials kept in the output), and y may be x (in place, with a
// workspace): the shift K comes from the partials' slot S, never from
// x[r][0], which chunk 0's workgroup may already have overwritten.
template <typename T, int E, int W, int U, int GK, bool PH>
__global__ __launch_bounds__(W *kWave) void layernorm_finish(
    const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b, T *y, int N,
    int64_t ldx, int64_t ldy, int S, int C, float inv_n, float eps, const char *pbase,
    int64_t prow, int part)
{
    const int64_t row = part == kFirstOnly ? blockIdx.x : blockIdx.x / S;
    const int s = part == kFirstOnly ? 0 : static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    output_range<T, E>(part, s, y + row * ldy, sp, S + 1, jbeg, jend);
    // the chunk's first loads go out before the summaries are read
    const auto first = ln_write_first<T, E, W, U>(xr - sp.h, sp, jbeg, jend);
    // Every wave merges the row's S summaries on its own (lane l takes
    // summaries l, l + 64, ...): no LDS, and every workgroup of the row forms
    // the same bits.  A chunk's count is that of the row columns its vectors
    // hold.
    Moments st{0.0f, 0.0f, 0.0f};
    const float2 *wr = row_partials(pbase, prow, row);
    const float K = wr[S].x;
    for (int i = static_cast<int>(threadIdx.x % kWave); i < S; i += kWave) {
        int jb, je;
        chunk_span<E>(sp, i, S, C, jb, je);
        const int lo = jb * E - sp.h > 0 ? jb * E - sp.h : 0;
        const int hi = je * E - sp.h < N ? je * E - sp.h : N;
        const float2 p = wr[i];
        st = merge(st, Moments{static_cast<float>(hi > lo ? hi - lo : 0), p.x, p.y});
    }
    st = wave_merge(st);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(st.m2, inv_n, eps));
    // the summaries in the output are overwritten below: every wave has read
    // them first
    if (part == kFirstOnly)
        __syncthreads();
    ln_write_range<T, E, W, U, GK>(xr - sp.h, w, b, y + row * ldy - sp.h, sp, jbeg, jend, K,
                                   st.mean, rstd, first);
}

// ------------------------------------------------------------------ host

namespace {

constexpr int kSplitW = 4;    // 256 threads per chunk

// Vectors per thread per step: 64 bytes of row per thread (four fp32 or two
// bf16 vectors), which with the weight and bias of the output pass fits the
// 128 VGPRs of a 1024-thread workgroup.
constexpr int step_vectors(int E) { return E == 8 ? 2 : 4; }

template <typename T, int E, bool PH, int W, int U = step_vectors(E)>
hipError_t stream_launch(const RowProblem &p)
{
    // one-wave rows go four to a workgroup
    constexpr int RB = W == 1 ? 4 : 1;
    auto kernel = p.gelu == RK_GELU_ERF    ? layernorm_stream<T, E, W, U, 1, RB, PH>
                  : p.gelu == RK_GELU_NONE ? layernorm_stream<T, E, W, U, 2, RB, PH>
                                           : layernorm_stream<T, E, W, U, 0, RB, PH>;
    return launch(kernel, dim3(static_cast<unsigned>((p.M + RB - 1) / RB)), dim3(W * kWave * RB),
                  p.stream, static_cast<const T *>(p.x), static_cast<const T *>(p.w),
                  static_cast<const T *>(p.b), static_cast<T *>(p.y), p.M, p.N, p.ldx, p.ldy,
                  static_cast<float>(1.0 / p.N), p.eps);
}

// One workgroup per row, 1 to 16 waves by the row's length.
template <typename T, int E, bool PH>
hipError_t stream_run(const RowProblem &p)
{
    const int64_t nvec = (p.N + 2 * E - 2) / E;
    if (nvec <= kShortRowVectors)
        return stream_launch<T, E, PH, 1, 1>(p);
    switch (stream_waves(nvec, step_vectors(E))) {
    case 16:
        return stream_launch<T, E, PH, 16>(p);
    case 4:
        return stream_launch<T, E, PH, 4>(p);
    default:
        return stream_launch<T, E, PH, 1>(p);
    }
}

// Split chunks: two vectors per thread per step for both formats (fp32 at
// four measured 12% slower on 64 rows of 262144: the 256-thread workgroups
// then hold more registers than they gain in loads in flight).
constexpr int split_vectors(int E) { return E == 1 ? 4 : 2; }

template <typename T, int E, bool PH>
hipError_t split_run(const RowProblem &p, int S, int C, SplitPartials pt)
{
    constexpr int U = split_vectors(E);
    const dim3 grid(static_cast<unsigned>(p.M * S));
    const dim3 block(kSplitW * kWave);
    const T *x = static_cast<const T *>(p.x);
    hipError_t err = launch(layernorm_partials<T, E, kSplitW, U, PH>, grid, block, p.stream, x,
                            p.N, p.ldx, S, C, pt.base, pt.row_bytes);
    if (err != hipSuccess)
        return err;
    auto kernel = p.gelu == RK_GELU_ERF    ? layernorm_finish<T, E, kSplitW, U, 1, PH>
                  : p.gelu == RK_GELU_NONE ? layernorm_finish<T, E, kSplitW, U, 2, PH>
                                           : layernorm_finish<T, E, kSplitW, U, 0, PH>;
    const T *w = static_cast<const T *>(p.w);
    const T *b = static_cast<const T *>(p.b);
    T *y = static_cast<T *>(p.y);
    const float inv_n = static_cast<float>(1.0 / p.N);
    if (!pt.in_output)
        return launch(kernel, grid, block, p.stream, x, w, b, y, p.N, p.ldx, p.ldy, S, C, inv_n,
                      p.eps, pt.base, pt.row_bytes, int{kAllChunks});
    err = launch(kernel, grid, block, p.stream, x, w, b, y, p.N, p.ldx, p.ldy, S, C, inv_n, p.eps,
                 pt.base, pt.row_bytes, int{kAllButFirst});
    if (err != hipSuccess)
        return err;
    return launch(kernel, dim3(static_cast<unsigned>(p.M)), block, p.stream, x, w, b, y, p.N,
                  p.ldx, p.ldy, S, C, inv_n, p.eps, pt.base, pt.row_bytes, int{kFirstOnly});
}

template <typename T>
hipError_t stream_io(const RowProblem &p, RowIo io)
{
    constexpr int E = Elem<T>::kVec;
    if (io == kIoAligned)
        return stream_run<T, E, false>(p);
    if (io == kIoPhased)
        return stream_run<T, E, true>(p);
    return stream_run<T, 1, false>(p);
}

template <typename T>
hipError_t split_io(const RowProblem &p, int S, int C, SplitPartials pt, RowIo io)
{
    constexpr int E = Elem<T>::kVec;
    if (io == kIoAligned)
        return split_run<T, E, false>(p, S, C, pt);
    if (io == kIoPhased)
        return split_run<T, E, true>(p, S, C, pt);
    return split_run<T, 1, false>(p, S, C, pt);
}

}  // namespace

hipError_t layernorm_stream_run(const RowProblem &p, RowIo io)
{
    return p.dtype == RK_F32 ? stream_io<float>(p, io) : stream_io<bf16_t>(p, io);
}

hipError_t layernorm_split_run(const RowProblem &p, int splits, int chunk, SplitPartials parts,
                               RowIo io)
{
    return p.dtype == RK_F32 ? split_io<float>(p, splits, chunk, parts, io)
                             : split_io<bf16_t>(p, splits, chunk, parts, io);
}

}  // namespace rk
