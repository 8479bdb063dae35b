// Online softmax for long rows ("Triton Kernel 实现练习" §2.5 "Online Softmax";
// "第 6 讲：GPU Kernels 与 Triton" §7.2 "Online Softmax").
//
// State of a scanned part of a row: (m, d) = (its max, sum of exp(x - m) over
// it).  A new block moves the state to m' = max(m, block max),
// d' = d exp(m - m') + sum exp(block - m').  Two partial states of disjoint
// parts merge with the same rescaling (rk::merge).
//
// online_stream    1, 4 or 16 waves per row by the row's length (four
//                  one-wave rows share a workgroup, otherwise one row
//                  each).  Pass 1: every lane folds the blocks it loads into
//                  its own state; lanes merge through DPP, waves through
//                  LDS.  Pass 2 re-reads the row and writes exp(x - m) / d.
//                  2 reads + 1 write per element.
// online_partials  split-row, first kernel: one workgroup per (row, chunk)
//                  writes the chunk's (m_s, d_s) to the workspace (or into
//                  the row's first output chunk).
// online_finish    split-row, second kernel: one workgroup per (row, chunk)
//                  merges the row's S partials (each lane a subset, then
//                  DPP) and writes its chunk.  With the partials kept in the
//                  output (no workspace), it runs twice: everything but the
//                  first vectors of each row (which hold the partials), then
//                  those vectors, one workgroup per row.  The output pass
//                  runs each range's steps last first (see last_step).
// Rows are read and written as aligned 16-byte vectors from whatever offset
// they start at (RowSpan), when input and output rows share that offset;
// E = 1 (one element per access) serves the rest.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// exp(x - m) of an output element: compensated for fp32 I/O.
template <typename T>
__device__ __forceinline__ float softmax_exp(float x, float m, float m_log2e)
{
    if constexpr (sizeof(T) == 4)
        return exp_shifted_accurate(x, m);
    else
        return exp_shifted_fast(x, m_log2e);
}

// exp(x - m) of a term of a partial sum d: errors average out there.
template <typename T>
__device__ __forceinline__ float softmax_term(float x, float m, float m_log2e)
{
    if constexpr (sizeof(T) == 4)
        return exp_shifted_term(x, m);
    else
        return exp_shifted_fast(x, m_log2e);
}

// Fold U vectors of E elements into a lane state.
template <typename T, int U, int E>
__device__ __forceinline__ SoftmaxState fold(SoftmaxState st, const float (&v)[U][E])
{
    float bm = -INFINITY;
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
        for (int e = 0; e < E; ++e)
            bm = nanmax(bm, v[u][e]);
    const float mn = nanmax(st.m, bm);
    float sum = 0.0f;
    if (mn != -INFINITY) {  // else every value seen is -inf: nothing to add
        const float mL = mn * 1.4426950408889634f;
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                sum += softmax_term<T>(v[u][e], mn, mL);
    }
    SoftmaxState r;
    r.m = mn;
    r.d = st.d * rescale_factor(st.m, mn) + sum;
    return r;
}

// Merge the lane states of a workgroup of W waves; every thread returns the
// same state.  `sm`/`sd` are W-entry LDS arrays.
template <int W>
__device__ __forceinline__ SoftmaxState block_merge(SoftmaxState st, float *sm, float *sd)
{
    st = wave_merge(st);
    if constexpr (W > 1) {
        const int wave = threadIdx.x / kWave;
        if (threadIdx.x % kWave == 0) {
            sm[wave] = st.m;
            sd[wave] = st.d;
        }
        __syncthreads();
        st = SoftmaxState{sm[0], sd[0]};
#pragma unroll
        for (int w = 1; w < W; ++w)
            st = merge(st, SoftmaxState{sm[w], sd[w]});
    }
    return st;
}

// Vectors [jbeg, jend) of a row (the aligned vectors of RowSpan<E>, base xb),
// U vectors per thread per step, folded into the thread's state.  The
// scan's loads are cached (CP = kCached) when the same data is read again
// soon.
template <typename T, int E, int W, int U, int CP>
__device__ __forceinline__ SoftmaxState scan_range(const T *__restrict__ xb, RowSpan<E> sp,
                                                   int jbeg, int jend)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    SoftmaxState st{-INFINITY, 0.0f};
    // a step is full when all its vectors hold row elements only and lie
    // below jend: no masks then
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    // software pipeline: the next step's loads are in flight while this
    // step's values are folded
    SpanLoad<T, E, U, NT, CP> cur;
    cur.issue(xb, jbeg + tid, jend, full(jbeg));
    for (int base = jbeg; base < jend; base += NT * U) {
        SpanLoad<T, E, U, NT, CP> nxt;
        const int next = base + NT * U;
        if (next < jend)
            nxt.issue(xb, next + tid, jend, full(next));
        float v[U][E];
        cur.finish(v, sp, jend, -INFINITY, full(base));
        st = fold<T, U, E>(st, v);
        cur = nxt;
    }
    return st;
}

// The loads of the first step write_range runs (the range's last), issued by
// the caller ahead of the merge that forms the row's state, so that they are
// in flight meanwhile.
template <typename T, int E, int W, int U>
__device__ __forceinline__ SpanLoad<T, E, U, W * kWave> write_first(const T *__restrict__ xb,
                                                                    RowSpan<E> sp, int jbeg,
                                                                    int jend)
{
    constexpr int NT = W * kWave;
    const int base = last_step(jbeg, jend, NT * U);
    SpanLoad<T, E, U, NT> cur;
    cur.issue(xb, base + static_cast<int>(threadIdx.x % NT), jend > jbeg ? jend : base,
              sp.step_full(base, jend, NT * U));
    return cur;
}

// Write exp(x - m) / d for vectors [jbeg, jend) of a row (bases xb, yb),
// last step first; that step's loads come issued (write_first).
template <typename T, int E, int W, int U>
__device__ __forceinline__ void write_range(const T *__restrict__ xb, T *__restrict__ yb,
                                            RowSpan<E> sp, int jbeg, int jend, SoftmaxState st,
                                            SpanLoad<T, E, U, W * kWave> cur)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    const float inv = 1.0f / st.d;
    const float mL = st.m * 1.4426950408889634f;
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    for (int base = last_step(jbeg, jend, NT * U); base >= jbeg; base -= NT * U) {
        SpanLoad<T, E, U, NT> nxt;
        const int next = base - NT * U;
        if (next >= jbeg)
            nxt.issue(xb, next + tid, jend, full(next));
        const bool f = full(base);
        float v[U][E];
        cur.finish(v, sp, jend, -INFINITY, f);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = softmax_exp<T>(v[u][e], st.m, mL) * inv;
        store_span<T, E, U, NT>(yb, base + tid, jend, sp, v, f);
        cur = nxt;
    }
}

// RB rows per workgroup, W waves each; several rows only for W == 1, where
// no barrier is taken and a wave past the last row may leave at once.  PH:
// rows at any offset (else every row starts on a 16-byte boundary).
template <typename T, int E, int W, int U, int RB, bool PH>
__global__ __launch_bounds__(W *kWave *RB) void online_stream(const T *__restrict__ x,
                                                               T *__restrict__ y, int64_t M,
                                                               int N, int64_t ldx, int64_t ldy)
{
    static_assert(RB == 1 || W == 1, "several rows per workgroup only with one wave each");
    __shared__ float sm[W], sd[W];
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RB + threadIdx.x / (W * kWave);
    if (RB > 1 && row >= M)
        return;
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    T *yb = y + row * ldy - sp.h;
    const int nv = sp.count();
    // pass 1 leaves the row in the caches for pass 2
    SoftmaxState st = scan_range<T, E, W, U, kCached>(xb, sp, 0, nv);
    const auto first = write_first<T, E, W, U>(xb, sp, 0, nv);
    st = block_merge<W>(st, sm, sd);
    write_range<T, E, W, U>(xb, yb, sp, 0, nv, st, first);
}

// Partials of chunk s = blockIdx.x % S of row blockIdx.x / S.
template <typename T, int E, int W, int U, bool PH>
__global__ __launch_bounds__(W *kWave) void online_partials(const T *__restrict__ x, int N,
                                                             int64_t ldx, int S, int C,
                                                             char *pbase, int64_t prow)
{
    __shared__ float sm[W], sd[W];
    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    // cached: the second kernel reads the chunk again (measured: 15% faster
    // than non-temporal loads here)
    SoftmaxState st = scan_range<T, E, W, U, kCached>(xr - sp.h, sp, jbeg, jend);
    st = block_merge<W>(st, sm, sd);
    if (threadIdx.x == 0)
        row_partials(pbase, prow, row)[s] = make_float2(st.m, st.d);
}

// Chunk s of row r: workgroup (r, s) of a grid of M S (kAllChunks,
// kAllButFirst) or workgroup r of a grid of M, s = 0 (kFirstOnly), over the
// range output_range gives.
// y and pbase may name the same memory (the partials kept in the output).
template <typename T, int E, int W, int U, bool PH>
__global__ __launch_bounds__(W *kWave) void online_finish(const T *__restrict__ x, T *y, int N,
                                                           int64_t ldx, int64_t ldy, int S, int C,
                                                           const char *pbase, int64_t prow,
                                                           int part)
{
    const int64_t row = part == kFirstOnly ? blockIdx.x : blockIdx.x / S;
    const int s = part == kFirstOnly ? 0 : static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    output_range<T, E>(part, s, y + row * ldy, sp, S, jbeg, jend);
    // the chunk's first loads go out before the partials are read
    const auto first = write_first<T, E, W, U>(xr - sp.h, sp, jbeg, jend);
    // Every wave merges the row's S partials on its own (lane l takes
    // partials l, l + 64, ...), so no LDS is needed, and every workgroup of
    // the row forms the same bits.
    SoftmaxState st{-INFINITY, 0.0f};
    const float2 *wr = row_partials(pbase, prow, row);
    for (int i = static_cast<int>(threadIdx.x % kWave); i < S; i += kWave) {
        const float2 p = wr[i];
        st = merge(st, SoftmaxState{p.x, p.y});
    }
    st = wave_merge(st);
    // the partials in the output are overwritten below: every wave has read
    // them first
    if (part == kFirstOnly)
        __syncthreads();
    write_range<T, E, W, U>(xr - sp.h, y + row * ldy - sp.h, sp, jbeg, jend, st, first);
}

// ------------------------------------------------------------------ host

namespace {

constexpr int kStreamU = 4;
constexpr int kSplitW = 4;    // 256 threads per chunk
constexpr int kSplitU = 4;

template <typename T, int E, bool PH, int W, int U = kStreamU>
hipError_t stream_launch(const RowProblem &p)
{
    // one-wave rows go four to a workgroup
    constexpr int RB = W == 1 ? 4 : 1;
    return launch(online_stream<T, E, W, U, RB, PH>,
                  dim3(static_cast<unsigned>((p.M + RB - 1) / RB)), dim3(W * kWave * RB), p.stream, static_cast<const T *>(p.x),
                  static_cast<T *>(p.y), p.M, p.N, p.ldx, p.ldy);
}

// One workgroup per row, 1 to 16 waves by the row's length.
template <typename T, int E, bool PH>
hipError_t stream_run(const RowProblem &p)
{
    const int64_t nvec = (p.N + 2 * E - 2) / E;
    if (nvec <= kShortRowVectors)
        return stream_launch<T, E, PH, 1, 1>(p);
    switch (stream_waves(nvec, kStreamU)) {
    case 16:
        return stream_launch<T, E, PH, 16>(p);
    case 4:
        return stream_launch<T, E, PH, 4>(p);
    default:
        return stream_launch<T, E, PH, 1>(p);
    }
}

template <typename T, int E, bool PH>
hipError_t split_run(const RowProblem &p, int S, int C, SplitPartials pt)
{
    const dim3 grid(static_cast<unsigned>(p.M * S));
    const dim3 block(kSplitW * kWave);
    hipError_t err = launch(online_partials<T, E, kSplitW, kSplitU, PH>, grid, block, p.stream,
                            static_cast<const T *>(p.x), p.N, p.ldx, S, C, pt.base, pt.row_bytes);
    if (err != hipSuccess)
        return err;
    auto finish = online_finish<T, E, kSplitW, kSplitU, PH>;
    const T *x = static_cast<const T *>(p.x);
    T *y = static_cast<T *>(p.y);
    if (!pt.in_output)
        return launch(finish, grid, block, p.stream, x, y, p.N, p.ldx, p.ldy, S, C, pt.base,
                      pt.row_bytes, int{kAllChunks});
    err = launch(finish, grid, block, p.stream, x, y, p.N, p.ldx, p.ldy, S, C, pt.base,
                 pt.row_bytes, int{kAllButFirst});
    if (err != hipSuccess)
        return err;
    return launch(finish, dim3(static_cast<unsigned>(p.M)), block, p.stream, x, y, p.N, p.ldx,
                  p.ldy, S, C, pt.base, pt.row_bytes, int{kFirstOnly});
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

hipError_t online_stream_run(const RowProblem &p, RowIo io)
{
    return p.dtype == RK_F32 ? stream_io<float>(p, io) : stream_io<bf16_t>(p, io);
}

hipError_t online_split_run(const RowProblem &p, int splits, int chunk, SplitPartials parts,
                            RowIo io)
{
    return p.dtype == RK_F32 ? split_io<float>(p, splits, chunk, parts, io)
                             : split_io<bf16_t>(p, splits, chunk, parts, io);
}

}  // namespace rk
