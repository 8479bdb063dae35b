// The exercise set's standalone primitives ("Triton Kernel 实现练习" §2.2
// "Row-wise Sum", §2.3 "Row-wise Max", §3.4 "Approx Activation"; CS336
// lecture 6 notes, "Triton GeLU").
//
// row_reduce  out[i] = sum_j x[i, j] (fp32 accumulation, stored in the input
//             format) or max_j x[i, j] (NaN-propagating; padding is -inf).
//             A row group of G waves loops over the row with U vectors per
//             lane in flight, keeps U partial results per lane, then reduces
//             them, the wave (DPP) and the G waves (LDS).  One HBM read per
//             element; the M results are the only writes.  A row at any
//             offset is read as the aligned 16-byte vectors that cover it
//             (RowSpan), its ends masked.
// row_reduce_partials + row_reduce_finish
//             long rows in few rows, split across workgroups ("Triton Kernel
//             实现练习" §6.3 on reducing a long dimension in pieces): the
//             first kernel writes each chunk's fp32 sum or max to a
//             workspace, the second reduces each row's S partials in a fixed
//             order and writes the result.
// gelu_flat   y = GeLU(x) elementwise over a contiguous buffer: 16-byte
//             vectors, U per thread per step, from whatever offset the
//             buffer starts at (the output at the same offset).
// gelu_rows   the same for rows with a pitch: one workgroup per row.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

template <int OP>
__device__ __forceinline__ float reduce_op(float a, float b)
{
    if constexpr (OP == RK_REDUCE_SUM)
        return a + b;
    else
        return nanmax(a, b);
}

template <typename T, int E, int G, int W, int U, int OP, bool PH>
__global__ __launch_bounds__(W *kWave) void row_reduce(const T *__restrict__ x, T *__restrict__ out,
                                                       int64_t M, int N, int64_t ldx)
{
    constexpr int RG = W / G;
    constexpr int L = G * kWave;
    constexpr float kPad = OP == RK_REDUCE_SUM ? 0.0f : -INFINITY;
    static_assert(W % G == 0, "whole row groups per workgroup");
    __shared__ float red[RG][G];

    // wave-uniform: row bases stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RG + grp;
    const bool ok = row < M;
    const T *xr = x + (ok ? row : 0) * ldx;
    // the row as the aligned vectors that cover it, whatever its offset
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    const int jend = ok ? sp.count() : 0;
    auto full = [&](int base) { return sp.step_full(base, jend, L * U); };

    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc[u] = kPad;
    // software pipeline: the next step's loads are in flight while this step
    // is reduced
    SpanLoad<T, E, U, L> cur;
    cur.issue(xb, li, jend, full(0));
    for (int base = 0; base < jend; base += L * U) {
        SpanLoad<T, E, U, L> nxt;
        const int next = base + L * U;
        if (next < jend)
            nxt.issue(xb, next + li, jend, full(next));
        float v[U][E];
        cur.finish(v, sp, jend, kPad, full(base));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[u] = reduce_op<OP>(acc[u], v[u][e]);
        cur = nxt;
    }
    float a = acc[0];
#pragma unroll
    for (int u = 1; u < U; ++u)
        a = reduce_op<OP>(a, acc[u]);
    if constexpr (OP == RK_REDUCE_SUM)
        a = wave_sum(a);
    else
        a = wave_max(a);
    if constexpr (G > 1) {
        if (threadIdx.x % kWave == 0)
            red[grp][wig] = a;
        __syncthreads();
        a = red[grp][0];
#pragma unroll
        for (int g = 1; g < G; ++g)
            a = reduce_op<OP>(a, red[grp][g]);
    }
    if (ok && li == 0)
        out[row] = Elem<T>::from_f32(a);
}

template <typename T, int E, int G, int W, int U, int OP, bool PH>
static hipError_t reduce_launch(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG - 1) / RG;
    return launch(row_reduce<T, E, G, W, U, OP, PH>, dim3(static_cast<unsigned>(blocks)),
                  dim3(W * kWave), p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y),
                  p.M, p.N, p.ldx);
}

// Row-group size by row length in vectors (phase included): one wave per
// row up to 1024 vectors (16 per lane), four waves up to 8192, sixteen
// beyond.
constexpr int64_t kReduceWave1 = 1024;
constexpr int64_t kReduceWave4 = 8192;

inline int64_t reduce_vectors(int64_t N, int E) { return (N + 2 * E - 2) / E; }

template <typename T, int OP, bool PH>
static hipError_t reduce_dispatch(const RowProblem &p)
{
    constexpr int E = Elem<T>::kVec;
    constexpr int U = 16 / E > 4 ? 4 : (16 / E < 2 ? 2 : 16 / E);
    const int64_t nv = reduce_vectors(p.N, E);
    if (nv <= kReduceWave1)
        return reduce_launch<T, E, 1, 4, U, OP, PH>(p);
    if (nv <= kReduceWave4)
        return reduce_launch<T, E, 4, 4, U, OP, PH>(p);
    return reduce_launch<T, E, 16, 16, U, OP, PH>(p);
}

int64_t row_reduce_blocks(int64_t M, int64_t N, rk_dtype dtype, int *threads)
{
    const int64_t nv = reduce_vectors(N, vec_elems(dtype));
    const int rows_per_block = nv <= kReduceWave1 ? 4 : 1;
    *threads = nv <= kReduceWave4 ? 256 : 1024;
    return (M + rows_per_block - 1) / rows_per_block;
}

// Rows that all start on 16-byte boundaries take the kernel compiled for
// that; others read each row from its own offset.
template <int OP>
static hipError_t reduce_run(const RowProblem &p)
{
    const int es = elem_size(p.dtype);
    const bool aligned = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && (p.ldx * es) % 16 == 0;
    if (p.dtype == RK_F32)
        return aligned ? reduce_dispatch<float, OP, false>(p) : reduce_dispatch<float, OP, true>(p);
    return aligned ? reduce_dispatch<bf16_t, OP, false>(p) : reduce_dispatch<bf16_t, OP, true>(p);
}

hipError_t row_reduce_run(const RowProblem &p, int op)
{
    return op == RK_REDUCE_SUM ? reduce_run<RK_REDUCE_SUM>(p) : reduce_run<RK_REDUCE_MAX>(p);
}

// ------------------------------------------------------ split row reduce

constexpr int kSplitReduceWaves = 4;  // 256-thread workgroups

// Chunk s = blockIdx.x % S of row blockIdx.x / S (the vectors chunk_span
// gives, over the aligned vectors that cover the row): its fp32 sum or max,
// U vectors per thread in flight, to part[row * S + s].  An empty chunk
// gives the identity (0 or -inf).
template <typename T, int E, int U, int OP, bool PH>
__global__ __launch_bounds__(kSplitReduceWaves *kWave) void row_reduce_partials(
    const T *__restrict__ x, float *__restrict__ part, int N, int64_t ldx, int S, int C)
{
    constexpr int W = kSplitReduceWaves;
    constexpr int NT = W * kWave;
    constexpr float kPad = OP == RK_REDUCE_SUM ? 0.0f : -INFINITY;
    __shared__ float red[W];

    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    const int tid = static_cast<int>(threadIdx.x);
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };

    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc[u] = kPad;
    SpanLoad<T, E, U, NT> cur;
    cur.issue(xb, jbeg + tid, jend, full(jbeg));
    for (int base = jbeg; base < jend; base += NT * U) {
        SpanLoad<T, E, U, NT> nxt;
        const int next = base + NT * U;
        if (next < jend)
            nxt.issue(xb, next + tid, jend, full(next));
        float v[U][E];
        cur.finish(v, sp, jend, kPad, full(base));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                acc[u] = reduce_op<OP>(acc[u], v[u][e]);
        cur = nxt;
    }
    float a = acc[0];
#pragma unroll
    for (int u = 1; u < U; ++u)
        a = reduce_op<OP>(a, acc[u]);
    if constexpr (OP == RK_REDUCE_SUM)
        a = wave_sum(a);
    else
        a = wave_max(a);
    if (tid % kWave == 0)
        red[tid / kWave] = a;
    __syncthreads();
    if (tid == 0) {
        float r = red[0];
#pragma unroll
        for (int w = 1; w < W; ++w)
            r = reduce_op<OP>(r, red[w]);
        part[row * S + s] = r;
    }
}

// out[row] from the row's S partials: one wave per row, four rows per
// workgroup; lane l folds partials l, l + 64, ... in that order, then the
// wave reduces (DPP), so every call adds in the same order.
template <typename T, int OP>
__global__ __launch_bounds__(kSplitReduceWaves *kWave) void row_reduce_finish(
    const float *__restrict__ part, T *__restrict__ out, int64_t M, int S)
{
    constexpr float kPad = OP == RK_REDUCE_SUM ? 0.0f : -INFINITY;
    const int64_t row = static_cast<int64_t>(blockIdx.x) * kSplitReduceWaves + threadIdx.x / kWave;
    const int lane = static_cast<int>(threadIdx.x % kWave);
    if (row >= M)  // the whole wave: no barrier follows
        return;
    const float *pr = part + row * S;
    float a = kPad;
    for (int i = lane; i < S; i += kWave)
        a = reduce_op<OP>(a, pr[i]);
    if constexpr (OP == RK_REDUCE_SUM)
        a = wave_sum(a);
    else
        a = wave_max(a);
    if (lane == 0)
        out[row] = Elem<T>::from_f32(a);
}

template <typename T, int OP, bool PH>
static hipError_t reduce_split_launch(const RowProblem &p, int splits, int chunk, float *part)
{
    constexpr int E = Elem<T>::kVec;
    constexpr int U = 16 / E > 4 ? 4 : (16 / E < 2 ? 2 : 16 / E);
    const hipError_t e = launch(row_reduce_partials<T, E, U, OP, PH>,
                                dim3(static_cast<unsigned>(p.M * splits)),
                                dim3(kSplitReduceWaves * kWave), p.stream,
                                static_cast<const T *>(p.x), part, p.N, p.ldx, splits, chunk);
    if (e != hipSuccess)
        return e;
    const int64_t blocks = (p.M + kSplitReduceWaves - 1) / kSplitReduceWaves;
    return launch(row_reduce_finish<T, OP>, dim3(static_cast<unsigned>(blocks)),
                  dim3(kSplitReduceWaves * kWave), p.stream, static_cast<const float *>(part),
                  static_cast<T *>(p.y), p.M, splits);
}

template <int OP>
static hipError_t reduce_split_run(const RowProblem &p, int splits, int chunk, float *part)
{
    const int es = elem_size(p.dtype);
    const bool aligned = reinterpret_cast<uintptr_t>(p.x) % 16 == 0 && (p.ldx * es) % 16 == 0;
    if (p.dtype == RK_F32)
        return aligned ? reduce_split_launch<float, OP, false>(p, splits, chunk, part)
                       : reduce_split_launch<float, OP, true>(p, splits, chunk, part);
    return aligned ? reduce_split_launch<bf16_t, OP, false>(p, splits, chunk, part)
                   : reduce_split_launch<bf16_t, OP, true>(p, splits, chunk, part);
}

hipError_t row_reduce_split_run(const RowProblem &p, int op, int splits, int chunk, float *part)
{
    return op == RK_REDUCE_SUM ? reduce_split_run<RK_REDUCE_SUM>(p, splits, chunk, part)
                               : reduce_split_run<RK_REDUCE_MAX>(p, splits, chunk, part);
}

// ----------------------------------------------------------- elementwise

constexpr int kGeluThreads = 256;
constexpr int kGeluU = 4;

// y = GeLU(x) over n contiguous elements whose first sits h elements past a
// 16-byte boundary, y at the same offset: the aligned vectors of x - h, U per
// thread per step, grid-stride.  Only the first and the last vector can hold
// elements outside the buffer; their loads stay in a block that holds one of
// its elements, and their stores go element by element.
template <typename T, int GK>
__global__ __launch_bounds__(kGeluThreads) void gelu_flat(const T *__restrict__ x,
                                                          T *__restrict__ y, int64_t n, int h)
{
    constexpr int E = Elem<T>::kVec;
    typedef typename RawVec<T, E>::type R;
    const T *xb = x - h;
    T *yb = y - h;
    const int64_t nvec = (h + n + E - 1) / E;
    const int64_t full_lo = h != 0 ? 1 : 0;
    const int64_t full_hi = (h + n) / E;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kGeluThreads * kGeluU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kGeluThreads * kGeluU + threadIdx.x;
         base < nvec; base += step) {
        R q[kGeluU];
#pragma unroll
        for (int u = 0; u < kGeluU; ++u) {
            const int64_t i = base + u * kGeluThreads;
            if (i < nvec)
                q[u] = ld<kStreaming>(reinterpret_cast<const R *>(xb + i * E));
        }
#pragma unroll
        for (int u = 0; u < kGeluU; ++u) {
            const int64_t i = base + u * kGeluThreads;
            if (i < nvec) {
                float v[E];
                unpack<T, E>(q[u], v);
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[e] = gelu<GK>(v[e]);
                if (i >= full_lo && i < full_hi) {
                    store_vec<T, E, kStreaming>(yb + i * E, v);
                } else {
#pragma unroll
                    for (int e = 0; e < E; ++e) {
                        const int64_t c = i * E + e - h;
                        if (c >= 0 && c < n)
                            y[c] = Elem<T>::from_f32(v[e]);
                    }
                }
            }
        }
    }
}

// The same for rows with a pitch: one workgroup per row, each row read and
// written as the aligned vectors that cover it (RowSpan; output rows at the
// same offsets), or element by element (E = 1).
template <typename T, int E, int GK, bool PH>
__global__ __launch_bounds__(kGeluThreads) void gelu_rows(const T *__restrict__ x,
                                                          T *__restrict__ y, int N, int64_t ldx,
                                                          int64_t ldy)
{
    constexpr int NT = kGeluThreads;
    const int64_t row = blockIdx.x;
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    T *yb = y + row * ldy - sp.h;
    const int nv = sp.count();
    const int tid = static_cast<int>(threadIdx.x);
    for (int base = 0; base < nv; base += NT * kGeluU) {
        const bool full = sp.step_full(base, nv, NT * kGeluU);
        SpanLoad<T, E, kGeluU, NT> l;
        l.issue(xb, base + tid, nv, full);
        float v[kGeluU][E];
        l.finish(v, sp, nv, 0.0f, full);
#pragma unroll
        for (int u = 0; u < kGeluU; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = gelu<GK>(v[u][e]);
        store_span<T, E, kGeluU, NT>(yb, base + tid, nv, sp, v, full);
    }
}

namespace {

template <typename T, int GK>
hipError_t flat_run(const RowProblem &p, int64_t n)
{
    constexpr int E = Elem<T>::kVec;
    const int h = static_cast<int>((reinterpret_cast<uintptr_t>(p.x) % 16) / sizeof(T));
    const int64_t per_block = int64_t{kGeluThreads} * kGeluU;
    int64_t blocks = ((h + n + E - 1) / E + per_block - 1) / per_block;
    if (blocks > 65536)
        blocks = 65536;  // grid-stride beyond
    return launch(gelu_flat<T, GK>, dim3(static_cast<unsigned>(blocks)), dim3(kGeluThreads),
                  p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y), n, h);
}

template <typename T, int E, int GK, bool PH>
hipError_t rows_run(const RowProblem &p)
{
    return launch(gelu_rows<T, E, GK, PH>, dim3(static_cast<unsigned>(p.M)), dim3(kGeluThreads),
                  p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y), p.N, p.ldx,
                  p.ldy);
}

template <typename T, int GK>
hipError_t rows_io(const RowProblem &p, RowIo io)
{
    constexpr int E = Elem<T>::kVec;
    if (io == kIoAligned)
        return rows_run<T, E, GK, false>(p);
    if (io == kIoPhased)
        return rows_run<T, E, GK, true>(p);
    return rows_run<T, 1, GK, false>(p);
}

template <int GK>
hipError_t gelu_dispatch(const RowProblem &p, bool flat, RowIo io)
{
    if (flat) {
        const int64_t n = p.M * p.N;
        return p.dtype == RK_F32 ? flat_run<float, GK>(p, n) : flat_run<bf16_t, GK>(p, n);
    }
    return p.dtype == RK_F32 ? rows_io<float, GK>(p, io) : rows_io<bf16_t, GK>(p, io);
}

}  // namespace

hipError_t gelu_run(const RowProblem &p, bool flat, RowIo io)
{
    return p.gelu == RK_GELU_ERF ? gelu_dispatch<1>(p, flat, io) : gelu_dispatch<0>(p, flat, io);
}

}  // namespace rk
