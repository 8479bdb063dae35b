// The exercise set's standalone primitives ("Triton Kernel 实现练习" §2.2
// "Row-wise Sum", §2.3 "Row-wise Max", §3.4 "Approx Activation"; CS336
// lecture 6 notes, "Triton GeLU").
//
// row_reduce  out[i] = sum_j x[i, j] (fp32 accumulation, stored in the input
//             format) or max_j x[i, j] (NaN-propagating; padding is -inf).
//             A row group of G waves loops over the row with U vectors per
//             lane in flight, keeps U partial results per lane, then reduces
//             them, the wave (DPP) and the G waves (LDS).  One HBM read per
//             element; the M results are the only writes.
// gelu_flat   y = GeLU(x) elementwise over a contiguous buffer: 16-byte
//             vectors, U per thread per step.
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

template <typename T, int E, int G, int W, int U, int OP>
__global__ __launch_bounds__(W *kWave) void row_reduce(const T *__restrict__ x, T *__restrict__ out,
                                                       int64_t M, int N, int64_t ldx)
{
    constexpr int RG = W / G;
    constexpr int L = G * kWave;
    constexpr float kPad = OP == RK_REDUCE_SUM ? 0.0f : -INFINITY;
    static_assert(W % G == 0, "whole row groups per workgroup");
    __shared__ float red[RG][G];

    const int wave = threadIdx.x / kWave;
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RG + grp;
    const bool ok = row < M;
    const T *xr = x + (ok ? row : 0) * ldx;
    const RowSplit<E> rs(N);
    const int vend = ok ? rs.count() : 0;
    const int lim = vend < rs.nfull ? vend : rs.nfull;

    float acc[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        acc[u] = kPad;
    // software pipeline: the next step's loads are in flight while this step
    // is reduced
    RowLoad<T, E, U, L> cur;
    cur.issue(xr, li, vend, rs, kPad, L * U <= lim);
    for (int base = 0; base < vend; base += L * U) {
        RowLoad<T, E, U, L> nxt;
        const int next = base + L * U;
        if (next < vend)
            nxt.issue(xr, next + li, vend, rs, kPad, next + L * U <= lim);
        float v[U][E];
        cur.finish(v, rs);
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

template <typename T, int E, int G, int W, int U, int OP>
static hipError_t reduce_launch(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG - 1) / RG;
    return launch(row_reduce<T, E, G, W, U, OP>, dim3(static_cast<unsigned>(blocks)),
                  dim3(W * kWave), p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y),
                  p.M, p.N, p.ldx);
}

// Row-group size by row length in vectors: one wave per row up to 1024
// vectors (16 per lane), four waves up to 8192, sixteen beyond.
template <typename T, int E, int OP>
static hipError_t reduce_dispatch(const RowProblem &p)
{
    constexpr int U = 16 / E > 4 ? 4 : (16 / E < 2 ? 2 : 16 / E);
    const int64_t nv = (p.N + E - 1) / E;
    if (nv <= 1024)
        return reduce_launch<T, E, 1, 4, U, OP>(p);
    if (nv <= 8192)
        return reduce_launch<T, E, 4, 4, U, OP>(p);
    return reduce_launch<T, E, 16, 16, U, OP>(p);
}

int64_t row_reduce_blocks(int64_t M, int64_t N, rk_dtype dtype, bool vectorized, int *threads)
{
    const int E = vectorized ? vec_elems(dtype) : 1;
    const int64_t nv = (N + E - 1) / E;
    const int rows_per_block = nv <= 1024 ? 4 : 1;
    *threads = nv <= 8192 ? 256 : 1024;
    return (M + rows_per_block - 1) / rows_per_block;
}

template <int OP>
static hipError_t reduce_run(const RowProblem &p, bool vectorized)
{
    if (p.dtype == RK_F32)
        return vectorized ? reduce_dispatch<float, 4, OP>(p) : reduce_dispatch<float, 1, OP>(p);
    return vectorized ? reduce_dispatch<bf16_t, 8, OP>(p) : reduce_dispatch<bf16_t, 1, OP>(p);
}

hipError_t row_reduce_run(const RowProblem &p, int op, bool vectorized)
{
    return op == RK_REDUCE_SUM ? reduce_run<RK_REDUCE_SUM>(p, vectorized)
                               : reduce_run<RK_REDUCE_MAX>(p, vectorized);
}

// ----------------------------------------------------------- elementwise

constexpr int kGeluThreads = 256;
constexpr int kGeluU = 4;

template <typename T, int GK>
__global__ __launch_bounds__(kGeluThreads) void gelu_flat(const T *__restrict__ x,
                                                          T *__restrict__ y, int64_t n)
{
    constexpr int E = Elem<T>::kVec;
    typedef typename RawVec<T, E>::type R;
    const int64_t nvec = n / E;
    const int64_t step = static_cast<int64_t>(gridDim.x) * kGeluThreads * kGeluU;
    for (int64_t base = static_cast<int64_t>(blockIdx.x) * kGeluThreads * kGeluU + threadIdx.x;
         base < nvec; base += step) {
        R q[kGeluU];
#pragma unroll
        for (int u = 0; u < kGeluU; ++u) {
            const int64_t i = base + u * kGeluThreads;
            if (i < nvec)
                q[u] = ld<kStreaming>(reinterpret_cast<const R *>(x) + i);
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
                store_vec<T, E, kStreaming>(y + i * E, v);
            }
        }
    }
    // the last n % E elements
    const int64_t t = nvec * E + static_cast<int64_t>(blockIdx.x) * kGeluThreads + threadIdx.x;
    if (t < n && blockIdx.x == 0)
        y[t] = Elem<T>::from_f32(gelu<GK>(Elem<T>::to_f32(x[t])));
}

template <typename T, int E, int GK>
__global__ __launch_bounds__(kGeluThreads) void gelu_rows(const T *__restrict__ x,
                                                          T *__restrict__ y, int N, int64_t ldx,
                                                          int64_t ldy)
{
    const int64_t row = blockIdx.x;
    const T *xr = x + row * ldx;
    T *yr = y + row * ldy;
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const int lim = rs.nfull;
    for (int base = 0; base < nv; base += kGeluThreads * kGeluU) {
        const bool full = base + kGeluThreads * kGeluU <= lim;
        float v[kGeluU][E];
        load_row<T, E, kGeluU, kGeluThreads>(xr, base + static_cast<int>(threadIdx.x), nv, rs,
                                              0.0f, v, full);
#pragma unroll
        for (int u = 0; u < kGeluU; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = gelu<GK>(v[u][e]);
        store_row<T, E, kGeluU, kGeluThreads>(yr, base + static_cast<int>(threadIdx.x), nv, rs, v,
                                              full);
    }
}

namespace {

template <typename T, int GK>
hipError_t flat_run(const RowProblem &p, int64_t n)
{
    constexpr int E = Elem<T>::kVec;
    const int64_t per_block = int64_t{kGeluThreads} * kGeluU;
    int64_t blocks = (n / E + per_block - 1) / per_block;
    if (blocks < 1)
        blocks = 1;  // the tail
    if (blocks > 65536)
        blocks = 65536;  // grid-stride beyond
    return launch(gelu_flat<T, GK>, dim3(static_cast<unsigned>(blocks)), dim3(kGeluThreads),
                  p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y), n);
}

template <typename T, int E, int GK>
hipError_t rows_run(const RowProblem &p)
{
    return launch(gelu_rows<T, E, GK>, dim3(static_cast<unsigned>(p.M)), dim3(kGeluThreads),
                  p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y), p.N, p.ldx,
                  p.ldy);
}

template <int GK>
hipError_t gelu_dispatch(const RowProblem &p, bool flat, bool vectorized)
{
    if (flat) {
        const int64_t n = p.M * p.N;
        return p.dtype == RK_F32 ? flat_run<float, GK>(p, n) : flat_run<bf16_t, GK>(p, n);
    }
    if (p.dtype == RK_F32)
        return vectorized ? rows_run<float, 4, GK>(p) : rows_run<float, 1, GK>(p);
    return vectorized ? rows_run<bf16_t, 8, GK>(p) : rows_run<bf16_t, 1, GK>(p);
}

}  // namespace

hipError_t gelu_run(const RowProblem &p, bool flat, bool vectorized)
{
    return p.gelu == RK_GELU_ERF ? gelu_dispatch<1>(p, flat, vectorized)
                                 : gelu_dispatch<0>(p, flat, vectorized);
}

}  // namespace rk
