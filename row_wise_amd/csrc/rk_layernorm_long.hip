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
//                     (row, chunk) writes the chunk's (mean, M2).
// layernorm_finish    split-row, second kernel: one workgroup per
//                     (row, chunk) merges the row's S summaries (each lane a
//                     subset, then DPP) and writes its chunk.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// Summary of one step: v holds U vectors of E elements (already shifted) at
// vector indices vi0 + u * STRIDE; only elements of the row that are below
// vend count (padding is 0 after the shift).  `full` promises that all of
// them count.
template <int E, int U, int STRIDE>
__device__ __forceinline__ Moments step_moments(const float (&v)[U][E], int vi0, int vend,
                                                RowSplit<E> rs, bool full)
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
        const int vi = vi0 + u * STRIDE;
#pragma unroll
        for (int e = 0; e < E; ++e) {
            valid[u][e] = vi < vend && (vi < rs.nfull || (vi == rs.nfull && e < rs.tail));
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

// Moments of vectors [vbeg, vend) of a row, U vectors per thread per step,
// software-pipelined (the next step's loads are in flight while this step is
// summarised).  Returns the thread's own summary.
template <typename T, int E, int W, int U, int CP>
__device__ __forceinline__ Moments scan_moments(const T *__restrict__ xr, RowSplit<E> rs,
                                                int vbeg, int vend, float K)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    const int lim = vend < rs.nfull ? vend : rs.nfull;
    Moments st{0.0f, 0.0f, 0.0f};
    // padding loads as K (an element of the row, exact in T): 0 once shifted
    RowLoad<T, E, U, NT, CP> cur;
    cur.issue(xr, vbeg + tid, vend, rs, K, vbeg + NT * U <= lim);
    for (int base = vbeg; base < vend; base += NT * U) {
        RowLoad<T, E, U, NT, CP> nxt;
        const int next = base + NT * U;
        if (next < vend)
            nxt.issue(xr, next + tid, vend, rs, K, next + NT * U <= lim);
        float v[U][E];
        cur.finish(v, rs);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] -= K;
        st = merge(st, step_moments<E, U, NT>(v, base + tid, vend, rs, base + NT * U <= lim));
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

// y = GeLU(((x - K) - mean_K) rstd w + b) for vectors [vbeg, vend) of a row.
template <typename T, int E, int W, int U, int GK>
__device__ __forceinline__ void ln_write_range(const T *__restrict__ xr,
                                               const T *__restrict__ w, const T *__restrict__ b,
                                               T *__restrict__ yr, RowSplit<E> rs, int vbeg,
                                               int vend, float K, float mean_k, float rstd)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    const int lim = vend < rs.nfull ? vend : rs.nfull;
    RowLoad<T, E, U, NT> cur;
    cur.issue(xr, vbeg + tid, vend, rs, 0.0f, vbeg + NT * U <= lim);
    for (int base = vbeg; base < vend; base += NT * U) {
        const bool full = base + NT * U <= lim;
        RowLoad<T, E, U, NT, kCached> wl, bl;
        wl.issue(w, base + tid, vend, rs, 0.0f, full);
        bl.issue(b, base + tid, vend, rs, 0.0f, full);
        RowLoad<T, E, U, NT> nxt;
        const int next = base + NT * U;
        if (next < vend)
            nxt.issue(xr, next + tid, vend, rs, 0.0f, next + NT * U <= lim);
        float v[U][E], wv[U][E], bv[U][E];
        cur.finish(v, rs);
        wl.finish(wv, rs);
        bl.finish(bv, rs);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = gelu<GK>(fmaf(((v[u][e] - K) - mean_k) * rstd, wv[u][e], bv[u][e]));
        store_row<T, E, U, NT>(yr, base + tid, vend, rs, v, full);
        cur = nxt;
    }
}

// RB rows per workgroup, W waves each; several rows only for W == 1, where
// no barrier is taken and a wave past the last row may leave at once.
template <typename T, int E, int W, int U, int GK, int RB>
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
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const float K = Elem<T>::to_f32(xr[0]);
    Moments st = scan_moments<T, E, W, U, kCached>(xr, rs, 0, nv, K);
    st = ln_block_merge<W>(st, sn, sm, sq);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(st.m2, inv_n, eps));
    ln_write_range<T, E, W, U, GK>(xr, w, b, y + row * ldy, rs, 0, nv, K, st.mean, rstd);
}

// Vector range [vbeg, vend) of chunk s (C elements, a multiple of E).
template <int E>
__device__ __forceinline__ void chunk_range(int N, int s, int C, int nv, int &vbeg, int &vend)
{
    const int64_t c0 = static_cast<int64_t>(s) * C;
    vbeg = static_cast<int>(c0 < N ? c0 / E : nv);
    vend = static_cast<int>(c0 + C < N ? (c0 + C) / E : nv);
}

template <typename T, int E, int W, int U>
__global__ __launch_bounds__(W *kWave) void layernorm_partials(const T *__restrict__ x, int N,
                                                                int64_t ldx, int S, int C,
                                                                float2 *__restrict__ ws)
{
    __shared__ float sn[W], sm[W], sq[W];
    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    const RowSplit<E> rs(N);
    int vbeg, vend;
    chunk_range<E>(N, s, C, rs.count(), vbeg, vend);
    // cached: the second kernel reads the chunk again.  Every chunk of a row
    // shifts by the same K, the row's first element.
    const T *xr = x + row * ldx;
    Moments st = scan_moments<T, E, W, U, kCached>(xr, rs, vbeg, vend, Elem<T>::to_f32(xr[0]));
    st = ln_block_merge<W>(st, sn, sm, sq);
    if (threadIdx.x == 0)
        ws[blockIdx.x] = make_float2(st.mean, st.m2);
}

template <typename T, int E, int W, int U, int GK>
__global__ __launch_bounds__(W *kWave) void layernorm_finish(
    const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b,
    T *__restrict__ y, int N, int64_t ldx, int64_t ldy, int S, int C, float inv_n, float eps,
    const float2 *__restrict__ ws)
{
    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    // Every wave merges the row's S summaries on its own (lane l takes
    // summaries l, l + 64, ...): no LDS, no barrier, and every workgroup of
    // the row forms the same bits.  A chunk's count follows from N, S and C.
    Moments st{0.0f, 0.0f, 0.0f};
    const float2 *wr = ws + row * S;
    for (int i = static_cast<int>(threadIdx.x % kWave); i < S; i += kWave) {
        const int64_t c0 = static_cast<int64_t>(i) * C;
        const int64_t cn = c0 >= N ? 0 : (N - c0 < C ? N - c0 : C);
        const float2 p = wr[i];
        st = merge(st, Moments{static_cast<float>(cn), p.x, p.y});
    }
    st = wave_merge(st);
    const float rstd = __builtin_amdgcn_rsqf(fmaf(st.m2, inv_n, eps));

    const RowSplit<E> rs(N);
    int vbeg, vend;
    chunk_range<E>(N, s, C, rs.count(), vbeg, vend);
    const T *xr = x + row * ldx;
    ln_write_range<T, E, W, U, GK>(xr, w, b, y + row * ldy, rs, vbeg, vend,
                                   Elem<T>::to_f32(xr[0]), st.mean, rstd);
}

// ------------------------------------------------------------------ host

namespace {

constexpr int kSplitW = 4;    // 256 threads per chunk

// Vectors per thread per step: 64 bytes of row per thread (four fp32 or two
// bf16 vectors), which with the weight and bias of the output pass fits the
// 128 VGPRs of a 1024-thread workgroup.
constexpr int step_vectors(int E) { return E == 8 ? 2 : 4; }

template <typename T, int E, int W>
hipError_t stream_launch(const RowProblem &p)
{
    constexpr int U = step_vectors(E);
    // one-wave rows go four to a workgroup
    constexpr int RB = W == 1 ? 4 : 1;
    auto kernel = p.gelu == RK_GELU_ERF ? layernorm_stream<T, E, W, U, 1, RB>
                                        : layernorm_stream<T, E, W, U, 0, RB>;
    return launch(kernel, dim3(static_cast<unsigned>((p.M + RB - 1) / RB)), dim3(W * kWave * RB),
                  p.stream, static_cast<const T *>(p.x), static_cast<const T *>(p.w),
                  static_cast<const T *>(p.b), static_cast<T *>(p.y), p.M, p.N, p.ldx, p.ldy,
                  static_cast<float>(1.0 / p.N), p.eps);
}

// One workgroup per row, 1 to 16 waves by the row's length.
template <typename T, int E>
hipError_t stream_run(const RowProblem &p)
{
    switch (stream_waves((p.N + E - 1) / E, step_vectors(E))) {
    case 16:
        return stream_launch<T, E, 16>(p);
    case 4:
        return stream_launch<T, E, 4>(p);
    default:
        return stream_launch<T, E, 1>(p);
    }
}

template <typename T, int E>
hipError_t split_run(const RowProblem &p, int S, int C, void *ws)
{
    constexpr int U = step_vectors(E);
    const dim3 grid(static_cast<unsigned>(p.M * S));
    hipError_t err = launch(layernorm_partials<T, E, kSplitW, U>, grid,
                            dim3(kSplitW * kWave), p.stream, static_cast<const T *>(p.x), p.N,
                            p.ldx, S, C, static_cast<float2 *>(ws));
    if (err != hipSuccess)
        return err;
    auto kernel = p.gelu == RK_GELU_ERF ? layernorm_finish<T, E, kSplitW, U, 1>
                                        : layernorm_finish<T, E, kSplitW, U, 0>;
    return launch(kernel, grid, dim3(kSplitW * kWave), p.stream, static_cast<const T *>(p.x),
                  static_cast<const T *>(p.w), static_cast<const T *>(p.b),
                  static_cast<T *>(p.y), p.N, p.ldx, p.ldy, S, C, static_cast<float>(1.0 / p.N),
                  p.eps, static_cast<const float2 *>(ws));
}

}  // namespace

hipError_t layernorm_stream_run(const RowProblem &p, bool vectorized)
{
    if (p.dtype == RK_F32)
        return vectorized ? stream_run<float, 4>(p) : stream_run<float, 1>(p);
    return vectorized ? stream_run<bf16_t, 8>(p) : stream_run<bf16_t, 1>(p);
}

hipError_t layernorm_split_run(const RowProblem &p, int splits, int chunk, void *workspace,
                               bool vectorized)
{
    if (p.dtype == RK_F32)
        return vectorized ? split_run<float, 4>(p, splits, chunk, workspace)
                          : split_run<float, 1>(p, splits, chunk, workspace);
    return vectorized ? split_run<bf16_t, 8>(p, splits, chunk, workspace)
                      : split_run<bf16_t, 1>(p, splits, chunk, workspace);
}

}  // namespace rk
