// Register-resident stable row softmax ("Triton Kernel 实现练习" §2.4 "Softmax",
// stable version; CS336 "Kernels, Triton" notes, "Triton Softmax").
//
// A row group of G waves (G x 64 lanes) holds one row in VGPRs as V 16-byte
// vectors per lane, so each element is read from HBM once and written once:
//   load -> per-lane max -> wave64 DPP max -> (G > 1) LDS combine
//        -> e = exp(x - m) kept in registers, per-lane sum -> wave / LDS sum
//        -> y = e * (1 / sum) -> store.
// Lanes of a row are contiguous 16-byte vectors, so a wave's load instruction
// covers 1 KiB of consecutive memory.  Columns beyond N are padded with -inf
// in registers (never loaded).
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// EXACT: compiled for N == V * L * E, i.e. every register slot of a row group
// is a column of its row: loads and stores need no masks and nothing is
// padded.  Rows past M (the last workgroup) then read row 0 and store
// nothing.
// PH: rows at any offset past a 16-byte boundary (the output's rows at the
// same offset), read and written as the aligned vectors that cover them
// (RowSpan), their ends masked.
template <typename T, int G, int V, int W, bool EXACT, bool PH>
__global__ __launch_bounds__(W *kWave) void softmax_tile(const T *__restrict__ x,
                                                          T *__restrict__ y, int64_t M, int N,
                                                          int64_t ldx, int64_t ldy)
{
    static_assert(!(EXACT && PH), "a phased row is never an exact fit");
    constexpr int E = Elem<T>::kVec;
    constexpr int RG = W / G;    // row groups per workgroup
    constexpr int L = G * kWave; // lanes per row
    static_assert(W % G == 0, "whole row groups per workgroup");
    __shared__ float red_max[RG][G];
    __shared__ float red_sum[RG][G];

    // wave-uniform: row bases stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const RowSplit<E> rs(N);

    const int64_t row = static_cast<int64_t>(blockIdx.x) * RG + grp;
    const bool row_ok = row < M;
    const int64_t r = row_ok ? row : 0;
    const T *xr = x + r * ldx;
    T *yr = y + r * ldy;

    const int vend = row_ok ? rs.count() : 0;
    // every vector slot of the row group holds a complete vector of a row
    const bool full = EXACT || (row_ok && V * L <= rs.nfull);

    float v[V][E];
    RowSpan<E> sp{0, N};
    int jend = 0;
    if constexpr (PH) {
        sp.h = row_phase<T, E>(xr);
        jend = row_ok ? sp.count() : 0;
        SpanLoad<T, E, V, L> l;
        l.issue(xr - sp.h, li, jend, false);
        l.finish(v, sp, jend, -INFINITY, false);
    } else {
        load_row<T, E, V, L>(xr, li, vend, rs, -INFINITY, v, full);
    }

    float m = -INFINITY;
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e)
            m = nanmax(m, v[k][e]);
    m = wave_max(m);
    if constexpr (G > 1) {
        if (threadIdx.x % kWave == 0)
            red_max[grp][wig] = m;
        __syncthreads();
        m = red_max[grp][0];
#pragma unroll
        for (int g = 1; g < G; ++g)
            m = nanmax(m, red_max[grp][g]);
    }

    float s = 0.0f;
    if constexpr (sizeof(T) == 4) {
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                v[k][e] = exp_shifted_accurate(v[k][e], m);
                s += v[k][e];
            }
    } else {
        const float mL = m * 1.4426950408889634f;
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                v[k][e] = exp_shifted_fast(v[k][e], mL);
                s += v[k][e];
            }
    }
    s = wave_sum(s);
    if constexpr (G > 1) {
        if (threadIdx.x % kWave == 0)
            red_sum[grp][wig] = s;
        __syncthreads();
        s = red_sum[grp][0];
#pragma unroll
        for (int g = 1; g < G; ++g)
            s += red_sum[grp][g];
    }

    // 1/s by the hardware reciprocal (1 ulp): one rounding more than a
    // division, once per row
    const float inv = __builtin_amdgcn_rcpf(s);
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[k][e] *= inv;
    if constexpr (PH) {
        store_span<T, E, V, L>(yr - sp.h, li, jend, sp, v, false);
    } else if (EXACT) {
        if (row_ok)
            store_row<T, E, V, L>(yr, li, vend, rs, v, true);
    } else {
        store_row<T, E, V, L>(yr, li, vend, rs, v, full);
    }
}

template <typename T, int G, int V, int W, bool EXACT, bool PH>
static hipError_t softmax_tile_run(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG - 1) / RG;
    return launch(softmax_tile<T, G, V, W, EXACT, PH>, dim3(static_cast<unsigned>(blocks)),
                  dim3(W * kWave), p.stream, static_cast<const T *>(p.x), static_cast<T *>(p.y),
                  p.M, p.N, p.ldx, p.ldy);
}

// A general variant (any N up to its capacity, and rows at any offset up to
// capacity - E + 1) and an exact one (N equal to its capacity).
// The phased form of a general tile (null for an exact one).
template <typename T, int G, int V, int W, bool EXACT>
constexpr hipError_t (*phased_run())(const RowProblem &)
{
    if constexpr (!EXACT)
        return &softmax_tile_run<T, G, V, W, false, true>;
    else
        return nullptr;
}

template <typename T, int G, int V, int W, bool EXACT = false>
constexpr TileVariant tile()
{
    return TileVariant{G, V, W, 1, G * V * kWave * Elem<T>::kVec, EXACT,
                       &softmax_tile_run<T, G, V, W, EXACT, false>, false,
                       phased_run<T, G, V, W, EXACT>()};
}
template <typename T, int G, int V, int W>
constexpr TileVariant exact()
{
    return tile<T, G, V, W, true>();
}

// Preference order: the dispatcher takes the first exact entry whose max_n is
// N, else the first general entry whose max_n covers N (general entries in
// ascending capacity).  alt(): run by index only, never picked.
static const TileVariant kSoftmaxF32[] = {
    exact<float, 1, 1, 4>(),   // N = 256
    exact<float, 1, 2, 4>(),   // N = 512
    exact<float, 1, 3, 4>(),   // N = 768
    exact<float, 2, 2, 4>(),   // N = 1024
    exact<float, 1, 8, 4>(),   // N = 2048
    exact<float, 4, 4, 4>(),   // N = 4096
    exact<float, 8, 4, 8>(),   // N = 8192
    exact<float, 16, 4, 16>(), // N = 16384
    tile<float, 1, 1, 4>(),    // N <= 256
    tile<float, 1, 2, 4>(),    // N <= 512
    tile<float, 1, 3, 4>(),    // N <= 768
    tile<float, 1, 4, 4>(),    // N <= 1024 (8192 x 1000: 12.91 us vs 13.14 for 2 x 2, trace)
    tile<float, 1, 8, 4>(),    // N <= 2048
    tile<float, 4, 4, 4>(),    // N <= 4096
    tile<float, 8, 4, 8>(),    // N <= 8192
    tile<float, 16, 4, 16>(),  // N <= 16384
    alt(tile<float, 2, 2, 4>()),
    alt(tile<float, 4, 1, 4>()),
    alt(tile<float, 2, 8, 4>()),
    alt(exact<float, 1, 4, 4>()),
    alt(exact<float, 8, 8, 8>()),  // large rows with fewer waves per row
    alt(tile<float, 8, 8, 8>()),
    alt(exact<float, 4, 8, 4>()),
};

static const TileVariant kSoftmaxBF16[] = {
    exact<bf16_t, 1, 1, 4>(),   // N = 512
    exact<bf16_t, 1, 2, 4>(),   // N = 1024
    exact<bf16_t, 1, 4, 4>(),   // N = 2048
    exact<bf16_t, 4, 2, 4>(),   // N = 4096
    exact<bf16_t, 8, 2, 8>(),   // N = 8192
    exact<bf16_t, 16, 2, 16>(), // N = 16384
    exact<bf16_t, 16, 4, 16>(), // N = 32768
    tile<bf16_t, 1, 1, 4>(),    // N <= 512
    tile<bf16_t, 1, 2, 4>(),    // N <= 1024
    tile<bf16_t, 1, 4, 4>(),    // N <= 2048
    tile<bf16_t, 4, 2, 4>(),    // N <= 4096
    tile<bf16_t, 8, 2, 8>(),    // N <= 8192
    tile<bf16_t, 16, 2, 16>(),  // N <= 16384
    tile<bf16_t, 16, 4, 16>(),  // N <= 32768
    alt(tile<bf16_t, 1, 8, 4>()),
    alt(tile<bf16_t, 2, 4, 4>()),
    alt(tile<bf16_t, 8, 1, 8>()),
    alt(exact<bf16_t, 1, 8, 4>()),
    alt(exact<bf16_t, 2, 4, 4>()),
    alt(exact<bf16_t, 8, 1, 8>()),
    alt(exact<bf16_t, 8, 8, 8>()),  // large rows with fewer waves per row
    alt(tile<bf16_t, 8, 8, 8>()),
    alt(exact<bf16_t, 8, 4, 8>()),
};

const TileVariant *softmax_variants(rk_dtype dtype, int *count)
{
    if (dtype == RK_F32) {
        *count = static_cast<int>(sizeof(kSoftmaxF32) / sizeof(kSoftmaxF32[0]));
        return kSoftmaxF32;
    }
    *count = static_cast<int>(sizeof(kSoftmaxBF16) / sizeof(kSoftmaxBF16[0]));
    return kSoftmaxBF16;
}

}  // namespace rk
