// RMSNorm and fused residual-add + RMSNorm ("Triton Kernel 实现练习" §4.2
// "RMSNorm" and §4.3 "Fused Residual RMSNorm").
//
// Per row: v = x (or v = x + residual, rounded to the storage format and
// written out as residual_out, so that y is exactly the RMSNorm of the stored
// residual_out, as with an unfused add followed by a norm);
// inv_rms = 1 / sqrt(sum v^2 / N + eps); y = v * inv_rms * w.  One reduction
// (fp32), no centring.  Padded columns hold 0, which adds nothing to the sum
// of squares, so no column select is needed even in the general variants.
//
// rmsnorm_tile  the row stays in VGPRs: one HBM read of each input and one
//               write of each output per element; weight is loaded once per
//               row group for its R rows.
// rmsnorm_loop  one workgroup per row, two passes over the row in memory;
//               any N, any alignment.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// v += u, then round v to the storage format T (a no-op for fp32).
template <typename T, int V, int E>
__device__ __forceinline__ void add_rounded(float (&v)[V][E], const float (&u)[V][E])
{
#pragma unroll
    for (int k = 0; k < V; ++k)
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[k][e] += u[k][e];
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            if constexpr (E == 1) {
                v[k][0] = Elem<T>::to_f32(Elem<T>::from_f32(v[k][0]));
            } else {
#pragma unroll
                for (int e = 0; e < E; e += 2) {
                    const f32x2_t f = {v[k][e], v[k][e + 1]};
                    const uint32_t q =
                        __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
                    v[k][e] = __uint_as_float(q << 16);
                    v[k][e + 1] = __uint_as_float(q & 0xFFFF0000u);
                }
            }
        }
    }
}

template <typename T, int G, int V, int W, int R, bool EXACT, bool RES>
__global__ __launch_bounds__(W *kWave) void rmsnorm_tile(
    const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
    T *__restrict__ y, T *__restrict__ ro, int64_t M, int N, int64_t ldx, int64_t ldr,
    int64_t ldy, int64_t ldo, float inv_n, float eps)
{
    constexpr int E = Elem<T>::kVec;
    constexpr int RG = W / G;
    constexpr int L = G * kWave;
    static_assert(W % G == 0, "whole row groups per workgroup");
    __shared__ float red[2][RG][G];

    const int wave = threadIdx.x / kWave;
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const bool slots_full = EXACT || V * L <= rs.nfull;

    auto row_of = [&](int r) { return (static_cast<int64_t>(blockIdx.x) * R + r) * RG + grp; };

    RowLoad<T, E, V, L> xl, rl;
    auto issue_row = [&](int r) {
        const int64_t row = row_of(r);
        const bool ok = row < M;
        const int64_t rr = ok ? row : 0;
        const bool full = EXACT || (ok && slots_full);
        xl.issue(x + rr * ldx, li, ok ? nv : 0, rs, 0.0f, full);
        if constexpr (RES)
            rl.issue(res + rr * ldr, li, ok ? nv : 0, rs, 0.0f, full);
    };
    issue_row(0);
    RowLoad<T, E, V, L, kCached> wl;
    wl.issue(w, li, nv, rs, 0.0f, slots_full);
    float wv[V][E];

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row_of(r);
        const bool row_ok = row < M;
        const int64_t rr = row_ok ? row : 0;
        const int vend = row_ok ? nv : 0;
        const bool store_full = EXACT || (row_ok && slots_full);

        float v[V][E];
        xl.finish(v, rs);
        if constexpr (RES) {
            float u[V][E];
            rl.finish(u, rs);
            add_rounded<T>(v, u);
        }
        if (r + 1 < R)
            issue_row(r + 1);
        if constexpr (RES) {
            if (!EXACT || row_ok)
                store_row<T, E, V, L>(ro + rr * ldo, li, vend, rs, v, store_full);
        }

        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                q = fmaf(v[k][e], v[k][e], q);
        q = wave_sum(q);
        if constexpr (G > 1) {
            const int buf = r & 1;
            if (threadIdx.x % kWave == 0)
                red[buf][grp][wig] = q;
            __syncthreads();
            q = red[buf][grp][0];
#pragma unroll
            for (int g = 1; g < G; ++g)
                q += red[buf][grp][g];
        }
        const float inv = __builtin_amdgcn_rsqf(fmaf(q, inv_n, eps));

        if (r == 0)
            wl.finish(wv, rs);
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[k][e] = v[k][e] * inv * wv[k][e];
        if (!EXACT || row_ok)
            store_row<T, E, V, L>(y + rr * ldy, li, vend, rs, v, store_full);
    }
}

template <typename T, int G, int V, int W, int R, bool EXACT, bool RES>
static hipError_t rmsnorm_tile_run(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG * R - 1) / (RG * R);
    const float inv_n = static_cast<float>(1.0 / p.N);
    return launch(rmsnorm_tile<T, G, V, W, R, EXACT, RES>, dim3(static_cast<unsigned>(blocks)),
                  dim3(W * kWave), p.stream, static_cast<const T *>(p.x),
                  static_cast<const T *>(p.r), static_cast<const T *>(p.w),
                  static_cast<T *>(p.y), static_cast<T *>(p.ro), p.M, p.N, p.ldx, p.ldr, p.ldy,
                  p.ldo, inv_n, p.eps);
}

template <typename T, bool RES, int G, int V, int W, int R = 1, bool EXACT = false>
constexpr TileVariant tile()
{
    return TileVariant{G, V, W, R, G * V * kWave * Elem<T>::kVec, EXACT,
                       &rmsnorm_tile_run<T, G, V, W, R, EXACT, RES>};
}
template <typename T, bool RES, int G, int V, int W, int R = 1>
constexpr TileVariant exact()
{
    return tile<T, RES, G, V, W, R, true>();
}

// Preference rule as for the LayerNorm tables: exact entries first, then
// general entries in ascending capacity; alt(): run by index only.
#define RK_RMS_TABLE(NAME, T, RES)                                                               \
    static const TileVariant NAME[] = {                                                          \
        exact<T, RES, 1, 1, 4>(),  exact<T, RES, 1, 2, 4>(),  exact<T, RES, 1, 3, 4>(),          \
        exact<T, RES, 1, 4, 4>(),  exact<T, RES, 1, 8, 4>(),  exact<T, RES, 4, 4, 4>(),          \
        exact<T, RES, 8, 4, 8>(),  exact<T, RES, 16, 4, 16>(), tile<T, RES, 1, 1, 4>(),          \
        tile<T, RES, 1, 2, 4>(),   tile<T, RES, 1, 3, 4>(),   tile<T, RES, 1, 4, 4>(),           \
        tile<T, RES, 1, 8, 4>(),   tile<T, RES, 4, 4, 4>(),   tile<T, RES, 8, 4, 8>(),           \
        tile<T, RES, 16, 4, 16>(),                                                               \
    }
// bf16 general entries between 8192 and 20480 use 8-wave row groups (N =
// 10000: 46 us against 68 us for 16 x 2 at 128 MiB, as for LayerNorm).
#define RK_RMS_TABLE_BF16(NAME, RES)                                                             \
    static const TileVariant NAME[] = {                                                          \
        exact<bf16_t, RES, 1, 1, 4>(),    exact<bf16_t, RES, 1, 2, 4>(),                         \
        exact<bf16_t, RES, 1, 4, 4>(),    exact<bf16_t, RES, 4, 2, 4, 2>(),                      \
        exact<bf16_t, RES, 8, 2, 8>(),    exact<bf16_t, RES, 16, 2, 16>(),                       \
        exact<bf16_t, RES, 16, 4, 16>(),  tile<bf16_t, RES, 1, 1, 4>(),                          \
        tile<bf16_t, RES, 1, 2, 4>(),     tile<bf16_t, RES, 1, 4, 4>(),                          \
        tile<bf16_t, RES, 2, 4, 4>(),     tile<bf16_t, RES, 8, 2, 8>(),                          \
        tile<bf16_t, RES, 8, 3, 8>(),     tile<bf16_t, RES, 8, 4, 8>(),                          \
        tile<bf16_t, RES, 8, 5, 8>(),     tile<bf16_t, RES, 16, 4, 16>(),                        \
        alt(exact<bf16_t, RES, 2, 4, 4>()), alt(exact<bf16_t, RES, 4, 2, 4>()),                  \
        alt(tile<bf16_t, RES, 16, 2, 16>()),                                                     \
    }

RK_RMS_TABLE(kRmsF32, float, false);
RK_RMS_TABLE(kResRmsF32, float, true);
RK_RMS_TABLE_BF16(kRmsBF16, false);
RK_RMS_TABLE_BF16(kResRmsBF16, true);

#undef RK_RMS_TABLE
#undef RK_RMS_TABLE_BF16

template <size_t K>
static const TileVariant *table(const TileVariant (&t)[K], int *count)
{
    *count = static_cast<int>(K);
    return t;
}

const TileVariant *rmsnorm_variants(rk_dtype dtype, bool residual, int *count)
{
    if (dtype == RK_F32)
        return residual ? table(kResRmsF32, count) : table(kRmsF32, count);
    return residual ? table(kResRmsBF16, count) : table(kRmsBF16, count);
}

// ------------------------------------------------------- looping kernel

template <typename T, int E, int W, int U, bool RES>
__global__ __launch_bounds__(W *kWave) void rmsnorm_loop(
    const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
    T *__restrict__ y, T *__restrict__ ro, int N, int64_t ldx, int64_t ldr, int64_t ldy,
    int64_t ldo, float inv_n, float eps)
{
    constexpr int NT = W * kWave;
    __shared__ float red[W];
    const int64_t row = blockIdx.x;
    const T *xr = x + row * ldx;
    const T *rr = RES ? res + row * ldr : nullptr;
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const int tid = static_cast<int>(threadIdx.x);

    float q = 0.0f;
    for (int base = 0; base < nv; base += NT * U) {
        float v[U][E];
        load_row<T, E, U, NT>(xr, base + tid, nv, rs, 0.0f, v);
        if constexpr (RES) {
            float u[U][E];
            load_row<T, E, U, NT>(rr, base + tid, nv, rs, 0.0f, u);
            add_rounded<T>(v, u);
        }
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e)
                q = fmaf(v[i][e], v[i][e], q);
    }
    q = wave_sum(q);
    if constexpr (W > 1) {
        if (tid % kWave == 0)
            red[tid / kWave] = q;
        __syncthreads();
        q = red[0];
#pragma unroll
        for (int i = 1; i < W; ++i)
            q += red[i];
    }
    const float inv = __builtin_amdgcn_rsqf(fmaf(q, inv_n, eps));

    for (int base = 0; base < nv; base += NT * U) {
        float v[U][E], wv[U][E];
        load_row<T, E, U, NT>(xr, base + tid, nv, rs, 0.0f, v);
        if constexpr (RES) {
            float u[U][E];
            load_row<T, E, U, NT>(rr, base + tid, nv, rs, 0.0f, u);
            add_rounded<T>(v, u);
            store_row<T, E, U, NT>(ro + row * ldo, base + tid, nv, rs, v);
        }
        load_row<T, E, U, NT, kCached>(w, base + tid, nv, rs, 0.0f, wv);
#pragma unroll
        for (int i = 0; i < U; ++i)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[i][e] = v[i][e] * inv * wv[i][e];
        store_row<T, E, U, NT>(y + row * ldy, base + tid, nv, rs, v);
    }
}

namespace {
constexpr int kLoopW = 4;
constexpr int kLoopU = 4;

template <typename T, int E, bool RES>
hipError_t loop_run(const RowProblem &p)
{
    return launch(rmsnorm_loop<T, E, kLoopW, kLoopU, RES>, dim3(static_cast<unsigned>(p.M)),
                  dim3(kLoopW * kWave), p.stream, static_cast<const T *>(p.x),
                  static_cast<const T *>(p.r), static_cast<const T *>(p.w),
                  static_cast<T *>(p.y), static_cast<T *>(p.ro), p.N, p.ldx, p.ldr, p.ldy, p.ldo,
                  static_cast<float>(1.0 / p.N), p.eps);
}

template <bool RES>
hipError_t loop_dispatch(const RowProblem &p, bool vectorized)
{
    if (p.dtype == RK_F32)
        return vectorized ? loop_run<float, 4, RES>(p) : loop_run<float, 1, RES>(p);
    return vectorized ? loop_run<bf16_t, 8, RES>(p) : loop_run<bf16_t, 1, RES>(p);
}
}  // namespace

hipError_t rmsnorm_loop_run(const RowProblem &p, bool residual, bool vectorized)
{
    return residual ? loop_dispatch<true>(p, vectorized) : loop_dispatch<false>(p, vectorized);
}

}  // namespace rk
