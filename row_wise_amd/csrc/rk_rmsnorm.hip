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
// rmsnorm_loop  1, 4 or 16 waves per row by its length, two passes over the
//               row in memory; any N, any alignment.
// rmsnorm_partials + rmsnorm_finish
//               long rows in few rows, split across workgroups: the first
//               kernel writes each chunk's sum of squares, the second sums
//               the row's S partials and writes its chunk (run twice when
//               the partials are kept in the output: everything but the
//               first vectors of each row, which hold them, then those).
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

// PH: rows at any offset past a 16-byte boundary (residual, y and
// residual_out rows at the same offset), read and written as the aligned
// vectors that cover them (RowSpan), their ends masked; the weight is shifted
// into each row's offset as it is used.  One row per row group.
template <typename T, int G, int V, int W, int R, bool EXACT, bool RES, bool PH>
__global__ __launch_bounds__(W *kWave) void rmsnorm_tile(
    const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
    T *__restrict__ y, T *__restrict__ ro, int64_t M, int N, int64_t ldx, int64_t ldr,
    int64_t ldy, int64_t ldo, float inv_n, float eps)
{
    static_assert(!PH || (!EXACT && R == 1), "phased rows: general tiles, one row per group");
    constexpr int E = Elem<T>::kVec;
    constexpr int RG = W / G;
    constexpr int L = G * kWave;
    static_assert(W % G == 0, "whole row groups per workgroup");
    __shared__ float red[2][RG][G];

    // wave-uniform: row bases stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const bool slots_full = EXACT || V * L <= rs.nfull;

    // kSame (an exact tile of one row group and two rows): a second row past
    // M is the first row again.  Its loads are issued before any store of the
    // first row, and it writes the same bytes again (in place too), so every
    // store is unconditional and the second row's loads can be awaited just
    // before the first row's output stores (wait_vmem) without also waiting
    // for those stores, which a branch around them would make the compiler do.
    constexpr bool kSame = EXACT && !PH && R == 2 && RG == 1;
    auto row_of = [&](int r) {
        const int64_t i = (static_cast<int64_t>(blockIdx.x) * R + r) * RG + grp;
        return kSame && i >= M ? M - 1 : i;
    };

    RowLoad<T, E, V, L> xl, rl;
    SpanLoad<T, E, V, L> xs, rsl;  // PH
    RowSpan<E> sp{0, N};
    int jend = 0;
    auto issue_row = [&](int r) {
        const int64_t row = row_of(r);
        const bool ok = kSame || row < M;
        const int64_t rr = ok ? row : 0;
        if constexpr (PH) {
            sp.h = row_phase<T, E>(x + rr * ldx);
            jend = ok ? sp.count() : 0;
            xs.issue(x + rr * ldx - sp.h, li, jend, false);
            if constexpr (RES)
                rsl.issue(res + rr * ldr - sp.h, li, jend, false);
        } else {
            const bool full = EXACT || (ok && slots_full);
            xl.issue(x + rr * ldx, li, ok ? nv : 0, rs, 0.0f, full);
            if constexpr (RES)
                rl.issue(res + rr * ldr, li, ok ? nv : 0, rs, 0.0f, full);
        }
    };
    issue_row(0);
    RowLoad<T, E, V, L, kCached> wl;
    // PH: the weight blocks of small tiles are loaded with the row (two per
    // vector); larger tiles load them as they are used
    constexpr bool kParamAhead = PH && V <= 2;
    ParamLoad<T, E> wp[kParamAhead ? V : 1];
    if constexpr (kParamAhead) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            wp[k].issue(w, k * L + li, sp.h, N, false);
    } else if constexpr (!PH) {
        wl.issue(w, li, nv, rs, 0.0f, slots_full);
    }
    float wv[V][E];

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row_of(r);
        const bool row_ok = kSame || row < M;
        const int64_t rr = row_ok ? row : 0;
        const int vend = row_ok ? nv : 0;
        const bool store_full = EXACT || (row_ok && slots_full);

        float v[V][E];
        if constexpr (PH)
            xs.finish(v, sp, jend, 0.0f, false);
        else
            xl.finish(v, rs);
        if constexpr (RES) {
            float u[V][E];
            if constexpr (PH)
                rsl.finish(u, sp, jend, 0.0f, false);
            else
                rl.finish(u, rs);
            add_rounded<T>(v, u);
        }
        if (r + 1 < R)
            issue_row(r + 1);
        if constexpr (RES) {
            if constexpr (PH)
                store_span<T, E, V, L>(ro + rr * ldo - sp.h, li, jend, sp, v, false);
            else if (!EXACT || row_ok)
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

        if constexpr (kParamAhead) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                wp[k].finish(wv[k], k * L + li, sp.h, N, false);
        } else if constexpr (PH) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                load_param<T, E>(w, k * L + li, sp.h, N, wv[k], false);
        } else if (r == 0) {
            wl.finish(wv, rs);
        }
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[k][e] = v[k][e] * inv * wv[k][e];
        if constexpr (kSame)
            if (r + 1 < R)
                wait_vmem();
        if constexpr (PH)
            store_span<T, E, V, L>(y + rr * ldy - sp.h, li, jend, sp, v, false);
        else if (!EXACT || row_ok)
            store_row<T, E, V, L>(y + rr * ldy, li, vend, rs, v, store_full);
    }
}

template <typename T, int G, int V, int W, int R, bool EXACT, bool RES, bool PH>
static hipError_t rmsnorm_tile_run(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG * R - 1) / (RG * R);
    const float inv_n = static_cast<float>(1.0 / p.N);
    return launch(rmsnorm_tile<T, G, V, W, R, EXACT, RES, PH>,
                  dim3(static_cast<unsigned>(blocks)),
                  dim3(W * kWave), p.stream, static_cast<const T *>(p.x),
                  static_cast<const T *>(p.r), static_cast<const T *>(p.w),
                  static_cast<T *>(p.y), static_cast<T *>(p.ro), p.M, p.N, p.ldx, p.ldr, p.ldy,
                  p.ldo, inv_n, p.eps);
}

// The phased form of a general one-row-per-group tile (null for others).
template <typename T, bool RES, int G, int V, int W, int R, bool EXACT>
constexpr hipError_t (*phased_run())(const RowProblem &)
{
    if constexpr (!EXACT && R == 1)
        return &rmsnorm_tile_run<T, G, V, W, 1, false, RES, true>;
    else
        return nullptr;
}

template <typename T, bool RES, int G, int V, int W, int R = 1, bool EXACT = false>
constexpr TileVariant tile()
{
    return TileVariant{G, V, W, R, G * V * kWave * Elem<T>::kVec, EXACT,
                       &rmsnorm_tile_run<T, G, V, W, R, EXACT, RES, false>, false,
                       phased_run<T, RES, G, V, W, R, EXACT>()};
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

// Row v = x (or x + residual, rounded) for U vectors per thread: the loads
// of one step, in flight together (x, and the residual with RES).
template <typename T, int E, int U, int NT, int CP, bool RES>
struct RmsStep {
    SpanLoad<T, E, U, NT, CP> xl, rl;

    __device__ __forceinline__ void issue(const T *__restrict__ xb, const T *__restrict__ rb,
                                          int j0, int jend, bool full)
    {
        xl.issue(xb, j0, jend, full);
        if constexpr (RES)
            rl.issue(rb, j0, jend, full);
    }

    __device__ __forceinline__ void finish(float (&v)[U][E], RowSpan<E> sp, int jend,
                                           bool full) const
    {
        xl.finish(v, sp, jend, 0.0f, full);
        if constexpr (RES) {
            float u[U][E];
            rl.finish(u, sp, jend, 0.0f, full);
            add_rounded<T>(v, u);  // padding stays 0
        }
    }
};

// This thread's part of the sum of v^2 over vectors [jbeg, jend) of a row
// (bases xb, rb at the row's phase), software-pipelined, cached loads: the
// output pass reads the row again.
template <typename T, int E, int W, int U, bool RES>
__device__ __forceinline__ float rms_scan(const T *__restrict__ xb, const T *__restrict__ rb,
                                          RowSpan<E> sp, int jbeg, int jend)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    float q = 0.0f;
    RmsStep<T, E, U, NT, kCached, RES> cur;
    cur.issue(xb, rb, jbeg + tid, jend, full(jbeg));
    for (int base = jbeg; base < jend; base += NT * U) {
        RmsStep<T, E, U, NT, kCached, RES> nxt;
        const int next = base + NT * U;
        if (next < jend)
            nxt.issue(xb, rb, next + tid, jend, full(next));
        float v[U][E];
        cur.finish(v, sp, jend, full(base));
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                q = fmaf(v[u][e], v[u][e], q);
        cur = nxt;
    }
    return q;
}

// The loads of the first step rms_write runs (the range's last), issued by
// the caller ahead of the reduction that forms inv, so that they are in
// flight meanwhile.
template <typename T, int E, int W, int U, bool RES>
__device__ __forceinline__ RmsStep<T, E, U, W * kWave, kStreaming, RES>
rms_write_first(const T *__restrict__ xb, const T *__restrict__ rb, RowSpan<E> sp, int jbeg,
                int jend)
{
    constexpr int NT = W * kWave;
    const int base = last_step(jbeg, jend, NT * U);
    RmsStep<T, E, U, NT, kStreaming, RES> cur;
    cur.issue(xb, rb, base + static_cast<int>(threadIdx.x % NT), jend > jbeg ? jend : base,
              sp.step_full(base, jend, NT * U));
    return cur;
}

// Store residual_out (RES) and y = v inv w for vectors [jbeg, jend) of a row,
// last step first; that step's loads come issued (rms_write_first).
template <typename T, int E, int W, int U, bool RES>
__device__ __forceinline__ void rms_write(const T *__restrict__ xb, const T *__restrict__ rb,
                                          const T *__restrict__ w, T *yb, T *ob, RowSpan<E> sp,
                                          int jbeg, int jend, float inv,
                                          RmsStep<T, E, U, W * kWave, kStreaming, RES> cur)
{
    constexpr int NT = W * kWave;
    const int tid = static_cast<int>(threadIdx.x % NT);
    auto full = [&](int base) { return sp.step_full(base, jend, NT * U); };
    for (int base = last_step(jbeg, jend, NT * U); base >= jbeg; base -= NT * U) {
        const bool f = full(base);
        // the weight, the next step's row and this step's row are all in
        // flight before the first wait
        ParamLoad<T, E> wl[U];
#pragma unroll
        for (int u = 0; u < U; ++u)
            wl[u].issue(w, base + tid + u * NT, sp.h, sp.n, f);
        RmsStep<T, E, U, NT, kStreaming, RES> nxt;
        const int next = base - NT * U;
        if (next >= jbeg)
            nxt.issue(xb, rb, next + tid, jend, full(next));
        float v[U][E], wv[U][E];
        cur.finish(v, sp, jend, f);
#pragma unroll
        for (int u = 0; u < U; ++u)
            wl[u].finish(wv[u], base + tid + u * NT, sp.h, sp.n, f);
        if constexpr (RES)
            store_span<T, E, U, NT>(ob, base + tid, jend, sp, v, f);
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[u][e] = v[u][e] * inv * wv[u][e];
        store_span<T, E, U, NT>(yb, base + tid, jend, sp, v, f);
        cur = nxt;
    }
}

// Sum of the W waves' parts (wave DPP, then LDS across waves).
template <int W>
__device__ __forceinline__ float rms_block_sum(float q, float *red)
{
    q = wave_sum(q);
    if constexpr (W > 1) {
        if (threadIdx.x % kWave == 0)
            red[threadIdx.x / kWave] = q;
        __syncthreads();
        q = red[0];
#pragma unroll
        for (int i = 1; i < W; ++i)
            q += red[i];
    }
    return q;
}

// One row per W waves, RB rows per workgroup (several only for W == 1,
// where no barrier is taken).  Pass 1 (cached loads) sums v^2; pass 2
// re-reads the row, stores residual_out (RES) and y = v inv w.  Rows are
// read as aligned vectors from their own phase (RowSpan): x, residual, y and
// residual_out share it, the weight is shifted into it.
template <typename T, int E, int W, int U, bool RES, int RB, bool PH>
__global__ __launch_bounds__(W *kWave *RB) void rmsnorm_loop(
    const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w,
    T *__restrict__ y, T *__restrict__ ro, int64_t M, int N, int64_t ldx, int64_t ldr,
    int64_t ldy, int64_t ldo, float inv_n, float eps)
{
    static_assert(RB == 1 || W == 1, "several rows per workgroup only with one wave each");
    __shared__ float red[W];
    const int64_t row = static_cast<int64_t>(blockIdx.x) * RB + threadIdx.x / (W * kWave);
    if (RB > 1 && row >= M)
        return;
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    const T *rb = RES ? res + row * ldr - sp.h : nullptr;
    const int nv = sp.count();
    float q = rms_scan<T, E, W, U, RES>(xb, rb, sp, 0, nv);
    const auto first = rms_write_first<T, E, W, U, RES>(xb, rb, sp, 0, nv);
    q = rms_block_sum<W>(q, red);
    const float inv = __builtin_amdgcn_rsqf(fmaf(q, inv_n, eps));
    rms_write<T, E, W, U, RES>(xb, rb, w, y + row * ldy - sp.h,
                               RES ? ro + row * ldo - sp.h : nullptr, sp, 0, nv, inv, first);
}

// Split rows, first kernel: workgroup (row, chunk) writes the chunk's sum of
// v^2 (as the first float of its partial).
template <typename T, int E, int W, int U, bool RES, bool PH>
__global__ __launch_bounds__(W *kWave) void rmsnorm_partials(const T *__restrict__ x,
                                                             const T *__restrict__ res, int N,
                                                             int64_t ldx, int64_t ldr, int S,
                                                             int C, char *pbase, int64_t prow)
{
    __shared__ float red[W];
    const int64_t row = blockIdx.x / S;
    const int s = static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    float q = rms_scan<T, E, W, U, RES>(xr - sp.h, RES ? res + row * ldr - sp.h : nullptr, sp,
                                        jbeg, jend);
    q = rms_block_sum<W>(q, red);
    if (threadIdx.x == 0)
        row_partials(pbase, prow, row)[s] = make_float2(q, 0.0f);
}

// Split rows, second kernel: chunk s of row r, workgroup (r, s) of a grid of
// M S (kAllChunks, kAllButFirst) or workgroup r of a grid of M, s = 0
// (kFirstOnly), over the range output_range gives.  Every wave sums the row's
// S partials on its own (lane l takes l, l + 64, ..., then DPP), so every
// workgroup of the row forms the same bits.  y and pbase may name the same
// memory (the partials kept in the output).
template <typename T, int E, int W, int U, bool RES, bool PH>
__global__ __launch_bounds__(W *kWave) void rmsnorm_finish(
    const T *__restrict__ x, const T *__restrict__ res, const T *__restrict__ w, T *y, T *ro,
    int N, int64_t ldx, int64_t ldr, int64_t ldy, int64_t ldo, int S, int C, float inv_n,
    float eps, const char *pbase, int64_t prow, int part)
{
    const int64_t row = part == kFirstOnly ? blockIdx.x : blockIdx.x / S;
    const int s = part == kFirstOnly ? 0 : static_cast<int>(blockIdx.x % S);
    const T *xr = x + row * ldx;
    const RowSpan<E> sp{row_phase<T, E, PH>(xr), N};
    const T *xb = xr - sp.h;
    const T *rb = RES ? res + row * ldr - sp.h : nullptr;
    int jbeg, jend;
    chunk_span<E>(sp, s, S, C, jbeg, jend);
    output_range<T, E>(part, s, y + row * ldy, sp, S, jbeg, jend);
    const auto first = rms_write_first<T, E, W, U, RES>(xb, rb, sp, jbeg, jend);
    float q = 0.0f;
    const float2 *pr = row_partials(pbase, prow, row);
    for (int i = static_cast<int>(threadIdx.x % kWave); i < S; i += kWave)
        q += pr[i].x;
    q = wave_sum(q);
    const float inv = __builtin_amdgcn_rsqf(fmaf(q, inv_n, eps));
    // the partials in the output are overwritten below: every wave has read
    // them first
    if (part == kFirstOnly)
        __syncthreads();
    rms_write<T, E, W, U, RES>(xb, rb, w, y + row * ldy - sp.h,
                               RES ? ro + row * ldo - sp.h : nullptr, sp, jbeg, jend, inv, first);
}

namespace {

// Vectors per thread per step: 64 bytes of row (two bf16 vectors), as in
// the LayerNorm streaming kernel.
constexpr int loop_vectors(int E) { return E == 8 ? 2 : 4; }

template <typename T, int E, bool RES, bool PH, int W, int U = loop_vectors(E)>
hipError_t loop_launch(const RowProblem &p)
{
    constexpr int RB = W == 1 ? 4 : 1;  // one-wave rows go four to a workgroup
    return launch(rmsnorm_loop<T, E, W, U, RES, RB, PH>,
                  dim3(static_cast<unsigned>((p.M + RB - 1) / RB)), dim3(W * kWave * RB),
                  p.stream, static_cast<const T *>(p.x), static_cast<const T *>(p.r),
                  static_cast<const T *>(p.w), static_cast<T *>(p.y), static_cast<T *>(p.ro),
                  p.M, p.N, p.ldx, p.ldr, p.ldy, p.ldo, static_cast<float>(1.0 / p.N), p.eps);
}

// 1, 4 or 16 waves per row by the row's length.
template <typename T, int E, bool RES, bool PH>
hipError_t loop_run(const RowProblem &p)
{
    const int64_t nvec = (p.N + 2 * E - 2) / E;
    if (nvec <= kShortRowVectors)
        return loop_launch<T, E, RES, PH, 1, 1>(p);
    switch (stream_waves(nvec, loop_vectors(E))) {
    case 16:
        return loop_launch<T, E, RES, PH, 16>(p);
    case 4:
        return loop_launch<T, E, RES, PH, 4>(p);
    default:
        return loop_launch<T, E, RES, PH, 1>(p);
    }
}

template <typename T, bool RES>
hipError_t loop_io(const RowProblem &p, RowIo io)
{
    constexpr int E = Elem<T>::kVec;
    if (io == kIoAligned)
        return loop_run<T, E, RES, false>(p);
    if (io == kIoPhased)
        return loop_run<T, E, RES, true>(p);
    return loop_run<T, 1, RES, false>(p);
}

template <bool RES>
hipError_t loop_dispatch(const RowProblem &p, RowIo io)
{
    return p.dtype == RK_F32 ? loop_io<float, RES>(p, io) : loop_io<bf16_t, RES>(p, io);
}

constexpr int kSplitW = 4;  // 256 threads per chunk

template <typename T, int E, bool RES, bool PH>
hipError_t split_run(const RowProblem &p, int S, int C, SplitPartials pt)
{
    constexpr int U = E == 1 ? 4 : loop_vectors(E);
    const dim3 grid(static_cast<unsigned>(p.M * S));
    const dim3 block(kSplitW * kWave);
    const T *x = static_cast<const T *>(p.x);
    const T *r = static_cast<const T *>(p.r);
    hipError_t err = launch(rmsnorm_partials<T, E, kSplitW, U, RES, PH>, grid, block, p.stream, x,
                            r, p.N, p.ldx, p.ldr, S, C, pt.base, pt.row_bytes);
    if (err != hipSuccess)
        return err;
    auto kernel = rmsnorm_finish<T, E, kSplitW, U, RES, PH>;
    const T *w = static_cast<const T *>(p.w);
    T *y = static_cast<T *>(p.y);
    T *ro = static_cast<T *>(p.ro);
    const float inv_n = static_cast<float>(1.0 / p.N);
    if (!pt.in_output)
        return launch(kernel, grid, block, p.stream, x, r, w, y, ro, p.N, p.ldx, p.ldr, p.ldy,
                      p.ldo, S, C, inv_n, p.eps, pt.base, pt.row_bytes, int{kAllChunks});
    err = launch(kernel, grid, block, p.stream, x, r, w, y, ro, p.N, p.ldx, p.ldr, p.ldy, p.ldo, S,
                 C, inv_n, p.eps, pt.base, pt.row_bytes, int{kAllButFirst});
    if (err != hipSuccess)
        return err;
    return launch(kernel, dim3(static_cast<unsigned>(p.M)), block, p.stream, x, r, w, y, ro, p.N,
                  p.ldx, p.ldr, p.ldy, p.ldo, S, C, inv_n, p.eps, pt.base, pt.row_bytes,
                  int{kFirstOnly});
}

template <typename T, bool RES>
hipError_t split_io(const RowProblem &p, int S, int C, SplitPartials pt, RowIo io)
{
    constexpr int E = Elem<T>::kVec;
    if (io == kIoAligned)
        return split_run<T, E, RES, false>(p, S, C, pt);
    if (io == kIoPhased)
        return split_run<T, E, RES, true>(p, S, C, pt);
    return split_run<T, 1, RES, false>(p, S, C, pt);
}

template <bool RES>
hipError_t split_dispatch(const RowProblem &p, int S, int C, SplitPartials pt, RowIo io)
{
    return p.dtype == RK_F32 ? split_io<float, RES>(p, S, C, pt, io)
                             : split_io<bf16_t, RES>(p, S, C, pt, io);
}

}  // namespace

hipError_t rmsnorm_loop_run(const RowProblem &p, bool residual, RowIo io)
{
    return residual ? loop_dispatch<true>(p, io) : loop_dispatch<false>(p, io);
}

hipError_t rmsnorm_split_run(const RowProblem &p, bool residual, int splits, int chunk,
                             SplitPartials parts, RowIo io)
{
    return residual ? split_dispatch<true>(p, splits, chunk, parts, io)
                    : split_dispatch<false>(p, splits, chunk, parts, io);
}

}  // namespace rk
