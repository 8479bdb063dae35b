// Fused LayerNorm + affine + GeLU ("Triton Kernel 实现练习" §4.1 "LayerNorm"
// and §3.4 "Approx Activation"; "PyTorch 自定义 CUDA 算子与 Triton 编程从 Python
// 原型到 GPU 极致性能" section 三, "Fused LayerNorm GELU Kernel").
//
// Per row: mu = sum x / N; var = sum (x - mu)^2 / N, both over the N true
// columns (padding never enters); rstd = 1 / sqrt(var + eps);
// z = (x - mu) rstd w + b; y = GeLU(z), the tanh approximation (GK = 0) or the
// exact erf form (GK = 1); or y = z (GK = 2: the LayerNorm of §4.1 alone).
//
// layernorm_gelu_tile  the row stays in VGPRs (one HBM read and write per
//                      element): sum -> wave DPP / LDS -> centre in registers
//                      -> sum of squares -> wave DPP / LDS -> epilogue.  A row
//                      group handles R rows in sequence and loads weight and
//                      bias once for all of them.  The exact bf16 tiles take
//                      both sums of x - x[0] in one pass and one DPP / LDS
//                      round (SH below).
// Rows beyond the register capacity, or not 16-byte aligned, go to the
// streaming and split-row kernels of rk_layernorm_long.hip.
#include <atomic>

#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

// EXACT: compiled for N == V * L * E, i.e. every register slot of a row group
// is a column of its row: no masks, no padding, no excluded columns.  Rows
// past M (the last workgroup) then read row 0 and store nothing.
// PH: rows at any offset past a 16-byte boundary (the output's rows at the
// same offset), read and written as the aligned vectors that cover them
// (RowSpan), their ends masked; weight and bias are shifted into each row's
// offset as they are used.  One row per row group.
// SH (EXACT, not PH): one pass over the registers for both sums, of
// d = x - K with K the row's first element: mean = K + sum d / N and
// var = sum d^2 / N - (sum d / N)^2, so both reductions share one barrier.
template <typename T, int G, int V, int W, int R, bool EXACT, int GK, bool PH, bool SH = false>
__global__ __launch_bounds__(W *kWave)
__attribute__((amdgpu_waves_per_eu(SH && EXACT && G == 4 && V == 2 && R == 2 ? 7 : 1)))
void layernorm_gelu_tile(
    const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b,
    T *__restrict__ y, int64_t M, int N, int64_t ldx, int64_t ldy, float inv_n, float eps)
{
    static_assert(!PH || (!EXACT && R == 1), "phased rows: general tiles, one row per group");
    static_assert(!SH || !PH, "one shifted pass: rows at 16-byte boundaries");
    constexpr int E = Elem<T>::kVec;
    constexpr int RG = W / G;
    constexpr int L = G * kWave;
    static_assert(W % G == 0, "whole row groups per workgroup");
    // two buffers per reduction: a wave may start the next row's reduction
    // while another still reads this row's partials
    __shared__ float red_sum[2][RG][G];
    __shared__ float red_var[2][RG][G];
    // SH: the (sum, sum of squares) of every 16-lane row of the group's waves
    constexpr int P = 4 * G;
    __shared__ f32x2_t red_sq[2][RG][SH && G <= 8 ? P : 1];

    // wave-uniform: row bases stay in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    const int grp = wave / G;
    const int wig = wave % G;
    const int li = wig * kWave + static_cast<int>(threadIdx.x % kWave);
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    // every vector slot of a row group holds a complete vector of the row
    const bool slots_full = EXACT || V * L <= rs.nfull;

    // kSame (a tile of one row group and two rows): a second
    // row past M is the first row again.  It is read before the first row's
    // stores and written twice with the same bytes (in place too), so every
    // store is unconditional, and the second row's loads can be awaited just
    // before the first row's stores (wait_vmem) without also waiting for
    // those stores, which a branch around them would make the compiler do.
    constexpr bool kSame = !PH && R == 2 && RG == 1;
    // Row r of this row group.
    auto row_of = [&](int r) {
        const int64_t i = (static_cast<int64_t>(blockIdx.x) * R + r) * RG + grp;
        return kSame && i >= M ? M - 1 : i;
    };

    // Loads in flight before any is waited for: the first row, then weight
    // and bias (shared by all R rows).  Each later row is issued while the
    // previous one is reduced.
    RowLoad<T, E, V, L> xl;
    SpanLoad<T, E, V, L> xs;  // PH
    // PH: the weight and bias blocks of tiles of up to three vectors per lane
    // are loaded with the row (two blocks each per vector); larger tiles load
    // them as they are used (measured: loading them early there costs more in
    // registers than it saves in latency)
    constexpr bool kParamAhead = PH && V <= 3;
    ParamLoad<T, E> wp[kParamAhead ? V : 1], bp[kParamAhead ? V : 1];
    RowSpan<E> sp{0, N};
    int jend = 0;
    if constexpr (PH) {
        const int64_t row = row_of(0);
        const bool ok = row < M;
        const T *xr = x + (ok ? row : 0) * ldx;
        sp.h = row_phase<T, E>(xr);
        jend = ok ? sp.count() : 0;
        xs.issue(xr - sp.h, li, jend, false);
        if constexpr (kParamAhead) {
#pragma unroll
            for (int k = 0; k < V; ++k) {
                wp[k].issue(w, k * L + li, sp.h, N, false);
                bp[k].issue(b, k * L + li, sp.h, N, false);
            }
        }
    } else {
        const int64_t row = row_of(0);
        const bool ok = row < M;
        xl.issue(x + (ok ? row : 0) * ldx, li, ok ? nv : 0, rs, 0.0f,
                 EXACT || (ok && slots_full));
    }
    // SH: the shift of the row being issued, loaded with it
    float k_next = SH ? Elem<T>::to_f32(x[(row_of(0) < M ? row_of(0) : 0) * ldx]) : 0.0f;
    RowLoad<T, E, V, L, kCached> wl, bl;
    if constexpr (!PH) {
        wl.issue(w, li, nv, rs, 0.0f, slots_full);
        bl.issue(b, li, nv, rs, 0.0f, slots_full);
    }
    float wv[R > 1 ? V : 1][E], bv[R > 1 ? V : 1][E];

#pragma unroll
    for (int r = 0; r < R; ++r) {
        const int64_t row = row_of(r);
        const bool row_ok = kSame || row < M;
        const int64_t rr = row_ok ? row : 0;
        const T *xr = x + rr * ldx;
        T *yr = y + rr * ldy;
        const int vend = row_ok ? nv : 0;
        const int buf = r & 1;

        float v[V][E];
        if constexpr (PH)
            xs.finish(v, sp, jend, 0.0f, false);
        else
            xl.finish(v, rs);
        const float K = k_next;
        if (r + 1 < R) {
            const int64_t nrow = row_of(r + 1);
            const bool nok = kSame || nrow < M;
            xl.issue(x + (nok ? nrow : 0) * ldx, li, nok ? nv : 0, rs, 0.0f,
                     EXACT || (nok && slots_full));
            if constexpr (SH)
                k_next = Elem<T>::to_f32(x[(nok ? nrow : 0) * ldx]);
        }

        // z = fma(fma(v, rstd, cen), w, b) once the statistics are known
        float rstd, cen = 0.0f;
        if constexpr (SH) {
            // the sums start from the first element (no add to a zero); a
            // padded slot of a general tile adds d = 0 to both
            float s = 0.0f, q = 0.0f;
#pragma unroll
            for (int k = 0; k < V; ++k) {
                const int vi = k * L + li;
#pragma unroll
                for (int e = 0; e < E; ++e) {
                    const bool valid =
                        EXACT || vi < rs.nfull || (vi == rs.nfull && e < rs.tail);
                    const float d = valid ? v[k][e] - K : 0.0f;
                    v[k][e] = d;
                    s = k == 0 && e == 0 ? d : s + d;
                    q = k == 0 && e == 0 ? d * d : fmaf(d, d, q);
                }
            }
            if constexpr (G > 1 && G <= 8) {
                // Sum each 16-lane row, publish the 4 G row sums, and let
                // every 16-lane row of the group add all of them in the same
                // order: no cross-row step within the wave, one LDS round
                // (16 waves: 64 partials, slower than the wave sums below).
                const int lane = static_cast<int>(threadIdx.x % kWave);
                s = group_reduce<16>(s, SumOp());
                q = group_reduce<16>(q, SumOp());
                if (lane % 16 == 0)
                    red_sq[buf][grp][4 * wig + lane / 16] = f32x2_t{s, q};
                __syncthreads();
                const f32x2_t *part = red_sq[buf][grp];
                constexpr int PL = P < 16 ? P : 16;  // lanes that share the partials
                f32x2_t t = part[lane % PL];
#pragma unroll
                for (int j = 1; j < P / 16; ++j)
                    t += part[lane % 16 + 16 * j];
                s = group_reduce<PL>(t[0], SumOp());
                q = group_reduce<PL>(t[1], SumOp());
            } else {
                s = wave_sum(s);
                q = wave_sum(q);
                if constexpr (G > 1) {
                    if (threadIdx.x % kWave == 0) {
                        red_sum[buf][grp][wig] = s;
                        red_var[buf][grp][wig] = q;
                    }
                    __syncthreads();
                    s = red_sum[buf][grp][0];
                    q = red_var[buf][grp][0];
#pragma unroll
                    for (int g = 1; g < G; ++g) {
                        s += red_sum[buf][grp][g];
                        q += red_var[buf][grp][g];
                    }
                }
            }
            const float mean_k = s * inv_n;
            const float var = fmaxf(fmaf(q, inv_n, -mean_k * mean_k), 0.0f);
            rstd = __builtin_amdgcn_rsqf(var + eps);
            cen = -mean_k * rstd;
        } else {
        float s = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                s += v[k][e];
        s = wave_sum(s);
        if constexpr (G > 1) {
            if (threadIdx.x % kWave == 0)
                red_sum[buf][grp][wig] = s;
            __syncthreads();
            s = red_sum[buf][grp][0];
#pragma unroll
            for (int g = 1; g < G; ++g)
                s += red_sum[buf][grp][g];
        }
        const float mean = s * inv_n;

        // centre in registers; padded columns are set to 0 so that they add
        // nothing to the variance
        float q = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int vi = k * L + li;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const bool valid =
                    PH ? vi < jend && sp.valid(vi, e)
                       : EXACT || vi < rs.nfull || (vi == rs.nfull && e < rs.tail);
                const float d = valid ? v[k][e] - mean : 0.0f;
                v[k][e] = d;
                q = fmaf(d, d, q);
            }
        }
        q = wave_sum(q);
        if constexpr (G > 1) {
            if (threadIdx.x % kWave == 0)
                red_var[buf][grp][wig] = q;
            __syncthreads();
            q = red_var[buf][grp][0];
#pragma unroll
            for (int g = 1; g < G; ++g)
                q += red_var[buf][grp][g];
        }
        // hardware reciprocal square root (1 ulp), once per row
        rstd = __builtin_amdgcn_rsqf(fmaf(q, inv_n, eps));
        }

        if constexpr (R > 1) {
            // weight and bias serve R rows: unpack them once
            if (r == 0) {
                wl.finish(wv, rs);
                bl.finish(bv, rs);
            }
#pragma unroll
            for (int k = 0; k < V; ++k)
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[k][e] = gelu<GK>(fmaf(SH ? fmaf(v[k][e], rstd, cen) : v[k][e] * rstd,
                                            wv[k][e], bv[k][e]));
        } else {
            // one row: unpack weight and bias a vector at a time, so that they
            // stay packed (half the registers for bf16) until used
#pragma unroll
            for (int k = 0; k < V; ++k) {
                float wk[E], bk[E];
                if constexpr (kParamAhead) {
                    wp[k].finish(wk, k * L + li, sp.h, N, false);
                    bp[k].finish(bk, k * L + li, sp.h, N, false);
                } else if constexpr (PH) {
                    load_param<T, E>(w, k * L + li, sp.h, N, wk, false);
                    load_param<T, E>(b, k * L + li, sp.h, N, bk, false);
                } else {
                    wl.finish_one(k, wk, rs);
                    bl.finish_one(k, bk, rs);
                }
#pragma unroll
                for (int e = 0; e < E; ++e)
                    v[k][e] = gelu<GK>(fmaf(SH ? fmaf(v[k][e], rstd, cen) : v[k][e] * rstd,
                                            wk[e], bk[e]));
            }
        }
        if constexpr (PH) {
            store_span<T, E, V, L>(yr - sp.h, li, jend, sp, v, false);
        } else if (EXACT) {
            if constexpr (kSame)
                if (r + 1 < R)
                    wait_vmem();
            if (row_ok)
                store_row<T, E, V, L>(yr, li, vend, rs, v, true);
        } else {
            if constexpr (kSame)
                if (r + 1 < R)
                    wait_vmem();
            store_row<T, E, V, L>(yr, li, vend, rs, v, row_ok && slots_full);
        }
    }
}

// The exact one-pass (SH) tile as a persistent grid: as many workgroups as
// are resident at once, each taking rows blockIdx.x, blockIdx.x + gridDim.x,
// ... in a loop with the next row's loads in flight.  Weight and bias are
// loaded and unpacked once per workgroup, and the grid ends in one round
// instead of a partly filled last one.  One row per workgroup (G = W): every
// row the loop visits exists, so the loads and stores need no branch, and the
// compiler can count the loads in flight exactly (a branch around them makes
// it wait for all of them, the next row's included).
template <typename T, int G, int V, int W, int GK>
__global__ __launch_bounds__(W *kWave) void layernorm_gelu_rows(
    const T *__restrict__ x, const T *__restrict__ w, const T *__restrict__ b,
    T *__restrict__ y, int64_t M, int N, int64_t ldx, int64_t ldy, float inv_n, float eps)
{
    constexpr int E = Elem<T>::kVec;
    constexpr int L = G * kWave;
    constexpr int P = 4 * G;  // 16-lane partial sums per row
    constexpr int PL = P < 16 ? P : 16;
    static_assert(W == G && G > 1, "one row of several waves per workgroup");
    // two buffers: a wave may publish the next row's partials while another
    // still reads this row's
    __shared__ f32x2_t red_sq[2][P];

    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x / kWave));
    __builtin_assume(wave >= 0 && wave < W);  // lane offsets are 32-bit and non-negative
    const int lane = static_cast<int>(threadIdx.x % kWave);
    const int li = wave * kWave + lane;
    const RowSplit<E> rs(N);
    const int nv = rs.count();
    const int64_t step = gridDim.x;
    const int64_t first = blockIdx.x;

    // Two load buffers used in turn (the loop is unrolled by two), so that
    // no register copy waits on the loads; the shift is carried as its raw
    // 16 bits and converted where it is used.
    RowLoad<T, E, V, L> xa, xb;
    T ka, kb;
    int64_t row = first;  // < M: the grid has no more workgroups than rows
    xa.issue(x + row * ldx, li, nv, rs, 0.0f, true);
    ka = x[row * ldx];
    float wv[V][E], bv[V][E];
    {
        RowLoad<T, E, V, L, kCached> wl, bl;
        wl.issue(w, li, nv, rs, 0.0f, true);
        bl.issue(b, li, nv, rs, 0.0f, true);
        wl.finish(wv, rs);
        bl.finish(bv, rs);
    }
    // the first row is needed at once; with no loads in flight on entry the
    // loop's own waits count only its loads
    wait_vmem();

    // One row: finish cur, issue the next row into nxt, normalize, store.
    auto one_row = [&](RowLoad<T, E, V, L> &cur, const T &kc, RowLoad<T, E, V, L> &nxt, T &kn,
                       int buf) {
        float v[V][E];
        cur.finish(v, rs);
        const float K = Elem<T>::to_f32(kc);
        // the next row, or after the last one the weight row (L2-resident,
        // never used): an unconditional load keeps the counts exact
        const int64_t nrow = row + step;
        const T *src = nrow < M ? x + nrow * ldx : w;
        nxt.issue(src, li, nv, rs, 0.0f, true);
        kn = src[0];

        float s = 0.0f, q = 0.0f;
#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e) {
                const float d = v[k][e] - K;
                v[k][e] = d;
                s = k == 0 && e == 0 ? d : s + d;
                q = k == 0 && e == 0 ? d * d : fmaf(d, d, q);
            }
        s = group_reduce<16>(s, SumOp());
        q = group_reduce<16>(q, SumOp());
        if (lane % 16 == 0)
            red_sq[buf][4 * wave + lane / 16] = f32x2_t{s, q};
        __syncthreads();
        f32x2_t t = red_sq[buf][lane % PL];
#pragma unroll
        for (int j = 1; j < P / 16; ++j)
            t += red_sq[buf][lane % 16 + 16 * j];
        s = group_reduce<PL>(t[0], SumOp());
        q = group_reduce<PL>(t[1], SumOp());
        const float mean_k = s * inv_n;
        const float var = fmaxf(fmaf(q, inv_n, -mean_k * mean_k), 0.0f);
        const float rstd = __builtin_amdgcn_rsqf(var + eps);
        const float cen = -mean_k * rstd;

#pragma unroll
        for (int k = 0; k < V; ++k)
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[k][e] = gelu<GK>(fmaf(fmaf(v[k][e], rstd, cen), wv[k][e], bv[k][e]));
        wait_vmem();  // the next row's loads (and the previous row's stores)
        store_row<T, E, V, L>(y + row * ldy, li, nv, rs, v, true);
        row = nrow;
    };

    for (;;) {
        one_row(xa, ka, xb, kb, 0);
        if (row >= M)
            break;
        one_row(xb, kb, xa, ka, 1);
        if (row >= M)
            break;
    }
}

// Workgroups of the persistent kernel: at most as many as the device holds at
// once (per device, from the occupancy calculator), and no more than needed
// for every workgroup to take the same number of rows, give or take one.
template <typename T, int G, int V, int W>
static hipError_t layernorm_gelu_rows_run(const RowProblem &p)
{
    constexpr int kDevices = 64;
    static std::atomic<int> resident[3][kDevices];
    const int gk = p.gelu == RK_GELU_ERF ? 1 : (p.gelu == RK_GELU_NONE ? 2 : 0);
    auto kernel = gk == 1   ? layernorm_gelu_rows<T, G, V, W, 1>
                  : gk == 2 ? layernorm_gelu_rows<T, G, V, W, 2>
                            : layernorm_gelu_rows<T, G, V, W, 0>;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    int n = dev < kDevices ? resident[gk][dev].load(std::memory_order_relaxed) : 0;
    if (n == 0) {
        int per_cu = 0, cus = 0;
        e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void *>(kernel),
                                                         W * kWave, 0);
        if (e != hipSuccess)
            return e;
        e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
        if (e != hipSuccess)
            return e;
        n = per_cu * cus > 0 ? per_cu * cus : 1;
        if (dev < kDevices)
            resident[gk][dev].store(n, std::memory_order_relaxed);
    }
    const int64_t groups = p.M;
    const int64_t iters = (groups + n - 1) / n;
    const int64_t blocks = iters > 0 ? (groups + iters - 1) / iters : 0;
    const float inv_n = static_cast<float>(1.0 / p.N);
    return launch(kernel, dim3(static_cast<unsigned>(blocks)), dim3(W * kWave), p.stream,
                  static_cast<const T *>(p.x), static_cast<const T *>(p.w),
                  static_cast<const T *>(p.b), static_cast<T *>(p.y), p.M, p.N, p.ldx, p.ldy,
                  inv_n, p.eps);
}

template <typename T, int G, int V, int W, int R, bool EXACT, bool PH, bool SH = false>
static hipError_t layernorm_gelu_tile_run(const RowProblem &p)
{
    constexpr int RG = W / G;
    const int64_t blocks = (p.M + RG * R - 1) / (RG * R);
    const float inv_n = static_cast<float>(1.0 / p.N);
    auto kernel = p.gelu == RK_GELU_ERF    ? layernorm_gelu_tile<T, G, V, W, R, EXACT, 1, PH, SH>
                  : p.gelu == RK_GELU_NONE ? layernorm_gelu_tile<T, G, V, W, R, EXACT, 2, PH, SH>
                                           : layernorm_gelu_tile<T, G, V, W, R, EXACT, 0, PH, SH>;
    return launch(kernel, dim3(static_cast<unsigned>(blocks)), dim3(W * kWave), p.stream,
                  static_cast<const T *>(p.x), static_cast<const T *>(p.w),
                  static_cast<const T *>(p.b), static_cast<T *>(p.y), p.M, p.N, p.ldx, p.ldy,
                  inv_n, p.eps);
}

// The phased form of a general one-row-per-group tile (null for others).
template <typename T, int G, int V, int W, int R, bool EXACT>
constexpr hipError_t (*phased_run())(const RowProblem &)
{
    if constexpr (!EXACT && R == 1)
        return &layernorm_gelu_tile_run<T, G, V, W, 1, false, true>;
    else
        return nullptr;
}

template <typename T, int G, int V, int W, int R = 1, bool EXACT = false>
constexpr TileVariant tile()
{
    return TileVariant{G, V, W, R, G * V * kWave * Elem<T>::kVec, EXACT,
                       &layernorm_gelu_tile_run<T, G, V, W, R, EXACT, false>, false,
                       phased_run<T, G, V, W, R, EXACT>()};
}
template <typename T, int G, int V, int W, int R = 1>
constexpr TileVariant exact()
{
    return tile<T, G, V, W, R, true>();
}
// An exact tile with the one shifted pass (SH).
template <typename T, int G, int V, int W, int R = 1>
constexpr TileVariant exact_shifted()
{
    return TileVariant{G, V, W, R, G * V * kWave * Elem<T>::kVec, true,
                       &layernorm_gelu_tile_run<T, G, V, W, R, true, false, true>, false,
                       nullptr};
}

// A general tile with the one shifted pass; its phased form (rows at any
// offset) keeps the two passes.
template <typename T, int G, int V, int W, int R = 1>
constexpr TileVariant tile_shifted()
{
    return TileVariant{G, V, W, R, G * V * kWave * Elem<T>::kVec, false,
                       &layernorm_gelu_tile_run<T, G, V, W, R, false, false, true>, false,
                       phased_run<T, G, V, W, R, false>()};
}

// The persistent form of an exact one-pass tile.  rows_per_group 1: the
// grid never has more workgroups than a one-row tile's.
template <typename T, int G, int V, int W>
constexpr TileVariant exact_rows()
{
    return TileVariant{G, V, W, 1, G * V * kWave * Elem<T>::kVec, true,
                       &layernorm_gelu_rows_run<T, G, V, W>, false, nullptr};
}

// Preference order as for softmax: first exact entry with max_n == N, else
// the first general entry that holds N.  General entries ascend in capacity
// so that a row takes the smallest tile that holds it: a tile's time per row
// follows its capacity (every register slot is loaded, reduced and passed
// through the epilogue), and the 16-wave tiles, one workgroup per CU at their
// register count, measured slower below capacity than the streaming kernel,
// which therefore takes the N between the last general entry and the exact
// 16384 (fp32) / 32768 (bf16).  alt(): run by index only.
static const TileVariant kLayerNormF32[] = {
    exact<float, 1, 1, 4>(),    // N = 256
    exact<float, 1, 2, 4>(),    // N = 512
    exact<float, 1, 3, 4>(),    // N = 768 (kernel trace, 4096 rows: 5.93 us; one-wave
                                // workgroups 5.96, two 6.01, eight 6.06; two rows
                                // per wave 6.36-6.58)
    exact<float, 1, 4, 4>(),    // N = 1024
    exact<float, 1, 8, 4>(),    // N = 2048
    exact<float, 4, 4, 4, 2>(), // N = 4096 (two rows: 47.1 us vs 51.5 for one, 64 MiB)
    exact<float, 8, 4, 8, 2>(), // N = 8192 (two rows: 47.6 us vs 50.0 for 4 x 8, one row)
    exact<float, 8, 8, 8>(),    // N = 16384 (48 us vs 54 us for 16 x 4)
    // Common hidden sizes between the powers of two, 64 MiB of input, µs
    // against the general tile that would take them: 1536 46.9 vs 48.1;
    // 2560 48.0 vs 50.1; 3072 47.4 vs 50.5; 5120 48.0 vs 51.2; 6144 47.7 vs
    // 51.0; 12288 51.3 vs 55.2; 14336 51.1 vs 56.1 (7168: no gain).  Two rows
    // per group take a missing last row as the first row again.
    exact<float, 2, 3, 2, 2>(), // N = 1536
    exact<float, 2, 5, 2, 2>(), // N = 2560
    exact<float, 4, 3, 4, 2>(), // N = 3072
    exact<float, 4, 5, 4, 2>(), // N = 5120
    exact<float, 8, 3, 8, 2>(), // N = 6144
    exact<float, 8, 6, 8>(),    // N = 12288
    exact<float, 8, 7, 8>(),    // N = 14336
    tile<float, 1, 1, 4>(),     // N <= 256
    tile<float, 1, 2, 4>(),     // N <= 512
    tile<float, 1, 3, 4>(),     // N <= 768
    tile<float, 1, 4, 4>(),     // N <= 1024
    tile<float, 1, 8, 4>(),     // N <= 2048
    tile<float, 4, 4, 4>(),     // N <= 4096
    tile<float, 8, 4, 8>(),     // N <= 8192
    tile<float, 8, 6, 8>(),     // N <= 12288 (N = 12000: 51 us vs 65 us for 16 x 4)
    tile<float, 8, 7, 8>(),     // N <= 14336
    alt(tile<float, 16, 4, 16>()),
    alt(tile<float, 8, 8, 8>()),
    alt(tile<float, 1, 3, 4, 2>()),
    alt(tile<float, 2, 2, 4>()),
    alt(exact<float, 1, 3, 4, 2>()),
    alt(exact<float, 1, 3, 4, 4>()),
    alt(exact<float, 8, 4, 8>()),
    alt(exact<float, 16, 4, 16>()),
    alt(exact_shifted<float, 1, 3, 4>()),  // 3x the error of two passes, no faster
    // the one-row exact tiles the two-row ones replaced
    alt(exact<float, 4, 4, 4>()),
    alt(exact<float, 4, 8, 4>()),
};

// bf16 exact tiles take the one shifted pass (SH): bf16 storage rounding
// (2^-9) dwarfs the pass's cancellation, and one barrier per row instead of
// two measured 48.5 -> 47.0 us at 16384 x 4096 (kernel trace average).
static const TileVariant kLayerNormBF16[] = {
    exact_shifted<bf16_t, 1, 1, 4>(),    // N = 512
    exact_shifted<bf16_t, 2, 1, 2, 2>(), // N = 1024 (128 MiB: 45.0 us vs 45.4 for one wave per row)
    exact_shifted<bf16_t, 1, 4, 4>(),    // N = 2048
    exact_shifted<bf16_t, 4, 2, 4, 2>(), // N = 4096
    exact_rows<bf16_t, 8, 2, 8>(),       // N = 8192 (persistent: 47.6 us vs 51.3 us at 8192 rows)
    exact_rows<bf16_t, 8, 4, 8>(),       // N = 16384 (persistent: 46.4 vs 50.4 us; 8 x 4 tile:
                                         // 49 us vs 55 us for 16 x 2)
    exact_shifted<bf16_t, 16, 4, 16>(),  // N = 32768
    // Common hidden sizes between the powers of two, 128 MiB of input, µs
    // against the general tile that would take them (two passes or one,
    // masked): 1536 46.6 vs 60.5; 2560 49.0 vs 66.8; 3072 46.8 vs 57.5;
    // 5120 49.2 vs 54.6; 6144 47.3 vs 54.4; 7168 47.1 vs 56.2; 12288 47.9
    // vs 55.3; 14336 48.3 vs 59.8.
    exact_shifted<bf16_t, 1, 3, 4>(),    // N = 1536
    exact_shifted<bf16_t, 1, 5, 4>(),    // N = 2560
    exact_shifted<bf16_t, 2, 3, 2, 2>(), // N = 3072
    exact_rows<bf16_t, 2, 5, 2>(),       // N = 5120
    exact_shifted<bf16_t, 4, 3, 4, 2>(), // N = 6144
    exact_rows<bf16_t, 2, 7, 2>(),       // N = 7168
    exact_rows<bf16_t, 8, 3, 8>(),       // N = 12288
    exact_rows<bf16_t, 4, 7, 4>(),       // N = 14336
    // General tiles: the one shifted pass where it measured faster (128 MiB,
    // one process, alternating with the two-pass build): N = 7168 53.0 vs
    // 59.4 us, 12288 53.5 vs 55.8, 3000 55.2 vs 57.6, 3072 55.5 vs 56.2.  The
    // others keep two passes: there its registers cost a wave of occupancy
    // (N = 1000: 53.2 vs 47.9 us; 1536 57.2 vs 55.9; 6144 53.9 vs 52.1;
    // 5120 and 14336 the same).
    tile<bf16_t, 1, 1, 4>(),            // N <= 512
    tile<bf16_t, 1, 2, 4>(),            // N <= 1024
    tile<bf16_t, 1, 4, 4>(),            // N <= 2048
    tile_shifted<bf16_t, 4, 2, 4>(),    // N <= 4096 (N = 3000: 59 us vs 65 us for 2 x 4)
    tile<bf16_t, 4, 3, 4>(),            // N <= 6144
    tile_shifted<bf16_t, 8, 2, 8>(),    // N <= 8192
    tile_shifted<bf16_t, 8, 3, 8>(),    // N <= 12288
    tile<bf16_t, 8, 4, 8>(),            // N <= 16384 (N = 14000: 60 us vs 87 us for 16 x 2)
    tile<bf16_t, 8, 5, 8>(),            // N <= 20480
    // the other form of the dispatched general tiles
    alt(tile_shifted<bf16_t, 4, 2, 4, 2>()),
    alt(tile_shifted<bf16_t, 4, 3, 4, 2>()),
    alt(tile_shifted<bf16_t, 8, 2, 8, 2>()),
    alt(tile_shifted<bf16_t, 8, 3, 8, 2>()),
    alt(tile_shifted<bf16_t, 8, 4, 8, 2>()),
    alt(tile_shifted<bf16_t, 1, 2, 4>()),
    alt(tile_shifted<bf16_t, 4, 3, 4>()),
    alt(tile<bf16_t, 4, 2, 4>()),
    alt(tile<bf16_t, 8, 2, 8>()),
    alt(tile<bf16_t, 8, 3, 8>()),
    alt(tile<bf16_t, 2, 4, 4>()),
    alt(tile<bf16_t, 16, 2, 16>()),
    alt(tile<bf16_t, 16, 4, 16>()),
    alt(tile<bf16_t, 8, 8, 8>()),
    alt(tile<bf16_t, 1, 8, 4>()),
    alt(exact<bf16_t, 4, 2, 4>()),
    alt(exact<bf16_t, 2, 4, 4>()),
    alt(exact<bf16_t, 1, 8, 4>()),
    alt(exact<bf16_t, 2, 4, 4, 2>()),
    alt(exact<bf16_t, 16, 2, 16>()),
    alt(exact<bf16_t, 8, 8, 8>()),
    alt(exact<bf16_t, 4, 8, 4>()),
    // the two-pass forms of the dispatched exact tiles
    alt(exact<bf16_t, 1, 1, 4>()),
    alt(exact<bf16_t, 1, 2, 4>()),
    alt(exact<bf16_t, 1, 4, 4>()),
    alt(exact<bf16_t, 4, 2, 4, 2>()),
    alt(exact<bf16_t, 8, 2, 8>()),
    alt(exact<bf16_t, 8, 4, 8>()),
    alt(exact<bf16_t, 16, 4, 16>()),
    alt(exact_shifted<bf16_t, 2, 4, 4, 2>()),
    // measured at 16384 x 4096 against the dispatched 4 x 2 x 4, two rows
    // (47.5 us): one wave per row 51-55 us, two waves 48.0, 8 x 1 48.3,
    // four rows 47.4; persistent 4 x 2 48.8 (80 VGPRs: six waves per SIMD)
    alt(exact_shifted<bf16_t, 1, 8, 4>()),
    alt(exact_shifted<bf16_t, 2, 4, 4>()),
    alt(exact_shifted<bf16_t, 4, 2, 4, 4>()),
    alt(exact_rows<bf16_t, 4, 2, 4>()),
    alt(exact_shifted<bf16_t, 1, 2, 4>()),     // N = 1024: 45.4 us
    // the runners-up at the common hidden sizes (above)
    alt(exact_rows<bf16_t, 2, 3, 2>()),        // 3072: 48.3 us
    alt(exact_shifted<bf16_t, 2, 5, 2, 2>()),  // 5120: 50.2 us
    alt(exact_rows<bf16_t, 4, 3, 4>()),        // 6144: 48.3 us
    alt(exact_shifted<bf16_t, 2, 7, 2, 2>()),  // 7168: 52.7 us
    alt(exact_shifted<bf16_t, 8, 3, 8, 2>()),  // 12288: 51.4 us
    alt(exact_shifted<bf16_t, 4, 7, 4>()),     // 14336: 52.2 us
    // the one-pass tiles the persistent form replaced (a persistent 16 x 4
    // for N = 32768 measured 90.6 us against 60.7 us for the tile)
    alt(exact_shifted<bf16_t, 8, 2, 8>()),
    alt(exact_shifted<bf16_t, 8, 4, 8>()),
};

const TileVariant *layernorm_gelu_variants(rk_dtype dtype, int *count)
{
    if (dtype == RK_F32) {
        *count = static_cast<int>(sizeof(kLayerNormF32) / sizeof(kLayerNormF32[0]));
        return kLayerNormF32;
    }
    *count = static_cast<int>(sizeof(kLayerNormBF16) / sizeof(kLayerNormBF16[0]));
    return kLayerNormBF16;
}

}  // namespace rk
