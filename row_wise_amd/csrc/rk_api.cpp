// C ABI of librowkern.so: argument validation (before any HIP call) and the
// choice of kernel for each call.  See include/rowkern.h for the contract.
#include <climits>
#include <initializer_list>
#include <cmath>
#include <cstdint>

#include "rk_internal.h"

using namespace rk;

namespace {

bool valid_dtype(rk_dtype d) { return d == RK_F32 || d == RK_BF16; }

// Longest row: kernels index vectors of a row with 32-bit integers.
constexpr int64_t kMaxN = int64_t{1} << 30;

struct Span {
    uintptr_t lo, hi;  // [lo, hi) in bytes
};

Span matrix_span(const void *p, int64_t M, int64_t N, int64_t ld, int es)
{
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    return Span{lo, lo + static_cast<uintptr_t>(((M - 1) * ld + N) * es)};
}

bool overlaps(Span a, Span b) { return a.lo < b.hi && b.lo < a.hi; }

bool aligned16(const void *p) { return reinterpret_cast<uintptr_t>(p) % 16 == 0; }

// Byte extent (M-1)*ld + N elements must be representable.
bool extent_ok(int64_t M, int64_t N, int64_t ld, int es)
{
    const int64_t lim = INT64_MAX / es - N;
    return M - 1 <= lim / ld;
}

// Validation shared by every row entry point.  Returns RK_OK also for M == 0
// (the caller then returns without launching).
rk_status check_rows(const void *x, const void *y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                     rk_dtype dtype)
{
    if (!valid_dtype(dtype))
        return RK_ERR_INVALID_ARG;
    if (M < 0 || N < 1 || N > INT32_MAX || ldx < N || ldy < N)
        return RK_ERR_INVALID_ARG;
    if (N > kMaxN)
        return RK_ERR_UNSUPPORTED;
    if (M == 0)
        return RK_OK;
    if (x == nullptr || y == nullptr)
        return RK_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (!extent_ok(M, N, ldx, es) || !extent_ok(M, N, ldy, es))
        return RK_ERR_INVALID_ARG;
    if (reinterpret_cast<uintptr_t>(x) % es || reinterpret_cast<uintptr_t>(y) % es)
        return RK_ERR_INVALID_ARG;
    const bool in_place = x == y && ldx == ldy;
    if (!in_place && overlaps(matrix_span(x, M, N, ldx, es), matrix_span(y, M, N, ldy, es)))
        return RK_ERR_INVALID_ARG;
    return RK_OK;
}

// The 16-byte vector path needs aligned bases and row pitches.
bool rows_aligned(const void *x, const void *y, int64_t ldx, int64_t ldy, int es)
{
    return aligned16(x) && aligned16(y) && (ldx * es) % 16 == 0 && (ldy * es) % 16 == 0;
}

// The row-in-memory kernels read each row as aligned 16-byte vectors from
// the row's own offset past a 16-byte boundary; the matrices they read or
// write by row must share that offset, row for row, for all M rows.
bool same_phase(const void *a, int64_t lda, const void *b, int64_t ldb, int es)
{
    return (reinterpret_cast<uintptr_t>(a) - reinterpret_cast<uintptr_t>(b)) % 16 == 0 &&
           ((lda - ldb) * es) % 16 == 0;
}

// gridDim.x * blockDim.x must stay below 2^32 work-items.
bool grid_ok(int64_t blocks, int threads)
{
    return blocks >= 1 && blocks <= (int64_t{UINT32_MAX} / threads);
}

rk_status hip_status(hipError_t e) { return e == hipSuccess ? RK_OK : RK_ERR_HIP; }

RowProblem make_problem(const void *x, void *y, const void *w, const void *b, int64_t M,
                        int64_t N, int64_t ldx, int64_t ldy, float eps, rk_dtype dtype,
                        hipStream_t stream)
{
    return RowProblem{x, y, w, b, M, static_cast<int>(N), ldx, ldy, eps, dtype, stream};
}

const TileVariant *variants(rk_op op, rk_dtype dtype, int *count)
{
    *count = 0;
    if (!valid_dtype(dtype))
        return nullptr;
    if (op == RK_OP_SOFTMAX)
        return softmax_variants(dtype, count);
    if (op == RK_OP_LAYERNORM_GELU)
        return layernorm_gelu_variants(dtype, count);
    if (op == RK_OP_RMSNORM)
        return rmsnorm_variants(dtype, false, count);
    if (op == RK_OP_RESIDUAL_RMSNORM)
        return rmsnorm_variants(dtype, true, count);
    return nullptr;
}

int pick_variant(rk_op op, rk_dtype dtype, int64_t N)
{
    int count = 0;
    const TileVariant *v = variants(op, dtype, &count);
    int general = -1;
    for (int i = 0; i < count; ++i) {
        if (v[i].alternative)
            continue;
        if (v[i].exact && N == v[i].max_n)
            return i;
        if (!v[i].exact && general < 0 && N <= v[i].max_n)
            general = i;
    }
    return general;
}

// The general tile whose phased form takes rows of N at any offset: the first
// dispatched general entry with room for N + E - 1 columns, or -1.
int pick_phased(rk_op op, rk_dtype dtype, int64_t N)
{
    int count = 0;
    const TileVariant *v = variants(op, dtype, &count);
    for (int i = 0; i < count; ++i)
        if (!v[i].alternative && !v[i].exact && v[i].accepts_phased(N, vec_elems(dtype)))
            return i;
    return -1;
}

int64_t tile_blocks(const TileVariant &v, int64_t M)
{
    const int64_t rows_per_block = int64_t{v.waves_per_block} / v.waves_per_row * v.rows_per_group;
    return (M + rows_per_block - 1) / rows_per_block;
}

constexpr int kStreamThreads = 1024;  // largest streaming workgroup (16 waves)
constexpr int kSplitThreads = 256;    // online_partials / online_finish
constexpr int kLoopThreads = 1024;    // largest rmsnorm_loop workgroup
constexpr int32_t kMaxSplits = 65536;

// Rates of the rows-in-memory kernels, in elements per microsecond, as
// measured on 1 to 64 rows of 2^18 to 2^20 elements: one workgroup streaming
// its row on one CU, and the split kernels with rows spread over the chip.
struct SplitRates {
    double row, all;
};

SplitRates split_rates(rk_op op, rk_dtype dtype)
{
    const bool f32 = dtype == RK_F32;
    if (op == RK_OP_LAYERNORM_GELU)
        return f32 ? SplitRates{4300.0, 530000.0} : SplitRates{5400.0, 850000.0};
    if (op == RK_OP_RMSNORM || op == RK_OP_RESIDUAL_RMSNORM)
        return f32 ? SplitRates{7000.0, 575000.0} : SplitRates{11500.0, 1100000.0};
    return f32 ? SplitRates{5500.0, 530000.0} : SplitRates{8500.0, 1000000.0};
}

// The first split kernel's launch and the second pass's merge cost about
// this much over one workgroup per row; keeping the partials in the output
// adds a third launch.
constexpr double kSplitExtraUs = 1.5;
constexpr double kOutputSplitExtraUs = 5.5;

// Split count for M rows of N: 1 where one workgroup per row is expected to
// be as fast.  A row streamed by one CU takes N / row microseconds; all rows
// spread over the chip take M N / all.  Splitting pays when the first exceeds
// the second by more than `extra_us`, and with a workspace also for rows of
// 2^16 or more in at most 128 rows, which leave half the CUs idle (measured
// 5-18% faster at 128 rows, 4-20% slower at 200).  Chunks are about 16 KiB
// (measured best from 4 KiB to 64 KiB) and at most 2048 workgroups run (more
// cost more to launch than they gain).
int32_t pick_splits(SplitRates r, int64_t M, int64_t N, rk_dtype dtype, double extra_us)
{
    if (M < 1 || N < 1 || M >= 256)
        return 1;
    const double gain = N / r.row - static_cast<double>(M) * N / r.all;
    const bool wide = extra_us <= kSplitExtraUs && N >= 65536 && M <= 128;
    if (!(gain > extra_us || wide))
        return 1;
    const int64_t chunk_elems = 16384 / elem_size(dtype);
    int64_t s = (N + chunk_elems - 1) / chunk_elems;
    const int64_t by_grid = 2048 / M;
    if (s > by_grid)
        s = by_grid;
    if (s > kMaxSplits)
        s = kMaxSplits;
    return static_cast<int32_t>(s < 2 ? 1 : s);
}

int32_t pick_splits(rk_op op, int64_t M, int64_t N, rk_dtype dtype, double extra_us)
{
    return pick_splits(split_rates(op, dtype), M, N, dtype, extra_us);
}

int32_t auto_splits(int64_t M, int64_t N, rk_dtype dtype)
{
    return pick_splits(RK_OP_SOFTMAX, M, N, dtype, kSplitExtraUs);
}

bool softmax_vectorized(const RowProblem &p)
{
    return same_phase(p.x, p.ldx, p.y, p.ldy, elem_size(p.dtype));
}

// Weight and bias are shifted into each row's phase from 16-byte alignment.
bool layernorm_vectorized(const RowProblem &p)
{
    return softmax_vectorized(p) && aligned16(p.w) && aligned16(p.b);
}

// Access mode of the kernels that keep rows in memory.
RowIo softmax_io(const RowProblem &p)
{
    if (rows_aligned(p.x, p.y, p.ldx, p.ldy, elem_size(p.dtype)))
        return kIoAligned;
    return softmax_vectorized(p) ? kIoPhased : kIoElement;
}

RowIo layernorm_io(const RowProblem &p)
{
    if (!aligned16(p.w) || !aligned16(p.b))
        return kIoElement;
    return softmax_io(p);
}

rk_status softmax_generic(const RowProblem &p)
{
    if (!grid_ok(p.M, kStreamThreads))
        return RK_ERR_UNSUPPORTED;
    return hip_status(online_stream_run(p, softmax_io(p)));
}

// The split partials kept in each output row.
SplitPartials output_partials(const RowProblem &p)
{
    return SplitPartials{static_cast<char *>(p.y), p.ldy * elem_size(p.dtype), true};
}

// Long rows in few rows split across workgroups even without a workspace:
// each row keeps its S partials (and `extra` more 8-byte slots: LayerNorm's
// shift) in its own output, inside the first chunk, which the last of three
// kernels writes after reading them.  That needs an output apart from the
// input and a first chunk with room for the S + extra slots and the step to
// the next 8-byte boundary; S is lowered until it has room.  Returns the
// splits to use (1: none) and, for more, their chunk length.
int32_t output_splits(const RowProblem &p, int32_t S, RowIo io, int64_t *chunk, int extra = 0)
{
    if (S <= 1 || p.x == p.y || p.M > INT64_MAX / S || !grid_ok(p.M * S, kSplitThreads))
        return 1;
    const int es = elem_size(p.dtype);
    const int vec = io != kIoElement ? vec_elems(p.dtype) : 1;
    // a phased row's first vector holds up to E - 1 columns before the row
    const int64_t lead = io == kIoPhased ? vec - 1 : 0;
    for (; S > 1; --S) {
        const int64_t c = split_chunk(p.N, S, vec);
        const int64_t first = c - lead < p.N ? c - lead : p.N;
        if (c <= INT32_MAX && first * es >= 8 * (int64_t{S} + extra) + 8) {
            *chunk = c;
            return S;
        }
    }
    return 1;
}

rk_status layernorm_generic(const RowProblem &p)
{
    if (!grid_ok(p.M, kStreamThreads))
        return RK_ERR_UNSUPPORTED;
    return hip_status(layernorm_stream_run(p, layernorm_io(p)));
}

bool valid_gelu(rk_gelu_kind g) { return g == RK_GELU_TANH || g == RK_GELU_ERF; }

// The LayerNorm epilogue also takes no activation (the LayerNorm alone).
bool valid_layernorm_act(rk_gelu_kind g) { return valid_gelu(g) || g == RK_GELU_NONE; }

int32_t layernorm_auto_splits(int64_t M, int64_t N, rk_dtype dtype,
                              double extra_us = kSplitExtraUs)
{
    // rows a register tile takes are read once there: no split
    if (pick_variant(RK_OP_LAYERNORM_GELU, dtype, N) >= 0)
        return 1;
    return pick_splits(RK_OP_LAYERNORM_GELU, M, N, dtype, extra_us);
}

// Bytes of the split-row workspace: two floats per chunk ((m, d) for softmax,
// (mean, M2) for LayerNorm), plus `extra` 8-byte slots per row.
size_t split_workspace_bytes(int64_t M, int64_t S, int extra = 0)
{
    if (S <= 1 || M > INT64_MAX / 8 / (S + extra))
        return 0;
    return static_cast<size_t>(M * (S + extra) * 8);
}

// LayerNorm's split kernels keep one more slot per row after the S chunk
// summaries: the row's shift K = x[r][0], stored by the first kernel, so that
// the output kernel never reads x[r][0] again (in place, another workgroup
// of the same launch may already have overwritten it).
constexpr int kLayerNormSlots = 1;

// Workspace checks shared by the split-row entry points: `spans` are the
// caller's matrices, which the workspace (written by the first kernel) must
// not overlap.
rk_status check_workspace(void *workspace, size_t workspace_bytes, size_t need, int64_t M,
                          int32_t S, std::initializer_list<Span> spans)
{
    if (need == 0)
        return RK_ERR_UNSUPPORTED;
    if (workspace != nullptr && reinterpret_cast<uintptr_t>(workspace) % 8 != 0)
        return RK_ERR_INVALID_ARG;
    if (workspace == nullptr || workspace_bytes < need)
        return RK_ERR_WORKSPACE;
    if (M > INT64_MAX / S || !grid_ok(M * S, kSplitThreads))
        return RK_ERR_UNSUPPORTED;
    const Span ws{reinterpret_cast<uintptr_t>(workspace),
                  reinterpret_cast<uintptr_t>(workspace) + need};
    for (const Span &sp : spans)
        if (overlaps(ws, sp))
            return RK_ERR_INVALID_ARG;
    return RK_OK;
}

rk_status run_tile(const TileVariant &v, const RowProblem &p, bool phased = false)
{
    const int64_t blocks = tile_blocks(v, p.M);
    if (!grid_ok(blocks, v.waves_per_block * 64))
        return RK_ERR_UNSUPPORTED;
    return hip_status(phased ? v.run_phased(p) : v.run(p));
}

// A tile forced by index: aligned rows run it as compiled; rows that share
// their offsets with the output (and, where given, weight and bias are
// aligned) run its phased form if it has one that holds them.
rk_status run_forced(const TileVariant &v, const RowProblem &p, bool aligned, bool vectorized)
{
    if (aligned && v.accepts(p.N))
        return run_tile(v, p);
    if (!aligned && vectorized && v.accepts_phased(p.N, vec_elems(p.dtype)))
        return run_tile(v, p, true);
    return RK_ERR_UNSUPPORTED;
}

rk_status check_layernorm(const void *x, const void *w, const void *b, const void *y, int64_t M,
                          int64_t N, int64_t ldx, int64_t ldy, float eps, rk_dtype dtype)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    if (!std::isfinite(eps) || !(eps > 0.0f))
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    if (w == nullptr || b == nullptr)
        return RK_ERR_INVALID_ARG;
    const int es = elem_size(dtype);
    if (reinterpret_cast<uintptr_t>(w) % es || reinterpret_cast<uintptr_t>(b) % es)
        return RK_ERR_INVALID_ARG;
    const Span ys = matrix_span(y, M, N, ldy, es);
    if (overlaps(ys, matrix_span(w, 1, N, N, es)) || overlaps(ys, matrix_span(b, 1, N, N, es)))
        return RK_ERR_INVALID_ARG;
    return RK_OK;
}

bool layernorm_aligned(const RowProblem &p)
{
    return rows_aligned(p.x, p.y, p.ldx, p.ldy, elem_size(p.dtype)) && aligned16(p.w) &&
           aligned16(p.b);
}

// LayerNorm+GeLU in one kernel: a register tile where one holds the row,
// else the streaming kernel.
rk_status layernorm_single(const RowProblem &p)
{
    int count = 0;
    const TileVariant *v = layernorm_gelu_variants(p.dtype, &count);
    const int idx = pick_variant(RK_OP_LAYERNORM_GELU, p.dtype, p.N);
    const bool aligned = layernorm_aligned(p);
    if (aligned && idx >= 0)
        return run_tile(v[idx], p);
    if (!aligned && layernorm_vectorized(p)) {
        const int ph = pick_phased(RK_OP_LAYERNORM_GELU, p.dtype, p.N);
        if (ph >= 0)
            return run_tile(v[ph], p, true);
    }
    return layernorm_generic(p);
}

bool valid_eps(float eps) { return std::isfinite(eps) && eps > 0.0f; }

bool elem_aligned(const void *p, int es) { return reinterpret_cast<uintptr_t>(p) % es == 0; }

// An output may be an input exactly (same pointer, same pitch) or be disjoint
// from it.
bool alias_ok(const void *out, int64_t ldo, const void *in, int64_t ldi, int64_t M, int64_t N,
              int es)
{
    if (out == in && ldo == ldi)
        return true;
    return !overlaps(matrix_span(out, M, N, ldo, es), matrix_span(in, M, N, ldi, es));
}

rk_status check_rmsnorm(const void *x, const void *w, const void *y, int64_t M, int64_t N,
                        int64_t ldx, int64_t ldy, float eps, rk_dtype dtype)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    if (!valid_eps(eps))
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const int es = elem_size(dtype);
    if (w == nullptr || !elem_aligned(w, es))
        return RK_ERR_INVALID_ARG;
    if (overlaps(matrix_span(y, M, N, ldy, es), matrix_span(w, 1, N, N, es)))
        return RK_ERR_INVALID_ARG;
    return RK_OK;
}

rk_status check_residual_rmsnorm(const void *x, const void *r, const void *w, const void *y,
                                 const void *ro, int64_t M, int64_t N, int64_t ldx, int64_t ldr,
                                 int64_t ldy, int64_t ldo, float eps, rk_dtype dtype)
{
    if (!valid_dtype(dtype))
        return RK_ERR_INVALID_ARG;
    if (M < 0 || N < 1 || N > INT32_MAX || ldx < N || ldr < N || ldy < N || ldo < N)
        return RK_ERR_INVALID_ARG;
    if (N > kMaxN)
        return RK_ERR_UNSUPPORTED;
    if (!valid_eps(eps))
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const int es = elem_size(dtype);
    for (const void *p : {x, r, w, static_cast<const void *>(y), static_cast<const void *>(ro)})
        if (p == nullptr || !elem_aligned(p, es))
            return RK_ERR_INVALID_ARG;
    for (int64_t ld : {ldx, ldr, ldy, ldo})
        if (!extent_ok(M, N, ld, es))
            return RK_ERR_INVALID_ARG;
    // outputs: each may be an input exactly, never the other output or the weight
    if (!alias_ok(y, ldy, x, ldx, M, N, es) || !alias_ok(y, ldy, r, ldr, M, N, es) ||
        !alias_ok(ro, ldo, x, ldx, M, N, es) || !alias_ok(ro, ldo, r, ldr, M, N, es))
        return RK_ERR_INVALID_ARG;
    if (overlaps(matrix_span(y, M, N, ldy, es), matrix_span(ro, M, N, ldo, es)))
        return RK_ERR_INVALID_ARG;
    const Span ws = matrix_span(w, 1, N, N, es);
    if (overlaps(matrix_span(y, M, N, ldy, es), ws) || overlaps(matrix_span(ro, M, N, ldo, es), ws))
        return RK_ERR_INVALID_ARG;
    return RK_OK;
}

bool rmsnorm_aligned(const RowProblem &p, bool residual)
{
    const int es = elem_size(p.dtype);
    bool ok = rows_aligned(p.x, p.y, p.ldx, p.ldy, es) && aligned16(p.w);
    if (residual)
        ok = ok && rows_aligned(p.r, p.ro, p.ldr, p.ldo, es);
    return ok;
}

bool rmsnorm_vectorized(const RowProblem &p, bool residual)
{
    const int es = elem_size(p.dtype);
    bool ok = same_phase(p.x, p.ldx, p.y, p.ldy, es) && aligned16(p.w);
    if (residual)
        ok = ok && same_phase(p.x, p.ldx, p.r, p.ldr, es) && same_phase(p.x, p.ldx, p.ro, p.ldo, es);
    return ok;
}

RowIo rmsnorm_io(const RowProblem &p, bool residual)
{
    if (rmsnorm_aligned(p, residual))
        return kIoAligned;
    return rmsnorm_vectorized(p, residual) ? kIoPhased : kIoElement;
}

rk_status rmsnorm_generic(const RowProblem &p, bool residual)
{
    if (!grid_ok(p.M, kLoopThreads))
        return RK_ERR_UNSUPPORTED;
    return hip_status(rmsnorm_loop_run(p, residual, rmsnorm_io(p, residual)));
}

// Long rows in few rows that no tile takes split with the partials kept in
// y, which may then alias neither input.
int32_t rmsnorm_output_splits(const RowProblem &p, bool residual, rk_op op, RowIo io,
                              int64_t *chunk)
{
    if (pick_variant(op, p.dtype, p.N) >= 0 || (residual && p.r == p.y))
        return 1;
    // the fused form splits exactly where the plain one does, so that its y
    // stays bitwise the plain RMSNorm of its residual_out
    return output_splits(p, pick_splits(RK_OP_RMSNORM, p.M, p.N, p.dtype, kOutputSplitExtraUs),
                         io, chunk);
}

rk_status rmsnorm_dispatch(const RowProblem &p, bool residual, int32_t index, bool forced)
{
    int count = 0;
    const TileVariant *v = rmsnorm_variants(p.dtype, residual, &count);
    const bool aligned = rmsnorm_aligned(p, residual);
    if (forced) {
        if (index < -1 || index >= count)
            return RK_ERR_INVALID_ARG;
        if (index == -1)
            return rmsnorm_generic(p, residual);
        return run_forced(v[index], p, aligned, rmsnorm_vectorized(p, residual));
    }
    const rk_op op = residual ? RK_OP_RESIDUAL_RMSNORM : RK_OP_RMSNORM;
    const int idx = pick_variant(op, p.dtype, p.N);
    if (aligned && idx >= 0)
        return run_tile(v[idx], p);
    if (!aligned && rmsnorm_vectorized(p, residual)) {
        const int ph = pick_phased(op, p.dtype, p.N);
        if (ph >= 0)
            return run_tile(v[ph], p, true);
    }
    const RowIo io = rmsnorm_io(p, residual);
    int64_t C = 0;
    const int32_t S = rmsnorm_output_splits(p, residual, op, io, &C);
    if (S > 1)
        return hip_status(
            rmsnorm_split_run(p, residual, S, static_cast<int>(C), output_partials(p), io));
    return rmsnorm_generic(p, residual);
}

}  // namespace

// ------------------------------------------------------------------ ABI

RK_EXPORT rk_status rk_softmax(const void *x, void *y, int64_t M, int64_t N, int64_t ldx,
                               int64_t ldy, rk_dtype dtype, hipStream_t stream)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK || M == 0)
        return st;
    const RowProblem p = make_problem(x, y, nullptr, nullptr, M, N, ldx, ldy, 0.0f, dtype, stream);
    const bool aligned = rows_aligned(x, y, ldx, ldy, elem_size(dtype));
    int count = 0;
    const TileVariant *v = softmax_variants(dtype, &count);
    const int idx = pick_variant(RK_OP_SOFTMAX, dtype, N);
    if (aligned && idx >= 0)
        return run_tile(v[idx], p);
    if (!aligned && softmax_vectorized(p)) {
        const int ph = pick_phased(RK_OP_SOFTMAX, dtype, N);
        if (ph >= 0)
            return run_tile(v[ph], p, true);
    }
    const RowIo io = softmax_io(p);
    int64_t C = 0;
    const int32_t S =
        output_splits(p, pick_splits(RK_OP_SOFTMAX, M, N, dtype, kOutputSplitExtraUs), io, &C);
    if (S > 1)
        return hip_status(online_split_run(p, S, static_cast<int>(C), output_partials(p), io));
    return softmax_generic(p);
}

RK_EXPORT int32_t rk_online_softmax_auto_splits(int64_t M, int64_t N, rk_dtype dtype)
{
    if (M < 1 || N < 1 || !valid_dtype(dtype))
        return 1;
    return auto_splits(M, N, dtype);
}

RK_EXPORT size_t rk_online_softmax_workspace_bytes(int64_t M, int64_t N, int32_t num_splits,
                                                   rk_dtype dtype)
{
    if (M < 1 || N < 1 || N > kMaxN || num_splits < 0 || num_splits > kMaxSplits ||
        !valid_dtype(dtype))
        return 0;
    const int64_t S = num_splits == 0 ? auto_splits(M, N, dtype) : num_splits;
    return split_workspace_bytes(M, S);
}

RK_EXPORT rk_status rk_online_softmax(const void *x, void *y, int64_t M, int64_t N, int64_t ldx,
                                      int64_t ldy, rk_dtype dtype, int32_t num_splits,
                                      void *workspace, size_t workspace_bytes, hipStream_t stream)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    if (num_splits < 0 || num_splits > kMaxSplits)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const RowProblem p = make_problem(x, y, nullptr, nullptr, M, N, ldx, ldy, 0.0f, dtype, stream);
    const int32_t S = num_splits == 0 ? auto_splits(M, N, dtype) : num_splits;
    if (S <= 1)
        return softmax_generic(p);
    const RowIo io = softmax_io(p);
    const bool vec = io != kIoElement;

    const int es = elem_size(dtype);
    st = check_workspace(workspace, workspace_bytes, split_workspace_bytes(M, S), M, S,
                         {matrix_span(x, M, N, ldx, es), matrix_span(y, M, N, ldy, es)});
    if (st != RK_OK)
        return st;
    const int64_t chunk = split_chunk(N, S, vec ? vec_elems(dtype) : 1);
    if (chunk > INT32_MAX)
        return RK_ERR_UNSUPPORTED;
    const SplitPartials pt{static_cast<char *>(workspace), int64_t{S} * 8, false};
    return hip_status(online_split_run(p, S, static_cast<int>(chunk), pt, io));
}

RK_EXPORT rk_status rk_online_softmax_noalloc(const void *x, void *y, int64_t M, int64_t N,
                                              int64_t ldx, int64_t ldy, rk_dtype dtype,
                                              int32_t num_splits, hipStream_t stream)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    if (num_splits < 0 || num_splits > kMaxSplits)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const RowProblem p = make_problem(x, y, nullptr, nullptr, M, N, ldx, ldy, 0.0f, dtype, stream);
    const int32_t S = num_splits == 0 ? auto_splits(M, N, dtype) : num_splits;
    if (S <= 1)
        return softmax_generic(p);
    const size_t need = split_workspace_bytes(M, S);
    if (need == 0 || need > kScratchBytes)
        return RK_ERR_SCRATCH;
    if (!grid_ok(M * S, kSplitThreads))
        return RK_ERR_UNSUPPORTED;
    const RowIo io = softmax_io(p);
    const int64_t chunk = split_chunk(N, S, io != kIoElement ? vec_elems(dtype) : 1);
    if (chunk > INT32_MAX)
        return RK_ERR_UNSUPPORTED;
    // the scratch of the current device, which the stream must run on
    int device = 0;
    if (hipGetDevice(&device) != hipSuccess)
        return RK_ERR_HIP;
    if (stream != nullptr) {
        int stream_device = 0;
        if (hipStreamGetDevice(stream, &stream_device) != hipSuccess || stream_device != device)
            return RK_ERR_INVALID_ARG;
    }
    void *scratch = nullptr;
    if (scratch_address(device, &scratch) != hipSuccess)
        return RK_ERR_HIP;
    const SplitPartials pt{static_cast<char *>(scratch), int64_t{S} * 8, false};
    return hip_status(online_split_run(p, S, static_cast<int>(chunk), pt, io));
}

RK_EXPORT int32_t rk_layernorm_gelu_auto_splits(int64_t M, int64_t N, rk_dtype dtype)
{
    if (M < 1 || N < 1 || !valid_dtype(dtype))
        return 1;
    return layernorm_auto_splits(M, N, dtype);
}

RK_EXPORT size_t rk_layernorm_gelu_workspace_bytes(int64_t M, int64_t N, int32_t num_splits,
                                                   rk_dtype dtype)
{
    if (M < 1 || N < 1 || N > kMaxN || num_splits < 0 || num_splits > kMaxSplits ||
        !valid_dtype(dtype))
        return 0;
    const int64_t S = num_splits == 0 ? layernorm_auto_splits(M, N, dtype) : num_splits;
    return split_workspace_bytes(M, S, kLayerNormSlots);
}

RK_EXPORT rk_status rk_layernorm_gelu_ex(const void *x, const void *weight, const void *bias,
                                         void *y, int64_t M, int64_t N, int64_t ldx, int64_t ldy,
                                         float eps, rk_dtype dtype, rk_gelu_kind gelu,
                                         int32_t num_splits, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream)
{
    rk_status st = check_layernorm(x, weight, bias, y, M, N, ldx, ldy, eps, dtype);
    if (st != RK_OK)
        return st;
    if (!valid_layernorm_act(gelu) || num_splits < 0 || num_splits > kMaxSplits)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    RowProblem p = make_problem(x, y, weight, bias, M, N, ldx, ldy, eps, dtype, stream);
    p.gelu = gelu;
    const int32_t S = num_splits == 0 ? layernorm_auto_splits(M, N, dtype) : num_splits;
    if (S <= 1)
        return layernorm_single(p);
    const int es = elem_size(dtype);
    st = check_workspace(workspace, workspace_bytes, split_workspace_bytes(M, S, kLayerNormSlots),
                         M, S,
                         {matrix_span(x, M, N, ldx, es), matrix_span(y, M, N, ldy, es),
                          matrix_span(weight, 1, N, N, es), matrix_span(bias, 1, N, N, es)});
    if (st != RK_OK)
        return st;
    const RowIo io = layernorm_io(p);
    const bool vec = io != kIoElement;
    const int64_t chunk = split_chunk(N, S, vec ? vec_elems(dtype) : 1);
    if (chunk > INT32_MAX)
        return RK_ERR_UNSUPPORTED;
    const SplitPartials pt{static_cast<char *>(workspace), (int64_t{S} + kLayerNormSlots) * 8,
                           false};
    return hip_status(layernorm_split_run(p, S, static_cast<int>(chunk), pt, io));
}

RK_EXPORT rk_status rk_layernorm_gelu(const void *x, const void *weight, const void *bias, void *y,
                                      int64_t M, int64_t N, int64_t ldx, int64_t ldy, float eps,
                                      rk_dtype dtype, hipStream_t stream)
{
    rk_status st = check_layernorm(x, weight, bias, y, M, N, ldx, ldy, eps, dtype);
    if (st != RK_OK || M == 0)
        return st;
    RowProblem p = make_problem(x, y, weight, bias, M, N, ldx, ldy, eps, dtype, stream);
    p.gelu = RK_GELU_TANH;
    const RowIo io = layernorm_io(p);
    int64_t C = 0;
    const int32_t S =
        output_splits(p, layernorm_auto_splits(M, N, dtype, kOutputSplitExtraUs), io, &C,
                      kLayerNormSlots);
    if (S > 1)
        return hip_status(layernorm_split_run(p, S, static_cast<int>(C), output_partials(p), io));
    return layernorm_single(p);
}

RK_EXPORT rk_status rk_rmsnorm(const void *x, const void *weight, void *y, int64_t M, int64_t N,
                               int64_t ldx, int64_t ldy, float eps, rk_dtype dtype,
                               hipStream_t stream)
{
    rk_status st = check_rmsnorm(x, weight, y, M, N, ldx, ldy, eps, dtype);
    if (st != RK_OK || M == 0)
        return st;
    const RowProblem p = make_problem(x, y, weight, nullptr, M, N, ldx, ldy, eps, dtype, stream);
    return rmsnorm_dispatch(p, false, 0, false);
}

RK_EXPORT rk_status rk_residual_rmsnorm(const void *x, const void *residual, const void *weight,
                                        void *y, void *residual_out, int64_t M, int64_t N,
                                        int64_t ldx, int64_t ldr, int64_t ldy, int64_t ldo,
                                        float eps, rk_dtype dtype, hipStream_t stream)
{
    rk_status st = check_residual_rmsnorm(x, residual, weight, y, residual_out, M, N, ldx, ldr,
                                          ldy, ldo, eps, dtype);
    if (st != RK_OK || M == 0)
        return st;
    RowProblem p = make_problem(x, y, weight, nullptr, M, N, ldx, ldy, eps, dtype, stream);
    p.r = residual;
    p.ro = residual_out;
    p.ldr = ldr;
    p.ldo = ldo;
    return rmsnorm_dispatch(p, true, 0, false);
}

// ------------------------------------------------- standalone primitives

namespace {

rk_status check_reduce(const void *x, const void *out, int64_t M, int64_t N, int64_t ldx,
                       rk_dtype dtype)
{
    if (!valid_dtype(dtype))
        return RK_ERR_INVALID_ARG;
    if (M < 0 || N < 1 || N > INT32_MAX || ldx < N)
        return RK_ERR_INVALID_ARG;
    if (N > kMaxN)
        return RK_ERR_UNSUPPORTED;
    if (M == 0)
        return RK_OK;
    const int es = elem_size(dtype);
    if (x == nullptr || out == nullptr || !elem_aligned(x, es) || !elem_aligned(out, es))
        return RK_ERR_INVALID_ARG;
    if (!extent_ok(M, N, ldx, es) || M > INT64_MAX / es)
        return RK_ERR_INVALID_ARG;
    // the results are written while other rows are still read: no overlap
    if (overlaps(matrix_span(x, M, N, ldx, es), matrix_span(out, 1, M, M, es)))
        return RK_ERR_INVALID_ARG;
    return RK_OK;
}

rk_status row_reduce_entry(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                           rk_dtype dtype, int op, hipStream_t stream)
{
    rk_status st = check_reduce(x, out, M, N, ldx, dtype);
    if (st != RK_OK || M == 0)
        return st;
    int threads = 0;
    if (!grid_ok(row_reduce_blocks(M, N, dtype, &threads), threads))
        return RK_ERR_UNSUPPORTED;
    const RowProblem p = make_problem(x, out, nullptr, nullptr, M, N, ldx, 1, 0.0f, dtype, stream);
    return hip_status(row_reduce_run(p, op));
}

// Rates of the row reductions (one read per element), elements per
// microsecond, measured on 1 to 64 rows of 2^18 to 2^20: one workgroup per
// row on one CU, and the split kernels with every CU busy.
SplitRates reduce_rates(rk_dtype dtype)
{
    return dtype == RK_F32 ? SplitRates{13000.0, 1600000.0} : SplitRates{20000.0, 2600000.0};
}

// The split's second launch: about 3 us back to back, against a single
// kernel that reads the data once.  Measured: 128 rows of 65536 take 8.3 us
// in one kernel and 8.8-9.3 split (fp32), 5.5 against 7.2 (bf16), so rows of
// 2^16 in at most 128 rows are not split here as they are for softmax.
constexpr double kReduceSplitExtraUs = 3.5;

int32_t reduce_auto_splits(int64_t M, int64_t N, rk_dtype dtype)
{
    return pick_splits(reduce_rates(dtype), M, N, dtype, kReduceSplitExtraUs);
}

// One float per (row, chunk).
size_t reduce_workspace_bytes(int64_t M, int64_t S)
{
    if (S <= 1 || M > INT64_MAX / 4 / S)
        return 0;
    return static_cast<size_t>(M * S * 4);
}

rk_status row_reduce_ex_entry(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                              rk_dtype dtype, int op, int32_t num_splits, void *workspace,
                              size_t workspace_bytes, hipStream_t stream)
{
    rk_status st = check_reduce(x, out, M, N, ldx, dtype);
    if (st != RK_OK)
        return st;
    if (num_splits < 0 || num_splits > kMaxSplits)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const int32_t S = num_splits == 0 ? reduce_auto_splits(M, N, dtype) : num_splits;
    if (S <= 1)
        return row_reduce_entry(x, out, M, N, ldx, dtype, op, stream);
    const int es = elem_size(dtype);
    st = check_workspace(workspace, workspace_bytes, reduce_workspace_bytes(M, S), M, S,
                         {matrix_span(x, M, N, ldx, es), matrix_span(out, 1, M, M, es)});
    if (st != RK_OK)
        return st;
    // rows are read as the aligned vectors that cover them, at any offset
    const int64_t chunk = split_chunk(N, S, vec_elems(dtype));
    if (chunk > INT32_MAX || !grid_ok((M + 3) / 4, kSplitThreads))
        return RK_ERR_UNSUPPORTED;
    const RowProblem p = make_problem(x, out, nullptr, nullptr, M, N, ldx, 1, 0.0f, dtype, stream);
    return hip_status(row_reduce_split_run(p, op, S, static_cast<int>(chunk),
                                           static_cast<float *>(workspace)));
}

}  // namespace

RK_EXPORT rk_status rk_row_sum(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                               rk_dtype dtype, hipStream_t stream)
{
    return row_reduce_entry(x, out, M, N, ldx, dtype, RK_REDUCE_SUM, stream);
}

RK_EXPORT rk_status rk_row_max(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                               rk_dtype dtype, hipStream_t stream)
{
    return row_reduce_entry(x, out, M, N, ldx, dtype, RK_REDUCE_MAX, stream);
}

RK_EXPORT int32_t rk_row_reduce_auto_splits(int64_t M, int64_t N, rk_dtype dtype)
{
    if (M < 1 || N < 1 || !valid_dtype(dtype))
        return 1;
    return reduce_auto_splits(M, N, dtype);
}

RK_EXPORT size_t rk_row_reduce_workspace_bytes(int64_t M, int64_t N, int32_t num_splits,
                                               rk_dtype dtype)
{
    if (M < 1 || N < 1 || N > kMaxN || num_splits < 0 || num_splits > kMaxSplits ||
        !valid_dtype(dtype))
        return 0;
    const int64_t S = num_splits == 0 ? reduce_auto_splits(M, N, dtype) : num_splits;
    return reduce_workspace_bytes(M, S);
}

RK_EXPORT rk_status rk_row_sum_ex(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                                  rk_dtype dtype, int32_t num_splits, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream)
{
    return row_reduce_ex_entry(x, out, M, N, ldx, dtype, RK_REDUCE_SUM, num_splits, workspace,
                               workspace_bytes, stream);
}

RK_EXPORT rk_status rk_row_max_ex(const void *x, void *out, int64_t M, int64_t N, int64_t ldx,
                                  rk_dtype dtype, int32_t num_splits, void *workspace,
                                  size_t workspace_bytes, hipStream_t stream)
{
    return row_reduce_ex_entry(x, out, M, N, ldx, dtype, RK_REDUCE_MAX, num_splits, workspace,
                               workspace_bytes, stream);
}

RK_EXPORT rk_status rk_gelu(const void *x, void *y, int64_t M, int64_t N, int64_t ldx,
                            int64_t ldy, rk_dtype dtype, rk_gelu_kind gelu, hipStream_t stream)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    if (!valid_gelu(gelu))
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    RowProblem p = make_problem(x, y, nullptr, nullptr, M, N, ldx, ldy, 0.0f, dtype, stream);
    p.gelu = gelu;
    const int es = elem_size(dtype);
    // a contiguous buffer is one flat array, read as aligned vectors from
    // its offset when the output shares it
    const bool contiguous = M == 1 || (ldx == N && ldy == N);
    const bool same_base_phase =
        (reinterpret_cast<uintptr_t>(x) - reinterpret_cast<uintptr_t>(y)) % 16 == 0;
    if (contiguous && same_base_phase)
        return hip_status(gelu_run(p, true, kIoAligned));
    if (!grid_ok(M, 256))
        return RK_ERR_UNSUPPORTED;
    RowIo io = kIoElement;
    if (rows_aligned(x, y, ldx, ldy, es))
        io = kIoAligned;
    else if (same_phase(x, ldx, y, ldy, es))
        io = kIoPhased;
    return hip_status(gelu_run(p, false, io));
}

// ------------------------------------------------------------ attention

namespace {

// Span of a [B][H][T][d] tensor with element strides s; false on overflow.
bool attn_span(const void *p, int64_t B, int64_t H, int64_t T, int64_t d, const int64_t *s,
               int es, Span *out)
{
    int64_t e = d, t;
    const int64_t n[3] = {B, H, T};
    for (int i = 0; i < 3; ++i) {
        if (__builtin_mul_overflow(n[i] - 1, s[i], &t) || __builtin_add_overflow(e, t, &e))
            return false;
    }
    if (__builtin_mul_overflow(e, int64_t{es}, &t))
        return false;
    const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
    *out = Span{lo, lo + static_cast<uintptr_t>(t)};
    return true;
}

// Rows of o (d elements each) are pairwise disjoint when the dimensions,
// ordered by stride, nest: each stride at least the extent of those inside it.
bool attn_rows_disjoint(int64_t B, int64_t H, int64_t T, int64_t d, const int64_t *s)
{
    int64_t n[3] = {B, H, T}, st[3] = {s[0], s[1], s[2]};
    // sort the dimensions by stride (size-1 dimensions never collide)
    for (int i = 0; i < 3; ++i)
        for (int j = i + 1; j < 3; ++j)
            if (st[j] < st[i]) {
                int64_t a = st[i], b = n[i];
                st[i] = st[j], n[i] = n[j];
                st[j] = a, n[j] = b;
            }
    int64_t extent = d;
    for (int i = 0; i < 3; ++i) {
        if (n[i] <= 1)
            continue;
        if (st[i] < extent)
            return false;
        int64_t t;
        if (__builtin_mul_overflow(n[i] - 1, st[i], &t) || __builtin_add_overflow(extent, t, &extent))
            return false;
    }
    return true;
}

}  // namespace

RK_EXPORT rk_status rk_flash_attention(const void *q, const void *k, const void *v, void *o,
                                       int64_t B, int64_t H, int64_t T, int64_t d,
                                       const int64_t *q_strides, const int64_t *k_strides,
                                       const int64_t *v_strides, const int64_t *o_strides,
                                       float scale, int32_t causal, rk_dtype dtype,
                                       hipStream_t stream)
{
    if (dtype != RK_BF16 && dtype != RK_F16 && dtype != RK_F32)
        return RK_ERR_INVALID_ARG;
    if (B < 0 || H < 0 || T < 0 || d < 1 || !std::isfinite(scale) || !(scale > 0.0f) ||
        (causal != 0 && causal != 1))
        return RK_ERR_INVALID_ARG;
    if (B == 0 || H == 0 || T == 0)
        return RK_OK;
    if (q == nullptr || k == nullptr || v == nullptr || o == nullptr)
        return RK_ERR_INVALID_ARG;
    const int64_t dense[3] = {H * T * d, T * d, d};
    if (H > INT64_MAX / T || H * T > INT64_MAX / d || B > INT64_MAX / (H * T * d))
        return RK_ERR_INVALID_ARG;
    const int64_t *st[4] = {q_strides ? q_strides : dense, k_strides ? k_strides : dense,
                            v_strides ? v_strides : dense, o_strides ? o_strides : dense};
    const void *base[4] = {q, k, v, o};
    Span span[4];
    for (int i = 0; i < 4; ++i) {
        if (st[i][0] < 0 || st[i][1] < 0 || st[i][2] < d)
            return RK_ERR_INVALID_ARG;
        if (!attn_span(base[i], B, H, T, d, st[i], 2, &span[i]))
            return RK_ERR_INVALID_ARG;
    }
    for (int i = 0; i < 3; ++i)
        if (overlaps(span[3], span[i]))
            return RK_ERR_INVALID_ARG;
    if (!attn_rows_disjoint(B, H, T, d, st[3]))
        return RK_ERR_INVALID_ARG;
    if (dtype == RK_F32 || (d != 64 && d != 128))
        return RK_ERR_UNSUPPORTED;
    for (int i = 0; i < 4; ++i) {
        if (!aligned16(base[i]) || st[i][0] % 8 || st[i][1] % 8 || st[i][2] % 8)
            return RK_ERR_UNSUPPORTED;
        // the kernel addresses a 64-key block with 32-bit byte offsets
        if (st[i][2] > ((int64_t{1} << 30) - d) / 64)
            return RK_ERR_UNSUPPORTED;
    }
    const int64_t bm = attention_block_rows(d);
    const int64_t nqb = (T + bm - 1) / bm;
    if (T > INT32_MAX || B * H > INT32_MAX || B * H > INT64_MAX / nqb ||
        !grid_ok(B * H * nqb, attention_block_threads(d)))
        return RK_ERR_UNSUPPORTED;
    AttentionProblem p{q, k, v, o, B, H, T, d, {}, {}, {}, {}, scale, causal != 0, dtype, stream};
    for (int j = 0; j < 3; ++j) {
        p.sq[j] = st[0][j];
        p.sk[j] = st[1][j];
        p.sv[j] = st[2][j];
        p.so[j] = st[3][j];
    }
    return hip_status(flash_attention_run(p));
}

RK_EXPORT const char *rk_status_string(rk_status status)
{
    switch (status) {
    case RK_OK:
        return "ok";
    case RK_ERR_INVALID_ARG:
        return "invalid argument";
    case RK_ERR_UNSUPPORTED:
        return "unsupported arguments";
    case RK_ERR_WORKSPACE:
        return "workspace missing or too small";
    case RK_ERR_HIP:
        return "HIP launch failed";
    case RK_ERR_SCRATCH:
        return "split partials exceed the library's fixed 1 MiB scratch";
    }
    return "unknown status";
}

RK_EXPORT int rk_version(void) { return RK_VERSION; }

// --------------------------------------------------------- tuning / probe

RK_EXPORT rk_status rk_probe_copy(const void *src, void *dst, size_t bytes, int32_t max_workgroups,
                                  hipStream_t stream)
{
    if (bytes == 0)
        return RK_OK;
    if (src == nullptr || dst == nullptr || !aligned16(src) || !aligned16(dst) || bytes % 16 != 0)
        return RK_ERR_INVALID_ARG;
    const Span s{reinterpret_cast<uintptr_t>(src), reinterpret_cast<uintptr_t>(src) + bytes};
    const Span d{reinterpret_cast<uintptr_t>(dst), reinterpret_cast<uintptr_t>(dst) + bytes};
    if (overlaps(s, d))
        return RK_ERR_INVALID_ARG;
    return hip_status(probe_copy_run(src, dst, bytes, max_workgroups, stream));
}

RK_EXPORT int32_t rk__variant_count(rk_op op, rk_dtype dtype)
{
    int count = 0;
    variants(op, dtype, &count);
    return count;
}

RK_EXPORT rk_status rk__variant_info(rk_op op, rk_dtype dtype, int32_t index,
                                     int32_t *waves_per_row, int32_t *vecs_per_lane,
                                     int32_t *waves_per_block, int32_t *rows_per_group,
                                     int64_t *max_n, int32_t *exact, int32_t *alternative)
{
    int count = 0;
    const TileVariant *v = variants(op, dtype, &count);
    if (v == nullptr || index < 0 || index >= count)
        return RK_ERR_INVALID_ARG;
    if (waves_per_row)
        *waves_per_row = v[index].waves_per_row;
    if (vecs_per_lane)
        *vecs_per_lane = v[index].vecs_per_lane;
    if (waves_per_block)
        *waves_per_block = v[index].waves_per_block;
    if (rows_per_group)
        *rows_per_group = v[index].rows_per_group;
    if (max_n)
        *max_n = v[index].max_n;
    if (exact)
        *exact = v[index].exact ? 1 : 0;
    if (alternative)
        *alternative = v[index].alternative ? 1 : 0;
    return RK_OK;
}

RK_EXPORT int32_t rk__variant_pick(rk_op op, rk_dtype dtype, int64_t N)
{
    return pick_variant(op, dtype, N);
}

RK_EXPORT rk_status rk__softmax_variant(int32_t index, const void *x, void *y, int64_t M, int64_t N,
                                        int64_t ldx, int64_t ldy, rk_dtype dtype,
                                        hipStream_t stream)
{
    rk_status st = check_rows(x, y, M, N, ldx, ldy, dtype);
    if (st != RK_OK)
        return st;
    int count = 0;
    const TileVariant *v = variants(RK_OP_SOFTMAX, dtype, &count);
    if (index < -1 || index >= count)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const RowProblem p = make_problem(x, y, nullptr, nullptr, M, N, ldx, ldy, 0.0f, dtype, stream);
    const bool aligned = rows_aligned(x, y, ldx, ldy, elem_size(dtype));
    if (index == -1)
        return softmax_generic(p);
    return run_forced(v[index], p, aligned, softmax_vectorized(p));
}

RK_EXPORT rk_status rk__layernorm_gelu_variant(int32_t index, const void *x, const void *weight,
                                               const void *bias, void *y, int64_t M, int64_t N,
                                               int64_t ldx, int64_t ldy, float eps, rk_dtype dtype,
                                               rk_gelu_kind gelu, hipStream_t stream)
{
    rk_status st = check_layernorm(x, weight, bias, y, M, N, ldx, ldy, eps, dtype);
    if (st != RK_OK)
        return st;
    if (!valid_layernorm_act(gelu))
        return RK_ERR_INVALID_ARG;
    int count = 0;
    const TileVariant *v = variants(RK_OP_LAYERNORM_GELU, dtype, &count);
    if (index < -1 || index >= count)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    RowProblem p = make_problem(x, y, weight, bias, M, N, ldx, ldy, eps, dtype, stream);
    p.gelu = gelu;
    const bool aligned = layernorm_aligned(p);
    if (index == -1)
        return layernorm_generic(p);
    return run_forced(v[index], p, aligned, layernorm_vectorized(p));
}

RK_EXPORT rk_status rk__rmsnorm_variant(int32_t index, const void *x, const void *weight, void *y,
                                        int64_t M, int64_t N, int64_t ldx, int64_t ldy, float eps,
                                        rk_dtype dtype, hipStream_t stream)
{
    rk_status st = check_rmsnorm(x, weight, y, M, N, ldx, ldy, eps, dtype);
    if (st != RK_OK)
        return st;
    int count = 0;
    rmsnorm_variants(dtype, false, &count);
    if (index < -1 || index >= count)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    const RowProblem p = make_problem(x, y, weight, nullptr, M, N, ldx, ldy, eps, dtype, stream);
    return rmsnorm_dispatch(p, false, index, true);
}

RK_EXPORT rk_status rk__residual_rmsnorm_variant(int32_t index, const void *x, const void *residual,
                                                 const void *weight, void *y, void *residual_out,
                                                 int64_t M, int64_t N, int64_t ldx, int64_t ldr,
                                                 int64_t ldy, int64_t ldo, float eps,
                                                 rk_dtype dtype, hipStream_t stream)
{
    rk_status st = check_residual_rmsnorm(x, residual, weight, y, residual_out, M, N, ldx, ldr,
                                          ldy, ldo, eps, dtype);
    if (st != RK_OK)
        return st;
    int count = 0;
    rmsnorm_variants(dtype, true, &count);
    if (index < -1 || index >= count)
        return RK_ERR_INVALID_ARG;
    if (M == 0)
        return RK_OK;
    RowProblem p = make_problem(x, y, weight, nullptr, M, N, ldx, ldy, eps, dtype, stream);
    p.r = residual;
    p.ro = residual_out;
    p.ldr = ldr;
    p.ldo = ldo;
    return rmsnorm_dispatch(p, true, index, true);
}
