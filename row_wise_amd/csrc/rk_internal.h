// Host-side glue shared by the kernel translation units and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <tuple>
#include <utility>

#include "rowkern.h"
#include "rowkern_tune.h"

#define RK_EXPORT extern "C" __attribute__((visibility("default")))

namespace rk {

// Launch a kernel through hipLaunchKernel so that the status of this launch
// (not a stale error of an earlier call) is returned.  Arguments are
// converted to the kernel's exact parameter types.
template <typename... KArgs, typename... Args>
inline hipError_t launch(void (*kernel)(KArgs...), dim3 grid, dim3 block, hipStream_t stream,
                         Args... args)
{
    static_assert(sizeof...(KArgs) == sizeof...(Args), "argument count");
    std::tuple<KArgs...> vals(static_cast<KArgs>(args)...);
    void *argv[sizeof...(KArgs)];
    std::apply(
        [&](auto &...v) {
            int i = 0;
            ((argv[i++] = static_cast<void *>(&v)), ...);
        },
        vals);
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), grid, block, argv, 0, stream);
}

// One row-wise problem as validated by the ABI layer.
struct RowProblem {
    const void *x;
    void *y;
    const void *w;  // normalizations: weight
    const void *b;  // LayerNorm: bias
    int64_t M;
    int N;
    int64_t ldx, ldy;
    float eps;  // normalizations
    rk_dtype dtype;
    hipStream_t stream;
    const void *r = nullptr;  // residual RMSNorm: residual input
    void *ro = nullptr;       // residual RMSNorm: residual output
    int64_t ldr = 0, ldo = 0;
    rk_gelu_kind gelu = RK_GELU_TANH;  // LayerNorm, GeLU: activation
};

// One attention problem as validated by the ABI layer: q, k, v, o of shape
// [B][H][T][d] with element strides (batch, head, seq) and unit d stride.
struct AttentionProblem {
    const void *q, *k, *v;
    void *o;
    int64_t B, H, T, d;
    int64_t sq[3], sk[3], sv[3], so[3];
    float scale;
    bool causal;
    rk_dtype dtype;
    hipStream_t stream;
};

// A compiled register-resident kernel shape.
struct TileVariant {
    int waves_per_row;    // G: waves cooperating on a row
    int vecs_per_lane;    // V: 16-byte vectors per lane
    int waves_per_block;  // W: waves per workgroup (W / G row groups)
    int rows_per_group;   // R: rows each row group handles in sequence
    int max_n;            // largest N the variant holds
    bool exact;           // compiled for N == max_n only: no masks, no padding
    hipError_t (*run)(const RowProblem &);
    bool alternative = false;  // reachable by index only, never dispatched
    // The same tile for rows at any offset past a 16-byte boundary (shared
    // by the row's input and output): general, one row per row group; a row
    // at offset h takes h + N register slots.  Null where not compiled.
    hipError_t (*run_phased)(const RowProblem &) = nullptr;

    bool accepts(int64_t n) const { return exact ? n == max_n : n <= max_n; }
    // every offset h < vec fits
    bool accepts_phased(int64_t n, int vec) const
    {
        return run_phased != nullptr && n + vec - 1 <= max_n;
    }
};

// Marks a table entry as an alternative: run by index (tuning, tests), never
// chosen by the dispatcher.
constexpr TileVariant alt(TileVariant v)
{
    v.alternative = true;
    return v;
}

// Variant tables (defined next to the kernels), in order of preference: the
// dispatcher takes the first exact variant with max_n == N, else the first
// general variant whose max_n covers N, skipping alternatives.  An N that no
// dispatched entry takes goes to the kernels that keep the row in memory.
const TileVariant *softmax_variants(rk_dtype dtype, int *count);
const TileVariant *layernorm_gelu_variants(rk_dtype dtype, int *count);
const TileVariant *rmsnorm_variants(rk_dtype dtype, bool residual, int *count);

// How the kernels that keep rows in memory access them: aligned 16-byte
// vectors (every row starts on a 16-byte boundary), aligned vectors from each
// row's own offset (rows and outputs share their offsets; RowSpan), or one
// element at a time.
enum RowIo { kIoElement = 0, kIoAligned = 1, kIoPhased = 2 };

// Where the split-row kernels keep each row's S partials (two floats each):
// a caller's workspace (row r at base + r row_bytes, 8-byte aligned, S * 8
// bytes apart), or the row's own output (the first 8-byte boundary of output
// row r, inside the row's first chunk).  In the output, the second kernel
// writes every chunk but the first, and a third kernel, one workgroup per
// row, reads the partials and then writes the first chunk over them.
struct SplitPartials {
    char *base;
    int64_t row_bytes;
    bool in_output;
};

// Generic paths (any alignment, any N).
hipError_t online_stream_run(const RowProblem &p, RowIo io);
hipError_t online_split_run(const RowProblem &p, int splits, int chunk, SplitPartials parts,
                            RowIo io);
hipError_t layernorm_stream_run(const RowProblem &p, RowIo io);
hipError_t layernorm_split_run(const RowProblem &p, int splits, int chunk, SplitPartials parts,
                               RowIo io);
hipError_t rmsnorm_loop_run(const RowProblem &p, bool residual, RowIo io);
hipError_t rmsnorm_split_run(const RowProblem &p, bool residual, int splits, int chunk,
                             SplitPartials parts, RowIo io);
enum { RK_REDUCE_SUM = 0, RK_REDUCE_MAX = 1 };
hipError_t row_reduce_run(const RowProblem &p, int op);
// Workgroups (and threads per workgroup) row_reduce_run launches.
int64_t row_reduce_blocks(int64_t M, int64_t N, rk_dtype dtype, int *threads);
// Split form: M * splits workgroups of 256 threads write one float per
// (row, chunk) to part ([M][splits]), then ceil(M / 4) workgroups reduce
// each row's partials into out.  chunk: elements per chunk, a multiple of
// the vector width.
hipError_t row_reduce_split_run(const RowProblem &p, int op, int splits, int chunk, float *part);
// flat: x and y contiguous and 16-byte aligned, processed as one buffer.
hipError_t gelu_run(const RowProblem &p, bool flat, RowIo io);
// Query rows and threads per workgroup of the attention kernel for head
// size d.
int attention_block_rows(int64_t d);
int attention_block_threads(int64_t d);
hipError_t flash_attention_run(const AttentionProblem &p);
hipError_t probe_copy_run(const void *src, void *dst, size_t bytes, int max_wg,
                          hipStream_t stream);

// Bytes of the fixed device scratch (rk_scratch.hip) that the allocation-free
// entry point keeps its split partials in: 1 MiB, 131072 (m, d) pairs.
constexpr size_t kScratchBytes = size_t{1} << 20;
// Device address of the scratch on `device`, which must be the current
// device; looked up once per device and kept.
hipError_t scratch_address(int device, void **address);

inline int elem_size(rk_dtype dt) { return dt == RK_F32 ? 4 : 2; }
inline int vec_elems(rk_dtype dt) { return 16 / elem_size(dt); }

// Waves per workgroup of a one-workgroup-per-row streaming kernel for a row of
// nvec vectors processed U per thread per step: the largest of 16, 4 and 1
// that still gives every thread at least two steps, so that short rows do
// not leave most of a 1024-thread workgroup idle.
inline int stream_waves(int64_t nvec, int U)
{
    if (nvec >= int64_t{16} * 64 * U * 2)
        return 16;
    if (nvec >= int64_t{4} * 64 * U * 2)
        return 4;
    return 1;
}

// Rows of at most this many vectors take one wave and one vector per lane
// per step: with U vectors per step, most of a short row's step would be
// masked padding.
constexpr int64_t kShortRowVectors = 128;

// First vector of the last step of [jbeg, jend) (steps of `span` vectors from
// jbeg), or jbeg - span for an empty range.  The softmax and RMSNorm output
// passes run their steps from there down to jbeg: the end of a range, read
// last by the pass before, is the part most likely still in the caches.
constexpr int last_step(int jbeg, int jend, int span)
{
    return jend > jbeg ? jbeg + (jend - jbeg - 1) / span * span : jbeg - span;
}

// Chunk length (elements) of the split-row variant: ceil(N / S) rounded up to
// whole 16-byte vectors when the vector path is used.
inline int64_t split_chunk(int64_t N, int64_t S, int vec)
{
    int64_t c = (N + S - 1) / S;
    return (c + vec - 1) / vec * vec;
}

}  // namespace rk
