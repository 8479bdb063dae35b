// Device-side building blocks shared by the row kernels (gfx950, wave64).
//
//  * 16-byte row vectors: 4 fp32 or 8 bf16 per lane per load/store; a
//    1-element form serves rows whose base or pitch is not 16-byte aligned.
//  * Wave64 reductions: four DPP steps inside each 16-lane row (quad
//    permutes, half-mirror, mirror), after which all 16 lanes of a row hold
//    the row's value, then one permlane32 swap and two readlanes combine the
//    four rows.  Every lane ends with the same bits, and the order of
//    operations is fixed, so results are deterministic run to run.
//  * exp(x - m) in two precisions: a compensated form for fp32 I/O (error a
//    few ulp whatever |x - m|), and a single fma + hardware exp2 for bf16 I/O.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace rk {

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // bf16 storage: the high half of an fp32 word
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// ----------------------------------------------------------------- DPP

// DPP controls (GFX9 encoding).
enum : int {
    kQuadSwap1 = 0xB1,    // quad_perm [1,0,3,2]
    kQuadSwap2 = 0x4E,    // quad_perm [2,3,0,1]
    kRowMirror = 0x140,   // lane i of a 16-lane row reads lane 15-i
    kHalfMirror = 0x141,  // lane i of an 8-lane half-row reads lane 7-i
};

template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    int i = __float_as_int(v);
    return __int_as_float(__builtin_amdgcn_update_dpp(i, i, CTRL, 0xF, 0xF, false));
}

// op(v[l], v[l ^ 32]) in every lane l.  permlane32_swap exchanges the upper
// half of its first operand with the lower half of its second; applied to
// (v, v) it returns two registers that hold, in every lane, v[l] and
// v[l ^ 32] in some order, so a commutative op of the two is the same bits in
// the lane and in its partner.
template <class Op>
__device__ __forceinline__ float combine_halves(float v, Op op)
{
    uint32_t u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return op(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float lane_value(float v, int lane)
{
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return fmaxf(a, b); }
};
struct SumOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// All-lanes reduction of one float over the 64 lanes of a wave.  Must be
// called with every lane of the wave active.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = op(v, dpp<kQuadSwap1>(v));
    v = op(v, dpp<kQuadSwap2>(v));
    v = op(v, dpp<kHalfMirror>(v));
    v = op(v, dpp<kRowMirror>(v));
    // each 16-lane row r now holds its value R_r in all lanes
    v = combine_halves(v, op);
    // lanes 0..15 hold op(R0, R2), lanes 16..31 op(R1, R3): combine lanes 0
    // and 16 as uniform (scalar) values
    float a = lane_value(v, 0), b = lane_value(v, 16);
    return op(a, b);
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp()); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, SumOp()); }

// ----------------------------------------------------------------- exp

// exp(x - m) for fp32 I/O.  The subtraction's rounding error is recovered
// exactly (two-sum), the product with log2(e) is split into a head and a
// tail (fma), and the tail corrects the hardware exp2 of the head to first
// order.  Accuracy: a few ulp for any x - m, not growing with |x - m|.
__device__ __forceinline__ float exp_shifted_accurate(float x, float m)
{
    constexpr float kL = 1.44269502162933349609375f;      // fp32(log2 e)
    constexpr float kLlo = 1.9259629911266175e-08f;      // log2 e - kL
    constexpr float kLn2 = 0.693147180559945309f;
    float d = x - m;
    float bp = d - x;
    float dl = (x - (d - bp)) + (-m - bp);  // d + dl == x - m exactly
    float t = d * kL;
    float tl = fmaf(d, kL, -t) + fmaf(dl, kL, d * kLlo);
    float e = __builtin_amdgcn_exp2f(t);
    float r = fmaf(e, tl * kLn2, e);
    // x = -inf (padding) or an underflowed exp: the tail may be inf/NaN there
    return e == 0.0f ? 0.0f : r;
}

// exp(x - m) for bf16 I/O: exp2(x log2e - m log2e) with one fma.  Relative
// error about |m| * 1e-7, far inside the bf16 tolerance.
__device__ __forceinline__ float exp_shifted_fast(float x, float m_log2e)
{
    constexpr float kL = 1.4426950408889634f;
    return __builtin_amdgcn_exp2f(fmaf(x, kL, -m_log2e));
}

// ------------------------------------------------- online softmax state

// exp(a - b) for a <= b where a may be -inf (then 0): the rescale factor of
// an online softmax state whose max moves from a to b.  The -inf guard keeps
// -inf - (-inf) from being formed.  Evaluated with the accurate exp: it scales
// whole partial sums, so its error is not averaged out.
__device__ __forceinline__ float rescale_factor(float a, float b)
{
    return a == -INFINITY ? 0.0f : exp_shifted_accurate(a, b);
}

// Merge of two partial softmax states (max, sum of exp(x - max)):
// (m1,d1) + (m2,d2) = (M, d1 e^{m1-M} + d2 e^{m2-M}), M = max(m1, m2),
// with (-inf, 0) as identity.  Commutative bit for bit.
struct SoftmaxState {
    float m, d;
};

__device__ __forceinline__ SoftmaxState merge(SoftmaxState a, SoftmaxState b)
{
    float M = fmaxf(a.m, b.m);
    SoftmaxState r;
    r.m = M;
    r.d = a.d * rescale_factor(a.m, M) + b.d * rescale_factor(b.m, M);
    return r;
}

template <int CTRL>
__device__ __forceinline__ SoftmaxState dpp(SoftmaxState s)
{
    return SoftmaxState{dpp<CTRL>(s.m), dpp<CTRL>(s.d)};
}

__device__ __forceinline__ SoftmaxState wave_merge(SoftmaxState s)
{
    s = merge(s, dpp<kQuadSwap1>(s));
    s = merge(s, dpp<kQuadSwap2>(s));
    s = merge(s, dpp<kHalfMirror>(s));
    s = merge(s, dpp<kRowMirror>(s));
    {
        uint32_t um = __float_as_uint(s.m), ud = __float_as_uint(s.d);
        auto rm = __builtin_amdgcn_permlane32_swap(um, um, false, false);
        auto rd = __builtin_amdgcn_permlane32_swap(ud, ud, false, false);
        s = merge(SoftmaxState{__uint_as_float(rm[0]), __uint_as_float(rd[0])},
                  SoftmaxState{__uint_as_float(rm[1]), __uint_as_float(rd[1])});
    }
    SoftmaxState a{lane_value(s.m, 0), lane_value(s.d, 0)};
    SoftmaxState b{lane_value(s.m, 16), lane_value(s.d, 16)};
    return merge(a, b);
}

// --------------------------------------------------------------- GeLU

// tanh-approximation GeLU, 0.5 z (1 + tanh(u)), u = sqrt(2/pi)(z + 0.044715 z^3),
// evaluated as z / (1 + exp(-2u)): the same function, finite for every finite
// z (-> z for z >> 0, -> -0 for z << 0) and without the cancellation of
// 1 + tanh(u) for z < 0.
__device__ __forceinline__ float gelu_tanh(float z)
{
    // -2 sqrt(2/pi) log2(e) and 0.044715 times it, so that
    // exp(-2u) = exp2(z (kA + kB z^2)).
    constexpr float kA = -2.3022081981443248f;
    constexpr float kB = -0.1029432395800235f;
    float z2 = z * z;
    float e = __builtin_amdgcn_exp2f(z * fmaf(z2, kB, kA));
    return z * __builtin_amdgcn_rcpf(1.0f + e);
}

// ------------------------------------------------------ row vectors

template <typename T>
struct Elem;

template <>
struct Elem<float> {
    static constexpr int kVec = 4;  // elements per 16-byte vector
    __device__ static __forceinline__ float to_f32(float v) { return v; }
    __device__ static __forceinline__ float from_f32(float v) { return v; }
};

template <>
struct Elem<bf16_t> {
    static constexpr int kVec = 8;
    __device__ static __forceinline__ float to_f32(bf16_t v)
    {
        return __uint_as_float(static_cast<uint32_t>(v) << 16);
    }
    // round to nearest even (hardware conversion)
    __device__ static __forceinline__ bf16_t from_f32(float v)
    {
        f32x2_t p = {v, 0.0f};
        bf16x2_t q = __builtin_convertvector(p, bf16x2_t);
        return __builtin_bit_cast(uint32_t, q) & 0xFFFFu;
    }
};

// Store E consecutive elements (E is the 16-byte width or 1).
template <typename T, int E>
__device__ __forceinline__ void store_vec(T *__restrict__ p, const float (&v)[E])
{
    if constexpr (E == 1) {
        *p = Elem<T>::from_f32(v[0]);
    } else if constexpr (sizeof(T) == 4) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    } else {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2_t f = {v[2 * i], v[2 * i + 1]};
            w[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
        }
        *reinterpret_cast<uint4 *>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
}

// Row geometry in units of E-element vectors: nfull complete vectors, then
// `tail` (0..E-1) trailing elements that form one partial vector.
template <int E>
struct RowSplit {
    int nfull;
    int tail;
    __device__ __forceinline__ explicit RowSplit(int n) : nfull(n / E), tail(n % E) {}
    __device__ __forceinline__ int count() const { return nfull + (tail ? 1 : 0); }
};

// Raw storage of one E-element vector.
template <typename T, int E>
struct RawVec;
template <>
struct RawVec<float, 4> {
    typedef float4 type;
};
template <>
struct RawVec<float, 1> {
    typedef float type;
};
template <>
struct RawVec<bf16_t, 8> {
    typedef uint4 type;
};
template <>
struct RawVec<bf16_t, 1> {
    typedef bf16_t type;
};

template <typename T, int E>
__device__ __forceinline__ void unpack(const typename RawVec<T, E>::type &q, float (&v)[E])
{
    if constexpr (E == 1) {
        v[0] = Elem<T>::to_f32(q);
    } else if constexpr (sizeof(T) == 4) {
        v[0] = q.x;
        v[1] = q.y;
        v[2] = q.z;
        v[3] = q.w;
    } else {
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float(w[i] << 16);
            v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
        }
    }
}

// Load V vectors of a row: vector k of this lane is vi = vi0 + k * STRIDE.
// Vectors at or beyond `vend` (<= rs.count()) are padded with `pad`; a
// partial last vector loads its `tail` elements and pads the rest.  All
// full-vector loads are issued before any result is used (no wait between
// them); the partial vector is handled behind a branch that is uniform over
// the grid, so rows whose N is a multiple of E never enter it.
template <typename T, int E, int V, int STRIDE>
__device__ __forceinline__ void load_row(const T *__restrict__ row, int vi0, int vend,
                                         RowSplit<E> rs, float pad, float (&v)[V][E])
{
    typedef typename RawVec<T, E>::type R;
    const int lim = vend < rs.nfull ? vend : rs.nfull;
    R q[V];
#pragma unroll
    for (int k = 0; k < V; ++k) {
        q[k] = R{};
        const int vi = vi0 + k * STRIDE;
        if (vi < lim)
            q[k] = *reinterpret_cast<const R *>(row + static_cast<int64_t>(vi) * E);
    }
#pragma unroll
    for (int k = 0; k < V; ++k) {
        unpack<T, E>(q[k], v[k]);
        const bool full = vi0 + k * STRIDE < lim;
#pragma unroll
        for (int e = 0; e < E; ++e)
            v[k][e] = full ? v[k][e] : pad;
    }
    if (rs.tail != 0 && rs.nfull < vend) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int vi = vi0 + k * STRIDE;
            if (vi == rs.nfull) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (e < rs.tail)
                        v[k][e] = Elem<T>::to_f32(row[static_cast<int64_t>(vi) * E + e]);
            }
        }
    }
}

// Store the vectors load_row covered (those below `vend`).
template <typename T, int E, int V, int STRIDE>
__device__ __forceinline__ void store_row(T *__restrict__ row, int vi0, int vend, RowSplit<E> rs,
                                          const float (&v)[V][E])
{
    const int lim = vend < rs.nfull ? vend : rs.nfull;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int vi = vi0 + k * STRIDE;
        if (vi < lim)
            store_vec<T, E>(row + static_cast<int64_t>(vi) * E, v[k]);
    }
    if (rs.tail != 0 && rs.nfull < vend) {
#pragma unroll
        for (int k = 0; k < V; ++k) {
            const int vi = vi0 + k * STRIDE;
            if (vi == rs.nfull) {
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (e < rs.tail)
                        row[static_cast<int64_t>(vi) * E + e] = Elem<T>::from_f32(v[k][e]);
            }
        }
    }
}

}  // namespace rk
