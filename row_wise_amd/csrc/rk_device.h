// Device-side building blocks shared by the row kernels (gfx950, wave64).
//
//  * 16-byte row vectors: 4 fp32 or 8 bf16 per lane per load/store; a
//    1-element form serves rows whose base or pitch is not 16-byte aligned.
//  * Wave64 reductions: four DPP steps inside each 16-lane row (quad
//    permutes, half-mirror, mirror), after which all 16 lanes of a row hold
//    the row's value, then one permlane32 swap and two readlanes combine the
//    four rows.  Every lane ends with the same bits, and the order of
//    operations is fixed, so results are deterministic run to run.
//  * exp(x - m) in two precisions: a compensated form for fp32 I/O, and a
//    single fma + hardware exp2 for bf16 I/O.
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

// All rows and banks enabled and bound_ctrl set: the compiler can fold the
// lane move into the consuming ALU instruction (v_add_f32_dpp and the like).
template <int CTRL>
__device__ __forceinline__ float dpp(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
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

// Maximum that propagates NaN (v_maximum_f32): a NaN anywhere in a row makes
// its max NaN, and with it every output of the row, as the definition says.
__device__ __forceinline__ float nanmax(float a, float b)
{
    return __builtin_elementwise_maximum(a, b);
}

struct MaxOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return nanmax(a, b); }
};
struct SumOp {
    __device__ __forceinline__ float operator()(float a, float b) const { return a + b; }
};

// op over aligned groups of L lanes (L = 4, 8 or 16), the result in every
// lane of the group.  Each step combines a lane with its mirror in the next
// larger group with a commutative op, so every lane of a group ends with the
// same bits.  Must be called with every lane of the wave active.
template <int L, class Op>
__device__ __forceinline__ float group_reduce(float v, Op op)
{
    static_assert(L == 4 || L == 8 || L == 16, "4, 8 or 16 lanes");
    v = op(v, dpp<kQuadSwap1>(v));
    v = op(v, dpp<kQuadSwap2>(v));
    if constexpr (L >= 8)
        v = op(v, dpp<kHalfMirror>(v));
    if constexpr (L >= 16)
        v = op(v, dpp<kRowMirror>(v));
    return v;
}

// All-lanes reduction of one float over the 64 lanes of a wave.  Must be
// called with every lane of the wave active.
template <class Op>
__device__ __forceinline__ float wave_reduce(float v, Op op)
{
    v = group_reduce<16>(v, op);
    // each 16-lane row r now holds its value R_r in all lanes
    v = combine_halves(v, op);
    // lanes 0..15 hold op(R0, R2), lanes 16..31 op(R1, R3): combine lanes 0
    // and 16 as uniform (scalar) values
    float a = lane_value(v, 0), b = lane_value(v, 16);
    return op(a, b);
}

// s_waitcnt vmcnt(0): every vector memory load and store of this wave has
// completed (expcnt and lgkmcnt at their maxima: no wait on them).  vmcnt
// counts loads and stores together, and a row's stores issued while the next
// row's loads are in flight make the next row's first use wait for those
// stores as well; waiting for the loads just before the stores instead (they
// have usually arrived by then) leaves nothing older than the stores to wait
// for.
// The scheduling barrier keeps the work above it (a row's epilogue) above the
// wait, so that the loads have that long to arrive.
__device__ __forceinline__ void wait_vmem()
{
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F70);
}

__device__ __forceinline__ float wave_max(float v) { return wave_reduce(v, MaxOp()); }
__device__ __forceinline__ float wave_sum(float v) { return wave_reduce(v, SumOp()); }

// ----------------------------------------------------------------- exp

// exp(x - m) for fp32 I/O.  d = x - m is formed in fp32 (exact when x and m
// are within a factor of two, e.g. rows offset far from zero); the product
// d log2(e) is split into a head t and a tail (fma), and the tail corrects the
// hardware exp2 of the head to first order.  Relative error about
// |d| * 6e-8 from the rounding of d (<= 2e-6 for |d| <= 30) plus an ulp or
// two, instead of |d| * 1.7e-7 for exp2(d * log2e) alone.
//
// d is clamped at -150 (exp2 of the head is then 0 and the tail finite), so
// that x = -inf (padding) gives 0 without a select.  The clamp maps a NaN d
// to 0 as well; the callers' NaN-propagating row max and the resulting zero
// sum still make every output of such a row NaN.
__device__ __forceinline__ float exp_shifted_accurate(float x, float m)
{
    constexpr float kL = 1.44269502162933349609375f;       // fp32(log2 e)
    constexpr float kLn2 = 0.693147180559945309f;
    constexpr float kLloLn2 = 1.3349758171622139e-08f;     // (log2 e - kL) ln 2
    const float d = fmaxf(x - m, -150.0f);
    const float t = d * kL;
    const float tl = fmaf(fmaf(d, kL, -t), kLn2, d * kLloLn2);  // tail, times ln 2
    const float e = __builtin_amdgcn_exp2f(t);
    return fmaf(e, tl, e);
}

// exp(x - m) as a term of a sum: the shift is formed in fp32 (exact when x and
// m are within a factor of two) and only the product with log2(e) rounds.
// The per-term error (|x - m| * 1.2e-7 relative) has no common part, so it
// averages out in the sum; two fewer operations than the compensated form.
__device__ __forceinline__ float exp_shifted_term(float x, float m)
{
    constexpr float kL = 1.4426950408889634f;
    return __builtin_amdgcn_exp2f((x - m) * kL);
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
    float M = nanmax(a.m, b.m);
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

// Exact GeLU, 0.5 z (1 + erf(z / sqrt 2)), evaluated as 0.5 z erfc(-z / sqrt 2):
// the same function without the cancellation of 1 + erf for z < 0.  erfc is
// the device math library's.
__device__ __forceinline__ float gelu_erf(float z)
{
    constexpr float kRsqrt2 = 0.70710678118654752f;
    return 0.5f * z * erfcf(-z * kRsqrt2);
}

// GeLU by kind: 0 the tanh approximation, 1 the exact erf form, 2 none (the
// LayerNorm epilogue then returns z itself).
template <int GK>
__device__ __forceinline__ float gelu(float z)
{
    if constexpr (GK == 0)
        return gelu_tanh(z);
    else if constexpr (GK == 1)
        return gelu_erf(z);
    else
        return z;
}

// ----------------------------------------------------- LayerNorm moments

// Summary of a part of a row for LayerNorm statistics: count, mean and M2,
// the sum of squared deviations from that mean.  Two summaries of disjoint
// parts combine by the pairwise update of Chan, Golub and LeVeque:
//   n = n1 + n2, delta = mean2 - mean1,
//   mean = mean1 + delta n2 / n,  M2 = M2_1 + M2_2 + delta^2 n1 n2 / n,
// with n = 0 (mean 0, M2 0) as the identity.
struct Moments {
    float n, mean, m2;
};

__device__ __forceinline__ Moments merge(Moments a, Moments b)
{
    const float n = a.n + b.n;
    const float r = b.n * __builtin_amdgcn_rcpf(n);  // share of b
    const float delta = b.mean - a.mean;
    Moments o;
    o.n = n;
    o.mean = fmaf(delta, r, a.mean);
    o.m2 = fmaf(delta * delta, a.n * r, a.m2 + b.m2);
    // exact identities: an empty side returns the other one unchanged
    if (a.n == 0.0f)
        o = b;
    if (b.n == 0.0f)
        o = a;
    return o;
}

template <int CTRL>
__device__ __forceinline__ Moments dpp(Moments s)
{
    return Moments{dpp<CTRL>(s.n), dpp<CTRL>(s.mean), dpp<CTRL>(s.m2)};
}

// Merge of the 64 lanes' summaries of a wave; every lane returns the same
// summary (the merge is not commutative bit for bit, so the wave-wide result
// is taken from lanes 0 and 16 as uniform values).
__device__ __forceinline__ Moments wave_merge(Moments s)
{
    s = merge(s, dpp<kQuadSwap1>(s));
    s = merge(s, dpp<kQuadSwap2>(s));
    s = merge(s, dpp<kHalfMirror>(s));
    s = merge(s, dpp<kRowMirror>(s));
    {
        uint32_t un = __float_as_uint(s.n), um = __float_as_uint(s.mean),
                 uq = __float_as_uint(s.m2);
        auto rn = __builtin_amdgcn_permlane32_swap(un, un, false, false);
        auto rm = __builtin_amdgcn_permlane32_swap(um, um, false, false);
        auto rq = __builtin_amdgcn_permlane32_swap(uq, uq, false, false);
        s = merge(Moments{__uint_as_float(rn[0]), __uint_as_float(rm[0]), __uint_as_float(rq[0])},
                  Moments{__uint_as_float(rn[1]), __uint_as_float(rm[1]), __uint_as_float(rq[1])});
    }
    Moments a{lane_value(s.n, 0), lane_value(s.mean, 0), lane_value(s.m2, 0)};
    Moments b{lane_value(s.n, 16), lane_value(s.mean, 16), lane_value(s.m2, 16)};
    return merge(a, b);
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

// Cache policy of a memory stream.  Row data is touched once per pass, so
// its loads and stores are marked non-temporal ("nt"): they do not displace
// reused lines (weight, bias, partial states) and leave no dirty lines in L2
// to be written back when the kernel ends.
enum CachePolicy { kCached = 0, kStreaming = 1 };

template <int CP, typename R>
__device__ __forceinline__ R ld(const R *p)
{
    if constexpr (CP == kStreaming)
        return __builtin_nontemporal_load(p);
    else
        return *p;
}

template <int CP, typename R>
__device__ __forceinline__ void st(R *p, R v)
{
    if constexpr (CP == kStreaming)
        __builtin_nontemporal_store(v, p);
    else
        *p = v;
}

typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

// Store E consecutive elements (E is the 16-byte width or 1).
template <typename T, int E, int CP>
__device__ __forceinline__ void store_vec(T *__restrict__ p, const float (&v)[E])
{
    if constexpr (E == 1) {
        st<CP>(p, Elem<T>::from_f32(v[0]));
    } else if constexpr (sizeof(T) == 4) {
        const f32x4_t q = {v[0], v[1], v[2], v[3]};
        st<CP>(reinterpret_cast<f32x4_t *>(p), q);
    } else {
        u32x4_t q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            f32x2_t f = {v[2 * i], v[2 * i + 1]};
            q[i] = __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
        }
        st<CP>(reinterpret_cast<u32x4_t *>(p), q);
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
    typedef f32x4_t type;
};
template <>
struct RawVec<float, 1> {
    typedef float type;
};
template <>
struct RawVec<bf16_t, 8> {
    typedef u32x4_t type;
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

// A raw vector whose every element is `pad` (pad must be exact in T).
template <typename T, int E>
__device__ __forceinline__ typename RawVec<T, E>::type raw_splat(float pad)
{
    if constexpr (E == 1) {
        return Elem<T>::from_f32(pad);
    } else if constexpr (sizeof(T) == 4) {
        return f32x4_t{pad, pad, pad, pad};
    } else {
        const uint32_t h = Elem<T>::from_f32(pad);
        const uint32_t w = h | (h << 16);
        return u32x4_t{w, w, w, w};
    }
}

// V vectors of a row in flight: vector k of this lane is vi = vi0 + k * STRIDE.
// issue() starts the loads of the complete vectors below `vend` (<= the row's
// vector count) and leaves the others holding the pad value; it never waits.
// finish() unpacks to fp32 and fills in a partial last vector element by
// element, behind a branch that is uniform over the grid (rows whose N is a
// multiple of E never take it).  Issuing every row's loads before finishing
// any of them keeps all of them in flight at once.
template <typename T, int E, int V, int STRIDE, int CP = kStreaming>
struct RowLoad {
    typedef typename RawVec<T, E>::type R;
    R q[V];
    float tl[E];  // elements of a partial last vector, if this lane holds it
    int vi0, vend;

    __device__ __forceinline__ bool has_tail(RowSplit<E> rs) const
    {
        return rs.tail != 0 && rs.nfull < vend;
    }

    // `full` (uniform over the wave) promises that every vector of every
    // lane is complete and below vend: the loads then need no masks and no
    // padding.
    __device__ __forceinline__ void issue(const T *__restrict__ row, int vi0_, int vend_,
                                          RowSplit<E> rs, float pad, bool full = false)
    {
        vi0 = vi0_;
        vend = full ? 0 : vend_;  // a full load has no partial vector to finish
        if (full) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                q[k] = ld<CP>(reinterpret_cast<const R *>(
                    row + static_cast<int64_t>(vi0 + k * STRIDE) * E));
            return;
        }
        const int lim = vend < rs.nfull ? vend : rs.nfull;
        const R p = raw_splat<T, E>(pad);
#pragma unroll
        for (int k = 0; k < V; ++k) {
            q[k] = p;
            const int vi = vi0 + k * STRIDE;
            if (vi < lim)
                q[k] = ld<CP>(reinterpret_cast<const R *>(row + static_cast<int64_t>(vi) * E));
        }
        // The partial vector is loaded element by element into registers of
        // its own, so that waiting for the full vectors never waits for it.
        if (has_tail(rs)) {
            const int off = rs.nfull - vi0;
            const bool mine = off >= 0 && off % STRIDE == 0 && off / STRIDE < V;
#pragma unroll
            for (int e = 0; e < E; ++e) {
                tl[e] = pad;
                if (mine && e < rs.tail)
                    tl[e] = Elem<T>::to_f32(row[static_cast<int64_t>(rs.nfull) * E + e]);
            }
        }
    }

    // Vector k alone (finish() unpacks all V; this keeps the rest packed).
    __device__ __forceinline__ void finish_one(int k, float (&v)[E], RowSplit<E> rs) const
    {
        unpack<T, E>(q[k], v);
        if (has_tail(rs) && vi0 + k * STRIDE == rs.nfull) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                v[e] = tl[e];
        }
    }

    __device__ __forceinline__ void finish(float (&v)[V][E], RowSplit<E> rs) const
    {
#pragma unroll
        for (int k = 0; k < V; ++k)
            unpack<T, E>(q[k], v[k]);
        if (has_tail(rs)) {
#pragma unroll
            for (int k = 0; k < V; ++k)
                if (vi0 + k * STRIDE == rs.nfull) {
#pragma unroll
                    for (int e = 0; e < E; ++e)
                        v[k][e] = tl[e];
                }
        }
    }
};

// issue + finish in one step (for rows that are used right away).
template <typename T, int E, int V, int STRIDE, int CP = kStreaming>
__device__ __forceinline__ void load_row(const T *__restrict__ row, int vi0, int vend,
                                         RowSplit<E> rs, float pad, float (&v)[V][E],
                                         bool full = false)
{
    RowLoad<T, E, V, STRIDE, CP> l;
    l.issue(row, vi0, vend, rs, pad, full);
    l.finish(v, rs);
}

// Store the vectors load_row covered (those below `vend`; all of them,
// without masks, when `full`).
template <typename T, int E, int V, int STRIDE, int CP = kStreaming>
__device__ __forceinline__ void store_row(T *__restrict__ row, int vi0, int vend, RowSplit<E> rs,
                                          const float (&v)[V][E], bool full = false)
{
    if (full) {
#pragma unroll
        for (int k = 0; k < V; ++k)
            store_vec<T, E, CP>(row + static_cast<int64_t>(vi0 + k * STRIDE) * E, v[k]);
        return;
    }
    const int lim = vend < rs.nfull ? vend : rs.nfull;
#pragma unroll
    for (int k = 0; k < V; ++k) {
        const int vi = vi0 + k * STRIDE;
        if (vi < lim)
            store_vec<T, E, CP>(row + static_cast<int64_t>(vi) * E, v[k]);
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

// ------------------------------------------- rows at any element offset
//
// A row that starts h elements (0 <= h < E) past a 16-byte boundary is read
// and written as the aligned vectors of base = row - h: vector j holds
// columns j*E - h .. j*E - h + E - 1, of which those in [0, N) are the row's.
// Only the first and the last vector can hold other columns.  The load of
// such a vector stays inside a 16-byte block that also holds an element of
// the row, hence inside that element's page, so it cannot fault; its
// outside values are replaced by a pad value, and its stores go element by
// element.  A row whose output (and any other operand read by row) has the
// same phase uses the same vector indices for all of them.
template <int E>
struct RowSpan {
    int h;  // phase: elements from the aligned base to the row's first element
    int n;  // row length

    __device__ __forceinline__ int count() const { return (h + n + E - 1) / E; }
    // vectors [full_begin(), full_end()) hold row elements only
    __device__ __forceinline__ int full_begin() const { return h != 0 ? 1 : 0; }
    __device__ __forceinline__ int full_end() const { return (h + n) / E; }
    __device__ __forceinline__ bool valid(int j, int e) const
    {
        return static_cast<unsigned>(j * E + e - h) < static_cast<unsigned>(n);
    }
    // the step of `span` vectors from `base` holds row elements only and lies
    // below jend: it needs no masks
    __device__ __forceinline__ bool step_full(int base, int jend, int span) const
    {
        const int fe = jend < full_end() ? jend : full_end();
        return base >= full_begin() && base + span <= fe;
    }
};

// Phase of a row's first element.  The same for every lane of a wave (a
// wave works on one row), so it is read into a scalar register.  PH = false
// promises aligned rows: the phase is then the constant 0 and the code that
// handles other phases folds away.
template <typename T, int E, bool PH = true>
__device__ __forceinline__ int row_phase(const T *row)
{
    if constexpr (E == 1 || !PH)
        return 0;
    else
        return __builtin_amdgcn_readfirstlane(
            static_cast<int>((reinterpret_cast<uintptr_t>(row) % 16) / sizeof(T)));
}

// Vector range [jbeg, jend) of chunk s of S when a row is split into chunks
// of C phased positions (C a multiple of E): positions [s C, s C + C), the
// last chunk running to the row's end.
template <int E>
__device__ __forceinline__ void chunk_span(RowSpan<E> sp, int s, int S, int C, int &jbeg,
                                           int &jend)
{
    const int nv = sp.count();
    const int64_t c0 = static_cast<int64_t>(s) * C;
    const int64_t len = static_cast<int64_t>(sp.h) + sp.n;
    jbeg = static_cast<int>(c0 < len ? c0 / E : nv);
    jend = static_cast<int>(s == S - 1 || c0 + C >= len ? nv : (c0 + C) / E);
}

// A row's split partials (two floats each): at the first 8-byte boundary of
// base + row * row_bytes (a workspace keeps them 8-byte aligned already).
__device__ __forceinline__ float2 *row_partials(char *base, int64_t row_bytes, int64_t row)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(base + row * row_bytes);
    return reinterpret_cast<float2 *>((a + 7) & ~uintptr_t{7});
}

__device__ __forceinline__ const float2 *row_partials(const char *base, int64_t row_bytes,
                                                      int64_t row)
{
    return row_partials(const_cast<char *>(base), row_bytes, row);
}

// What a split-row output kernel writes: every chunk; every chunk but the
// first vectors of the first chunk, which hold the partials kept in the
// output; or only those first vectors (one workgroup per row, after every
// wave has read the partials).
enum SplitPart { kAllChunks = 0, kAllButFirst = 1, kFirstOnly = 2 };

// The vectors [0, P) of a row (at phase sp.h from its aligned base) that
// hold the S partials kept in the output row yrow (at its first 8-byte
// boundary, as row_partials places them).
template <typename T, int E>
__device__ __forceinline__ int partials_prefix(const T *yrow, RowSpan<E> sp, int S)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(yrow);
    const int pad = static_cast<int>(((a + 7) & ~uintptr_t{7}) - a);
    constexpr int vb = E * static_cast<int>(sizeof(T));
    return (sp.h * static_cast<int>(sizeof(T)) + pad + 8 * S + vb - 1) / vb;
}

// The vector range a split-row output kernel writes for chunk s of a row:
// [jbeg, jend) of the chunk, less (kAllButFirst) or only (kFirstOnly) the
// first chunk's partials prefix.
template <typename T, int E>
__device__ __forceinline__ void output_range(int part, int s, const T *yrow, RowSpan<E> sp, int S,
                                             int &jbeg, int &jend)
{
    if (part == kAllChunks || s != 0)
        return;
    int pre = partials_prefix<T, E>(yrow, sp, S);
    pre = pre < jend ? pre : jend;
    if (part == kFirstOnly)
        jend = pre;
    else
        jbeg = pre;
}

// U vectors of a row in flight: vector k of this lane is j0 + k * STRIDE.
// issue() starts the loads of the vectors below jend (all of them, unmasked,
// when `full`) and never waits; finish() unpacks to fp32 and replaces
// elements outside the row or at or past jend by `pad`.
template <typename T, int E, int U, int STRIDE, int CP = kStreaming>
struct SpanLoad {
    typedef typename RawVec<T, E>::type R;
    R q[U];
    int j0;

    __device__ __forceinline__ void issue(const T *__restrict__ base, int j0_, int jend, bool full)
    {
        j0 = j0_;
#pragma unroll
        for (int k = 0; k < U; ++k) {
            const int j = j0 + k * STRIDE;
            if (full) {
                q[k] = ld<CP>(reinterpret_cast<const R *>(base + static_cast<int64_t>(j) * E));
            } else {
                q[k] = R{};
                if (j < jend)
                    q[k] = ld<CP>(reinterpret_cast<const R *>(base + static_cast<int64_t>(j) * E));
            }
        }
    }

    __device__ __forceinline__ void finish(float (&v)[U][E], RowSpan<E> sp, int jend, float pad,
                                           bool full) const
    {
#pragma unroll
        for (int k = 0; k < U; ++k)
            unpack<T, E>(q[k], v[k]);
        if (!full) {
#pragma unroll
            for (int k = 0; k < U; ++k) {
                const int j = j0 + k * STRIDE;
#pragma unroll
                for (int e = 0; e < E; ++e)
                    if (!(j < jend && sp.valid(j, e)))
                        v[k][e] = pad;
            }
        }
    }
};

// Store the row elements of the vectors a SpanLoad covered below jend.
template <typename T, int E, int U, int STRIDE, int CP = kStreaming>
__device__ __forceinline__ void store_span(T *__restrict__ base, int j0, int jend, RowSpan<E> sp,
                                           const float (&v)[U][E], bool full)
{
    if (full) {
#pragma unroll
        for (int k = 0; k < U; ++k)
            store_vec<T, E, CP>(base + static_cast<int64_t>(j0 + k * STRIDE) * E, v[k]);
        return;
    }
    const int fb = sp.full_begin();
    const int fe = sp.full_end();
#pragma unroll
    for (int k = 0; k < U; ++k) {
        const int j = j0 + k * STRIDE;
        if (j >= jend)
            continue;
        if (j >= fb && j < fe) {
            store_vec<T, E, CP>(base + static_cast<int64_t>(j) * E, v[k]);
        } else {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (sp.valid(j, e))
                    base[static_cast<int64_t>(j) * E + e] = Elem<T>::from_f32(v[k][e]);
        }
    }
}

// out = the E elements that start H elements before hi[0]: the last H of lo,
// then the first E - H of hi (H < E; other H never occur and copy hi).
template <int H, int E>
__device__ __forceinline__ void shift_in(const float (&lo)[E], const float (&hi)[E],
                                         float (&out)[E])
{
    if constexpr (H > 0 && H < E) {
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = e < H ? lo[E - H + e] : hi[e - H];
    } else {
#pragma unroll
        for (int e = 0; e < E; ++e)
            out[e] = hi[e];
    }
}

// The E elements of a per-column parameter p[n] (16-byte aligned, cached)
// that meet vector j of a row at phase h: p[j*E - h + e], 0 outside [0, n).
// Two aligned loads straddle the shift; each reads a 16-byte block that
// holds an element of p.  issue() starts the loads, finish() waits, unpacks
// and shifts.  `full` promises that vector j holds row elements only: no
// checks then.
template <typename T, int E>
struct ParamLoad {
    typedef typename RawVec<T, E>::type R;
    R qh, ql;

    // The block at column j*E and the one before it.  A block is read only
    // if it holds an element of p: lanes of a masked step may sit past the
    // row.
    __device__ __forceinline__ void issue(const T *__restrict__ p, int j, int h, int n, bool full)
    {
        const R *pv = reinterpret_cast<const R *>(p);
        qh = R{};
        ql = R{};
        if (full || j * E < n)
            qh = pv[j];
        if (h != 0 && (full || (j >= 1 && (j - 1) * E < n)))
            ql = pv[j - 1];
    }

    __device__ __forceinline__ void finish(float (&out)[E], int j, int h, int n, bool full) const
    {
        float hi[E], lo[E];
        unpack<T, E>(qh, hi);
        unpack<T, E>(ql, lo);
        // element e comes from lo[E - h + e] (e < h) or hi[e - h]; h is
        // uniform over the wave, so one case runs
        switch (h) {
        case 1:
            shift_in<1>(lo, hi, out);
            break;
        case 2:
            shift_in<2>(lo, hi, out);
            break;
        case 3:
            shift_in<3>(lo, hi, out);
            break;
        case 4:
            shift_in<4>(lo, hi, out);
            break;
        case 5:
            shift_in<5>(lo, hi, out);
            break;
        case 6:
            shift_in<6>(lo, hi, out);
            break;
        case 7:
            shift_in<7>(lo, hi, out);
            break;
        default:
            shift_in<0>(lo, hi, out);
            break;
        }
        // columns outside [0, n) read as 0 (the elements of a block that are
        // not p's, or a block that was not loaded)
        if (!full) {
#pragma unroll
            for (int e = 0; e < E; ++e)
                if (static_cast<unsigned>(j * E + e - h) >= static_cast<unsigned>(n))
                    out[e] = 0.0f;
        }
    }
};

template <typename T, int E>
__device__ __forceinline__ void load_param(const T *__restrict__ p, int j, int h, int n,
                                           float (&out)[E], bool full)
{
    ParamLoad<T, E> l;
    l.issue(p, j, h, n, full);
    l.finish(out, j, h, n, full);
}

}  // namespace rk
