// Attention forward with the online softmax fused into the value product
// ("Triton Kernel 实现练习" §5.2 "FlashAttention-style Forward"; "第 6 讲：GPU
// Kernels 与 Triton" §7.2-7.3 and §8).
//
// Per (batch, head) and query row i: S_ij = scale q_i . k_j (causal: keys
// j <= i only), o_i = sum_j softmax(S_i)_j v_j.  Key/value blocks are scanned
// with a per-row state m (max so far), l (sum of exp so far) and acc (the
// exp-weighted sum of value rows so far); a new block moves the state by
// alpha = exp(m - m_new): l = alpha l + sum p, acc = alpha acc + p V.  At the
// end o = acc / l.  Scores and probabilities live only in registers.
//
// CDNA4 mapping (16x16x32 MFMA, bf16 or fp16 operands, fp32 accumulation):
//   a workgroup of W waves owns BM = 16 QT W query rows of one (batch, head);
//   each wave owns 16 QT of them as QT 16-row tiles, with its Q fragments in
//   registers for the whole kernel.  Per step of BN = 64 keys the workgroup
//   stages K (row-major) and V (transposed) in LDS; every wave then forms
//   S^T = K Q^T (keys x queries, so that each lane holds one query's scores
//   for 16 of the keys), the row max across the four 16-lane groups
//   (permlane16/32 swaps), p = exp2((S - m) scale log2e), and O^T += V^T P^T,
//   where P^T is the S^T fragments rounded to the operand type in place; the
//   row sum l comes from one more MFMA per 32-key step (A all ones).  K
//   rows are staged in a permuted order (k_slot) that leaves each lane 8
//   consecutive keys per 32-key step, so that its V^T operand is one 16-byte
//   read of the key-ordered V^T.
//   The next block's K/V are loaded into registers while this one is used.
#include "rk_device.h"
#include "rk_internal.h"

namespace rk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4v_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Operand traits: DT = RK_BF16 or RK_F16 (both 16-bit storage).
template <int DT>
struct Operand;

template <>
struct Operand<RK_BF16> {
    typedef bf16x8_t vec;
    __device__ static __forceinline__ f32x4v_t mfma(vec a, vec b, f32x4v_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
    }
    // two fp32 -> two packed 16-bit values, round to nearest even
    __device__ static __forceinline__ uint32_t pack2(float a, float b)
    {
        f32x2_t f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, bf16x2_t));
    }
    // eight 1.0 values (bf16 0x3f80)
    __device__ static __forceinline__ vec ones()
    {
        return __builtin_bit_cast(vec, u32x4_t{0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u});
    }
};

template <>
struct Operand<RK_F16> {
    typedef f16x8_t vec;
    __device__ static __forceinline__ f32x4v_t mfma(vec a, vec b, f32x4v_t c)
    {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack2(float a, float b)
    {
        f32x2_t f = {a, b};
        return __builtin_bit_cast(uint32_t, __builtin_convertvector(f, f16x2_t));
    }
    // eight 1.0 values (fp16 0x3c00)
    __device__ static __forceinline__ vec ones()
    {
        return __builtin_bit_cast(vec, u32x4_t{0x3c003c00u, 0x3c003c00u, 0x3c003c00u, 0x3c003c00u});
    }
};

// Value of lane l and of lane l ^ 16 (in the order even row, odd row of the
// pair of 16-lane rows, identical in both lanes).
__device__ __forceinline__ u32x2_t swap16(float v)
{
    uint32_t u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    return u32x2_t{r[0], r[1]};
}
__device__ __forceinline__ u32x2_t swap32(float v)
{
    uint32_t u = __float_as_uint(v);
    auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    return u32x2_t{r[0], r[1]};
}
// max over the four lanes l, l^16, l^32, l^48 (same bits in all four)
__device__ __forceinline__ float group4_max(float v)
{
    u32x2_t a = swap16(v);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    u32x2_t b = swap32(v);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

constexpr int kAttnBN = 64;  // keys per step

// K and V^T row pitches carry 32 bytes of padding.  Each fragment read is
// one 16-byte ds_read_b128 per lane, lane (g, l16) at row 16 t + l16 and
// 16-byte chunk 4 s + g.  Measured with the hardware's bank-conflict counter
// on gfx950 (a probe issuing only such reads): with 16 bytes of padding
// (272- and 144-byte rows) every such read costs 4 conflict cycles on top of
// its 4, with 32 bytes (288 and 160) none, as for a linear read.
template <int D>
struct AttnLds {
    static constexpr int kKStride = D + 16;        // K row pitch (elements)
    static constexpr int kVStride = kAttnBN + 16;  // V^T row pitch (elements)
    uint16_t k[kAttnBN * kKStride];
    uint16_t vt[D * kVStride];
};

// LDS row of key j (0..63) of a K block.  The S^T tile kt = 2 ks + t reads
// rows 16 kt .. 16 kt + 15 in order, and its row 4 g + r (the rows that lane
// group g's accumulators hold) is key 32 ks + 8 g + 4 t + r: each lane then
// ends with 8 consecutive keys of every 32-key step (4 from each tile), which
// its P^T operand takes in that order, so that V^T, staged in key order,
// gives the matching operand in one 16-byte read.
__device__ __forceinline__ int k_slot(int j)
{
    return 32 * (j / 32) + 16 * ((j % 8) / 4) + 4 * ((j % 32) / 8) + j % 4;
}

// Strides in elements; the head_dim stride is 1.
struct AttnStrides {
    int64_t b, h, t;
};

// W waves per workgroup, each owning QT tiles of 16 query rows.
template <int DT, int D, bool CAUSAL, int W, int QT>
__global__ __launch_bounds__(W *kWave) __attribute__((amdgpu_waves_per_eu(QT == 1 ? 4 : (QT == 2 ? 2 : 1))))
void flash_attention_fwd(
    const uint16_t *__restrict__ q, const uint16_t *__restrict__ k,
    const uint16_t *__restrict__ v, uint16_t *__restrict__ o, int H, int T, int nqb, int BH,
    AttnStrides sq, AttnStrides sk, AttnStrides sv, AttnStrides so, float scale_log2e)
{
    typedef Operand<DT> Op;
    typedef typename Op::vec vec;
    constexpr int DS = D / 32;   // 32-wide d steps of S
    constexpr int DT16 = D / 16; // 16-wide d tiles of O
    constexpr int NKT = kAttnBN / 16;
    constexpr int NKS = kAttnBN / 32;
    constexpr int CH = D / 8;    // 16-byte chunks per K/V row
    constexpr int NT = W * kWave;
    constexpr int BM = 16 * QT * W;  // query rows per workgroup
    constexpr int LOADS = kAttnBN * CH / NT;  // K chunks per thread
    static_assert(LOADS >= 1 && LOADS * NT == kAttnBN * CH, "whole K block per workgroup");
    static_assert(kAttnBN == 64 && (D == 64 || D == 128), "shapes of this kernel");
    // two buffers: block j is read from buffer j % 2 while block j + 1 is
    // written to the other, with one barrier per block
    __shared__ AttnLds<D> lds[2];

    // heaviest query blocks first (causal), and every query block of one
    // (batch, head) on the same XCD when BH is a multiple of 8
    const int rank = static_cast<int>(blockIdx.x) / BH;
    const int bh = static_cast<int>(blockIdx.x) % BH;
    const int qb = nqb - 1 - rank;
    const int b = bh / H, h = bh % H;
    const uint16_t *qh = q + b * sq.b + h * sq.h;
    const uint16_t *kh = k + b * sk.b + h * sk.h;
    const uint16_t *vh = v + b * sv.b + h * sv.h;
    uint16_t *oh = o + b * so.b + h * so.h;

    const int tid = static_cast<int>(threadIdx.x);
    const int wave = tid / kWave;
    const int lane = tid % kWave;
    const int l16 = lane % 16;
    const int g = lane / 16;
    const int q0 = qb * BM;
    const int qw = q0 + 16 * QT * wave;  // first query row of this wave

    // Q fragments (B operand of S^T = K Q^T): query qw + 16 qt + l16,
    // d = 32 ds + 8 g .. + 8.  Rows past T read row T - 1 (never stored).
    vec qf[QT][DS];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        int row = qw + 16 * qt + l16;
        row = row < T ? row : T - 1;
#pragma unroll
        for (int ds = 0; ds < DS; ++ds)
            qf[qt][ds] = *reinterpret_cast<const vec *>(qh + row * sq.t + 32 * ds + 8 * g);
    }

    f32x4v_t acc[QT][DT16];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int dt = 0; dt < DT16; ++dt)
            acc[qt][dt] = f32x4v_t{0.0f, 0.0f, 0.0f, 0.0f};
    // m: the reference max of each query row.  l, the row sum of p, is
    // formed on the matrix cores: one more MFMA per 32-key step, with A all
    // ones and B the step's P^T, sums the rounded p that also weight V, and
    // leaves the whole row's sum in every lane of the query (in element 0,
    // the only one read and rescaled; this replaces a VALU add per score).
    float m[QT];
    f32x4v_t lacc[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        m[qt] = -INFINITY;
        lacc[qt] = f32x4v_t{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const vec ones = Op::ones();

    // K/V staging: K chunk i of this thread is key (tid + 256 i) / CH,
    // column 8 ((tid + 256 i) % CH).  V: keys LOADS kq .. LOADS kq + LOADS - 1
    // at columns 8 cv .. 8 cv + 7, so that the LOADS keys of one column pack
    // into one V^T write; kq runs fastest across the lanes, so that the lanes
    // writing together fill one contiguous V^T row segment (no bank
    // conflicts), while each key row is still read 64 bytes at a time.
    constexpr int NKQ = kAttnBN / LOADS;  // key groups
    u32x4_t kreg[LOADS], vreg[LOADS];
    // byte offsets of this thread's loads from the block's first key row
    // (32-bit: the host keeps 64 seq strides + d below 2^30 elements)
    uint32_t koff[LOADS], voff[LOADS];
    {
        const int kq = tid % NKQ;
        const int cv = tid / NKQ;
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int idx = tid + NT * i;
            koff[i] = static_cast<uint32_t>(((idx / CH) * sk.t + 8 * (idx % CH)) * 2);
            voff[i] = static_cast<uint32_t>(((LOADS * kq + i) * sv.t + 8 * cv) * 2);
        }
    }
    auto load_block = [&](int kb) {
        const int kq = tid % NKQ;
        const int cv = tid / NKQ;  // 0 .. CH - 1
        if (kb + kAttnBN <= T) {  // the whole block is in range: no guards
            const char *kbase = reinterpret_cast<const char *>(kh + kb * sk.t);
            const char *vbase = reinterpret_cast<const char *>(vh + kb * sv.t);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                kreg[i] = *reinterpret_cast<const u32x4_t *>(kbase + koff[i]);
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                vreg[i] = *reinterpret_cast<const u32x4_t *>(vbase + voff[i]);
            return;
        }
        // keys past T: read row T - 1 (in bounds) and zero the data
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int idx = tid + NT * i;
            const int key = kb + idx / CH;
            const u32x4_t val = *reinterpret_cast<const u32x4_t *>(
                kh + (key < T ? key : T - 1) * sk.t + 8 * (idx % CH));
            kreg[i] = key < T ? val : u32x4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int key = kb + LOADS * kq + i;
            const u32x4_t val = *reinterpret_cast<const u32x4_t *>(
                vh + (key < T ? key : T - 1) * sv.t + 8 * cv);
            vreg[i] = key < T ? val : u32x4_t{0, 0, 0, 0};
        }
    };
    auto store_block = [&](AttnLds<D> &buf) {
#pragma unroll
        for (int i = 0; i < LOADS; ++i) {
            const int idx = tid + NT * i;
            *reinterpret_cast<u32x4_t *>(&buf.k[k_slot(idx / CH) * AttnLds<D>::kKStride +
                                                8 * (idx % CH)]) = kreg[i];
        }
        const int kq = tid % NKQ;
        const int cv = tid / NKQ;
        // V^T[d][keys LOADS kq .. + LOADS]: LOADS (= 2 or 4) keys per write
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            uint16_t vals[LOADS];
#pragma unroll
            for (int i = 0; i < LOADS; ++i)
                vals[i] = static_cast<uint16_t>(vreg[i][e / 2] >> (16 * (e % 2)));
            uint16_t *dst = &buf.vt[(8 * cv + e) * AttnLds<D>::kVStride + LOADS * kq];
            if constexpr (LOADS == 4) {
                const uint32_t lo = vals[0] | (uint32_t{vals[1]} << 16);
                const uint32_t hi = vals[2] | (uint32_t{vals[3]} << 16);
                *reinterpret_cast<u32x2_t *>(dst) = u32x2_t{lo, hi};
            } else if constexpr (LOADS == 2) {
                *reinterpret_cast<uint32_t *>(dst) = vals[0] | (uint32_t{vals[1]} << 16);
            } else {
                *dst = vals[0];
            }
        }
    };

    const int kend = CAUSAL ? (q0 + BM < T ? q0 + BM : T) : T;

    // S^T of the block at key kb (K in buf): s[qt][kt] holds, in lane
    // (g, l16), query qw + 16 qt + l16 and keys kb + 32 (kt / 2) + 8 g +
    // 4 (kt % 2) + r (k_slot); keys past T and (causal) keys after the query
    // are masked.
    auto scores = [&](const AttnLds<D> &buf, int kb, f32x4v_t(&s)[QT][NKT]) {
        // The K fragments of d-step ds + 1 are read while the MFMAs of d-step
        // ds run; consecutive MFMAs on one accumulator are NKT * QT apart.
#pragma unroll
        for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
                s[qt][kt] = f32x4v_t{0.0f, 0.0f, 0.0f, 0.0f};
        vec ka[2][NKT];
        auto read_k = [&](int ds, vec(&dst)[NKT]) {
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
                dst[kt] = *reinterpret_cast<const vec *>(
                    &buf.k[(16 * kt + l16) * AttnLds<D>::kKStride + 32 * ds + 8 * g]);
        };
        read_k(0, ka[0]);
#pragma unroll
        for (int ds = 0; ds < DS; ++ds) {
            if (ds + 1 < DS)
                read_k(ds + 1, ka[(ds + 1) & 1]);
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    s[qt][kt] = Op::mfma(ka[ds & 1][kt], qf[qt][ds], s[qt][kt]);
        }

        // mask keys past T and (causal) keys after the query, on the raw
        // scores (scale > 0: the max commutes with it)
        const bool edge = kb + kAttnBN > T || (CAUSAL && kb + kAttnBN - 1 > qw);
        if (edge) {
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                const int qi = qw + 16 * qt + l16;
#pragma unroll
                for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int key = kb + 32 * (kt / 2) + 8 * g + 4 * (kt % 2) + r;
                        if (key >= T || (CAUSAL && key > qi))
                            s[qt][kt][r] = -INFINITY;
                    }
            }
        }

    };

    // The online softmax update of one block: p = exp2(...) into s, the
    // state m, l and acc moved, P^T packed into pk.
    auto softmax_step = [&](f32x4v_t(&s)[QT][NKT], uint32_t(&pk)[QT][NKS][4]) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
            float mx = -INFINITY;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    mx = fmaxf(mx, s[qt][kt][r]);
            // m is the reference max of the row in raw score units, and
            // p = exp(scale (s - m)) = exp2(s c - m c), c = scale log2(e).
            // Softmax does not depend on the reference as long as l and acc
            // share it, so m moves only when this block's max exceeds it by
            // more than 2^8 in p (p stays <= 256, far inside the operand
            // range); a moved m rescales l and acc by alpha.  A row that has
            // seen no key keeps m = -inf (the comparison with NaN is false)
            // and shifts by 0, so that its -inf scores give p = 0.  The row
            // max across its four lanes is formed only when some lane's own
            // max would move m (rare after the first block): otherwise no
            // lane's scores exceed the bound and m stays, the same in all.
            bool bump = false;
            if (__any((mx - m[qt]) * scale_log2e > 8.0f)) {
                mx = group4_max(mx);
                bump = (mx - m[qt]) * scale_log2e > 8.0f;
            }
            const float m_new = bump ? mx : m[qt];
            const float shift = m_new == -INFINITY ? 0.0f : m_new * scale_log2e;
            const float alpha =
                !bump ? 1.0f
                      : (m[qt] == -INFINITY ? 0.0f
                                            : __builtin_amdgcn_exp2f(fmaf(m[qt], scale_log2e, -shift)));
            m[qt] = m_new;
#pragma unroll
            for (int kt = 0; kt < NKT; ++kt)
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    s[qt][kt][r] =
                        __builtin_amdgcn_exp2f(fmaf(s[qt][kt][r], scale_log2e, -shift));
            // rescale the output and l only when some row's reference moved
            if (!__all(alpha == 1.0f)) {
#pragma unroll
                for (int dt = 0; dt < DT16; ++dt)
                    acc[qt][dt] *= alpha;
                lacc[qt][0] *= alpha;
            }
            // 32-key step ks: slots 0..3 are keys 32 ks + 8 g + r (tile 2 ks),
            // slots 4..7 keys 32 ks + 8 g + 4 + r (tile 2 ks + 1)
#pragma unroll
            for (int ks = 0; ks < NKS; ++ks) {
                pk[qt][ks][0] = Op::pack2(s[qt][2 * ks][0], s[qt][2 * ks][1]);
                pk[qt][ks][1] = Op::pack2(s[qt][2 * ks][2], s[qt][2 * ks][3]);
                pk[qt][ks][2] = Op::pack2(s[qt][2 * ks + 1][0], s[qt][2 * ks + 1][1]);
                pk[qt][ks][3] = Op::pack2(s[qt][2 * ks + 1][2], s[qt][2 * ks + 1][3]);
            }
        }

    };

    // O^T += V^T P^T for one block (V^T in buf).
    auto value_step = [&](const AttnLds<D> &buf, const uint32_t(&pk)[QT][NKS][4]) {
        // O^T += V^T P^T: A = V^T rows d = 16 dt + l16 at the lane's 8 keys of
        // the step (one 16-byte read), B = P^T of the lane's query
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks) {
            vec bq[QT];
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) {
                u32x4_t w = {pk[qt][ks][0], pk[qt][ks][1], pk[qt][ks][2], pk[qt][ks][3]};
                bq[qt] = __builtin_bit_cast(vec, w);
                lacc[qt] = Op::mfma(ones, bq[qt], lacc[qt]);  // l += sum of the step's p
            }
            // V^T fragments (keys 32 ks + 8 g .. + 8 of d row 16 dt + l16, one
            // 16-byte read) are read two d-tiles ahead of their MFMAs
            auto read_v = [&](int dt) {
                const uint16_t *row = &buf.vt[(16 * dt + l16) * AttnLds<D>::kVStride + 32 * ks];
                return *reinterpret_cast<const vec *>(row + 8 * g);
            };
            vec va[3];
            va[0] = read_v(0);
            va[1] = read_v(1);
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt) {
                if (dt + 2 < DT16)
                    va[(dt + 2) % 3] = read_v(dt + 2);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt)
                    acc[qt][dt] = Op::mfma(va[dt % 3], bq[qt], acc[qt][dt]);
            }
        }

    };

    load_block(0);
    store_block(lds[0]);
    __syncthreads();

    f32x4v_t s[QT][NKT];
    uint32_t pk[QT][NKS][4];  // P^T operand words
    for (int kb = 0, it = 0; kb < kend; kb += kAttnBN, ++it) {
        const bool more = kb + kAttnBN < kend;
        const AttnLds<D> &cur = lds[it & 1];
        if (more)
            load_block(kb + kAttnBN);
        // causal: a block whose keys all follow this wave's last query row
        // adds nothing (every p would be 0); the wave still stages and waits
        if (!CAUSAL || kb <= qw + 16 * QT - 1) {
            scores(cur, kb, s);
            softmax_step(s, pk);
            value_step(cur, pk);
        }
        // The other buffer was last read in the previous step, which every
        // wave finished before the barrier ending that step.
        if (more)
            store_block(lds[(it + 1) & 1]);
        __syncthreads();  // the next block is visible; this one is free
    }

    // o = acc / l; lane (g, l16) holds query qw + 16 qt + l16, d = 16 dt + 4 g + r
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
        const int qi = qw + 16 * qt + l16;
        const float inv = 1.0f / lacc[qt][0];
        if (qi < T) {
            uint16_t *orow = oh + qi * so.t;
#pragma unroll
            for (int dt = 0; dt < DT16; ++dt) {
                const f32x4v_t a = acc[qt][dt];
                const u32x2_t w = {Op::pack2(a[0] * inv, a[1] * inv), Op::pack2(a[2] * inv, a[3] * inv)};
                *reinterpret_cast<u32x2_t *>(orow + 16 * dt + 4 * g) = w;
            }
        }
    }
}

namespace {

AttnStrides strides_of(const int64_t *s) { return AttnStrides{s[0], s[1], s[2]}; }

// Launch shape by head size: W waves of QT query tiles each (BM = 16 QT W
// query rows per workgroup).  Measured on 4 x 32 x 4096 x 128 bf16: 8 x 2
// (256 rows, two waves per SIMD, one workgroup per CU) 900 TFLOP/s; 4 x 2:
// 845; 8 x 1 (four waves per SIMD, twice the LDS reads per MFMA): 700; 4 x 4
// (one wave per SIMD, spills): 490.  Waves 0-3 and 4-7 run half a step apart
// (one softmax overlapping the other group's MFMAs, two barriers per step):
// the same speed as 8 x 2 in step, so not kept.  With d = 64 the kernel holds
// 142 registers, so 4 x 2 fits three workgroups per CU, whose independent
// steps overlap: 816 against 734 TFLOP/s for 8 x 2 on 4 x 32 x 4096 x 64.
template <int D>
struct AttnShape {
    static constexpr int W = D == 64 ? 4 : 8;
    static constexpr int QT = 2;
    static constexpr int BM = 16 * QT * W;
};

template <int DT, int D, bool CAUSAL>
hipError_t attn_launch(const AttentionProblem &p)
{
    typedef AttnShape<D> S;
    const int nqb = static_cast<int>((p.T + S::BM - 1) / S::BM);
    const int BH = static_cast<int>(p.B * p.H);
    const float scale_log2e = p.scale * 1.4426950408889634f;
    return launch(flash_attention_fwd<DT, D, CAUSAL, S::W, S::QT>,
                  dim3(static_cast<unsigned>(int64_t{nqb} * BH)), dim3(S::W * kWave),
                  p.stream, static_cast<const uint16_t *>(p.q), static_cast<const uint16_t *>(p.k),
                  static_cast<const uint16_t *>(p.v), static_cast<uint16_t *>(p.o),
                  static_cast<int>(p.H), static_cast<int>(p.T), nqb, BH, strides_of(p.sq),
                  strides_of(p.sk), strides_of(p.sv), strides_of(p.so), scale_log2e);
}

template <int DT, int D>
hipError_t attn_causal(const AttentionProblem &p)
{
    return p.causal ? attn_launch<DT, D, true>(p) : attn_launch<DT, D, false>(p);
}

template <int DT>
hipError_t attn_dim(const AttentionProblem &p)
{
    return p.d == 64 ? attn_causal<DT, 64>(p) : attn_causal<DT, 128>(p);
}

}  // namespace

int attention_block_rows(int64_t d) { return d == 64 ? AttnShape<64>::BM : AttnShape<128>::BM; }

int attention_block_threads(int64_t d)
{
    return (d == 64 ? AttnShape<64>::W : AttnShape<128>::W) * kWave;
}

hipError_t flash_attention_run(const AttentionProblem &p)
{
    return p.dtype == RK_BF16 ? attn_dim<RK_BF16>(p) : attn_dim<RK_F16>(p);
}

}  // namespace rk
