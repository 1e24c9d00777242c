// Exact indexer dot products on gfx950.
//
// The indexer score is the exact dot product of the indexer query and key,
// rounded once to fp32. Four lanes (a "quad") share one key row: each lane
// loads a contiguous quarter of the row with 16-byte loads (so a wave reads
// 16 whole rows as one contiguous span) and widens its elements to fp64.
//
// Two accumulators, chosen by the element types:
//  * bf16 query x E4M3 key (the decode path): products have at most 12
//    significant bits and are multiples of u = 2^(e_min - 16), e_min being the
//    smallest exponent of a nonzero query element; their magnitudes stay below
//    2^(e_max + 16). Plain fp64 FMAs are therefore exact - in any order,
//    including the cross-lane combine - whenever the query's nonzero elements
//    span at most 2^21 in magnitude (e_max - e_min <= 21).
//  * every other pair (an fp32 query or key, bf16 x bf16): products have up to
//    48 significant bits, so a plain fp64 sum can round. These accumulate as a
//    double-double (hi, lo): every add of hi is an error-free TwoSum whose
//    rounding error goes to lo. All terms, sums and errors are multiples of u
//    (the product of the two smallest element units), and the errors add up to
//    at most 2^-47 of the sum of |products|, so lo stays exact - and hi + lo is
//    the exact dot product - whenever that sum is below 2^100 u, i.e. whenever
//    the exponents of the query's and the key's nonzero elements together span
//    less than about 46 binades. The exact value is then rounded once to fp32
//    by round-to-odd into fp64 followed by round-to-nearest-even into fp32
//    (53 >= 24 + 2 bits, so the double rounding is innocuous).
#pragma once

#include "device.hpp"

namespace csa2 {

enum : int { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

template <int KT> struct ElemBytes;
template <> struct ElemBytes<kF32> { static constexpr int v = 4; };
template <> struct ElemBytes<kBF16> { static constexpr int v = 2; };
template <> struct ElemBytes<kE4M3> { static constexpr int v = 1; };

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Double-double partial sum (see above): hi + lo is the exact sum of the terms.
struct DD {
    double hi, lo;
};

// Error-free sum: s + e == a + b exactly, s = fl(a + b).
__device__ __forceinline__ void two_sum(double a, double b, double& s, double& e) {
    s = a + b;
    const double bb = s - a;
    e = (a - (s - bb)) + (b - bb);
}

__device__ __forceinline__ DD dd_add(DD a, double b) {
    double s, e;
    two_sum(a.hi, b, s, e);
    return DD{s, a.lo + e};
}

__device__ __forceinline__ DD operator+(DD a, DD b) {
    double s, e;
    two_sum(a.hi, b.hi, s, e);
    return DD{s, a.lo + b.lo + e};
}

// fp32 nearest-even of an exact fp64 sum.
__device__ __forceinline__ float round_score(double v) { return (float)v; }

// fp32 nearest-even of the exact value hi + lo: renormalize, round to odd in
// fp64 (truncate toward zero, then force the last bit to 1 when inexact), then
// round to fp32.
__device__ __forceinline__ float round_score(DD v) {
    double s, e;
    two_sum(v.hi, v.lo, s, e);
    if (e == 0.0) return (float)s;
    uint64_t u = (uint64_t)__double_as_longlong(s);
    if ((e < 0.0) != (s < 0.0)) u -= 1u;       // |s + e| < |s|: truncation is one ulp toward zero
    return (float)__longlong_as_double((long long)(u | 1u));
}

// Accumulator of a (key type, query type) pair: plain fp64 for bf16 x E4M3,
// double-double otherwise.
template <int KT, int QT> struct AccOf { using type = DD; };
template <> struct AccOf<kE4M3, kBF16> { using type = double; };

__device__ __forceinline__ double acc_zero(double*) { return 0.0; }
__device__ __forceinline__ DD acc_zero(DD*) { return DD{0.0, 0.0}; }
__device__ __forceinline__ double acc_fma(double acc, double a, double b) { return fma(a, b, acc); }
__device__ __forceinline__ DD acc_fma(DD acc, double a, double b) { return dd_add(acc, a * b); }

// Per-lane slice of one key row: PER elements, RAW 16-byte words. dot()
// returns this lane's partial sum in the pair's accumulator type.
template <int KT, int D, int QT = kBF16>
struct KeySlice {
    using Part = typename AccOf<KT, QT>::type;
    static constexpr int PER = D / 4;
    static constexpr int ROW_BYTES = D * ElemBytes<KT>::v;
    static constexpr int RAW = PER * ElemBytes<KT>::v / 16;
    uint4 raw[RAW];

    __device__ __forceinline__ void load(const uint8_t* row, int lq) {
        const uint8_t* p = row + lq * (ROW_BYTES / 4);
#pragma unroll
        for (int j = 0; j < RAW; ++j) raw[j] = ld_stream16(p + 16 * j);
    }

    __device__ __forceinline__ Part dot(const double (&q)[PER]) const {
        Part acc = acc_zero((Part*)nullptr);
        const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
        if constexpr (KT == kE4M3) {
#pragma unroll
            for (int i = 0; i < PER / 4; ++i) {
                const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                acc = acc_fma(acc, (double)a.x, q[4 * i + 0]);
                acc = acc_fma(acc, (double)a.y, q[4 * i + 1]);
                acc = acc_fma(acc, (double)b.x, q[4 * i + 2]);
                acc = acc_fma(acc, (double)b.y, q[4 * i + 3]);
            }
        } else if constexpr (KT == kBF16) {
#pragma unroll
            for (int i = 0; i < PER / 2; ++i) {
                acc = acc_fma(acc, (double)__uint_as_float(w[i] << 16), q[2 * i + 0]);
                acc = acc_fma(acc, (double)__uint_as_float(w[i] & 0xFFFF0000u), q[2 * i + 1]);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) acc = acc_fma(acc, (double)__uint_as_float(w[i]), q[i]);
        }
        return acc;
    }
};

// Load this lane's quarter of the indexer query as fp64.
template <int QT, int D>
__device__ __forceinline__ void load_query_slice(const void* q_row, int lq, double (&q)[D / 4]) {
    constexpr int PER = D / 4;
    if constexpr (QT == kBF16) {
        const uint16_t* p = reinterpret_cast<const uint16_t*>(q_row) + lq * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) q[i] = (double)bf16_bits_to_f32(p[i]);
    } else {
        const float* p = reinterpret_cast<const float*>(q_row) + lq * PER;
#pragma unroll
        for (int i = 0; i < PER; ++i) q[i] = (double)p[i];
    }
}

// Sum over the 4 lanes of a quad (lanes 4j..4j+3); every lane gets the total.
__device__ __forceinline__ double quad_sum(double v) {
    v += shfl_xor_f64(v, 1);
    v += shfl_xor_f64(v, 2);
    return v;
}

__device__ __forceinline__ DD quad_sum(DD v) {
    v = v + DD{shfl_xor_f64(v.hi, 1), shfl_xor_f64(v.lo, 1)};
    v = v + DD{shfl_xor_f64(v.hi, 2), shfl_xor_f64(v.lo, 2)};
    return v;
}

// fp64 value of the quad lane named by the DPP quad permutation CTRL.
template <int CTRL>
__device__ __forceinline__ double quad_perm_f64(double v) {
    const int2 p = __builtin_bit_cast(int2, v);
    int2 r;
    r.x = __builtin_amdgcn_mov_dpp(p.x, CTRL, 0xF, 0xF, false);
    r.y = __builtin_amdgcn_mov_dpp(p.y, CTRL, 0xF, 0xF, false);
    return __builtin_bit_cast(double, r);
}

// Transposed quad reduction: lane lq (0..3) of a quad holds partial sums
// acc[0..3] of four keys; it returns the sum over the quad of key lq. Step 1
// exchanges with lane lq ^ 1 (each lane keeps the keys whose bit 0 is its
// own), step 2 with lane lq ^ 2; 6 cross-lane moves instead of 16.
__device__ __forceinline__ double quad_transpose_sum(const double (&acc)[4], int lq) {
    constexpr int kXor1 = 0xB1;                 // quad_perm [1, 0, 3, 2]
    constexpr int kXor2 = 0x4E;                 // quad_perm [2, 3, 0, 1]
    const bool b0 = lq & 1, b1 = lq & 2;
    const double t0 = (b0 ? acc[1] : acc[0]) + quad_perm_f64<kXor1>(b0 ? acc[0] : acc[1]);   // key b0
    const double t1 = (b0 ? acc[3] : acc[2]) + quad_perm_f64<kXor1>(b0 ? acc[2] : acc[3]);   // key 2 + b0
    return (b1 ? t1 : t0) + quad_perm_f64<kXor2>(b1 ? t0 : t1);
}

template <int CTRL>
__device__ __forceinline__ DD quad_perm_dd(DD v) {
    return DD{quad_perm_f64<CTRL>(v.hi), quad_perm_f64<CTRL>(v.lo)};
}

// The transposed quad reduction of double-double partial sums.
__device__ __forceinline__ DD quad_transpose_sum(const DD (&acc)[4], int lq) {
    constexpr int kXor1 = 0xB1;
    constexpr int kXor2 = 0x4E;
    const bool b0 = lq & 1, b1 = lq & 2;
    const DD t0 = (b0 ? acc[1] : acc[0]) + quad_perm_dd<kXor1>(b0 ? acc[0] : acc[1]);
    const DD t1 = (b0 ? acc[3] : acc[2]) + quad_perm_dd<kXor1>(b0 ? acc[2] : acc[3]);
    return (b1 ? t1 : t0) + quad_perm_dd<kXor2>(b1 ? t0 : t1);
}

}  // namespace csa2
