// Exact indexer dot products on gfx950.
//
// The indexer score is the exact dot product of the indexer query and key,
// rounded once to fp32. Four lanes (a "quad") share one key row: each lane
// loads a contiguous quarter of the row with 16-byte loads (so a wave reads
// 16 whole rows as one contiguous span), widens its elements to fp64 and
// accumulates q*k with fp64 FMAs. Every product of a bf16/fp32 query element
// and an E4M3/bf16/fp32 key element is exact in fp64 (at most 48 significant
// bits), so the fp64 sum - in any order, including the cross-lane combine -
// is the exact sum whenever the terms fit one 2^53-wide window; rounding that
// to fp32 gives the same value on every order of evaluation.
#pragma once

#include "device.hpp"

namespace csa2 {

enum : int { kF32 = 0, kBF16 = 1, kE4M3 = 2 };

template <int KT> struct ElemBytes;
template <> struct ElemBytes<kF32> { static constexpr int v = 4; };
template <> struct ElemBytes<kBF16> { static constexpr int v = 2; };
template <> struct ElemBytes<kE4M3> { static constexpr int v = 1; };

typedef float f32x2 __attribute__((ext_vector_type(2)));

// Per-lane slice of one key row: PER elements, RAW 16-byte words.
template <int KT, int D>
struct KeySlice {
    static constexpr int PER = D / 4;
    static constexpr int ROW_BYTES = D * ElemBytes<KT>::v;
    static constexpr int RAW = PER * ElemBytes<KT>::v / 16;
    uint4 raw[RAW];

    __device__ __forceinline__ void load(const uint8_t* row, int lq) {
        const uint8_t* p = row + lq * (ROW_BYTES / 4);
#pragma unroll
        for (int j = 0; j < RAW; ++j) raw[j] = ld_stream16(p + 16 * j);
    }

    __device__ __forceinline__ double dot(const double (&q)[PER]) const {
        double acc = 0.0;
        const uint32_t* w = reinterpret_cast<const uint32_t*>(raw);
        if constexpr (KT == kE4M3) {
#pragma unroll
            for (int i = 0; i < PER / 4; ++i) {
                const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
                const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
                acc = fma((double)a.x, q[4 * i + 0], acc);
                acc = fma((double)a.y, q[4 * i + 1], acc);
                acc = fma((double)b.x, q[4 * i + 2], acc);
                acc = fma((double)b.y, q[4 * i + 3], acc);
            }
        } else if constexpr (KT == kBF16) {
#pragma unroll
            for (int i = 0; i < PER / 2; ++i) {
                acc = fma((double)__uint_as_float(w[i] << 16), q[2 * i + 0], acc);
                acc = fma((double)__uint_as_float(w[i] & 0xFFFF0000u), q[2 * i + 1], acc);
            }
        } else {
#pragma unroll
            for (int i = 0; i < PER; ++i) acc = fma((double)__uint_as_float(w[i]), q[i], acc);
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

}  // namespace csa2
