// Per-group FP4 quantizers shared by the quantize kernels and the KV
// projection's epilogue: a 16-channel group with an E4M3 scale, or a
// 32-channel MXFP4 block with an E8M0 scale (the rules are described where
// the kernels use them, in quant.hip).
#pragma once

#include "device.hpp"

namespace csa2 {

typedef float f32x2 __attribute__((ext_vector_type(2)));

// E2M1 code by thresholds t*S (t = 0.25 .. 5): strict '>' where the lower
// neighbour has the even code, '>=' where the upper one does.
__device__ __forceinline__ uint32_t code_by_thresholds(uint32_t hb, float S) {
    const float v = bf16_bits_to_f32(hb & 0x7FFFu);
    uint32_t c = (uint32_t)(v > 0.25f * S) + (uint32_t)(v >= 0.75f * S) + (uint32_t)(v > 1.25f * S) +
                 (uint32_t)(v >= 1.75f * S) + (uint32_t)(v > 2.5f * S) + (uint32_t)(v >= 3.5f * S) +
                 (uint32_t)(v > 5.0f * S);
    return c | ((hb >> 12) & 8u);               // sign bit of the bf16 -> code bit 3
}

// y rounded to 12 significant bits (half away from zero on the magnitude).
__device__ __forceinline__ float round12(float y) { return __uint_as_float((__float_as_uint(y) + 0x400u) & ~0x7FFu); }

// Codes of the bf16 pair in w (channels 2j, 2j+1), times r, into byte J of acc.
template <int J>
__device__ __forceinline__ uint32_t put_pair(uint32_t acc, uint32_t w, float r) {
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(acc, round12(bf16_bits_to_f32(w & 0xFFFFu) * r),
                                                    round12(__uint_as_float(w & 0xFFFF0000u) * r), 1.0f, J);
}

// E2M1 values (unit scale) of the two codes in byte J of w.
template <int J>
__device__ __forceinline__ f32x2 fp4_pair(uint32_t w) {
    return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, J);
}

// 16 bf16 values (w[j]: channels 2j, 2j+1) -> packed codes and the scale byte.
__device__ __forceinline__ uint2 quant_group(const uint32_t (&w)[8], uint32_t& sc) {
    uint32_t amax_bits = 0;                     // |x| of non-NaN bf16 orders like its bits
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        amax_bits = max(amax_bits, w[i] & 0x7FFFu);
        amax_bits = max(amax_bits, (w[i] >> 16) & 0x7FFFu);
    }
    const float amax = bf16_bits_to_f32(amax_bits);
    sc = f32_to_e4m3_sat(__fdiv_rn(amax, 6.0f));
    const float S = e4m3_to_f32(sc);
    uint32_t lo = 0, hi = 0;
    if (S > 0.0f && amax_bits < 0x7F80u) {
        const float r = __frcp_rn(S);
        lo = put_pair<0>(lo, w[0], r);
        lo = put_pair<1>(lo, w[1], r);
        lo = put_pair<2>(lo, w[2], r);
        lo = put_pair<3>(lo, w[3], r);
        hi = put_pair<0>(hi, w[4], r);
        hi = put_pair<1>(hi, w[5], r);
        hi = put_pair<2>(hi, w[6], r);
        hi = put_pair<3>(hi, w[7], r);
    } else if (S > 0.0f) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const uint32_t hb = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
            const uint32_t c = code_by_thresholds(hb, S);
            if (i < 8) lo |= c << (4 * i);
            else hi |= c << (4 * (i - 8));
        }
    }
    return make_uint2(lo, hi);
}

// 32 bf16 values (w[j]: channels 2j, 2j+1) of one MXFP4 block -> 16 code
// bytes (c[0..3]) and the E8M0 scale byte.
__device__ __forceinline__ uint32_t quant_block_mx(const uint32_t (&w)[16], uint32_t (&c)[4]) {
    uint32_t amax_bits = 0;
#pragma unroll
    for (int i = 0; i < 16; ++i) amax_bits = max(amax_bits, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    const int32_t e = (int32_t)(amax_bits >> 7) - 2;     // bf16 exponent field - 2
    const uint32_t sc = (uint32_t)(e > 0 ? e : 0);
    const float inv = __uint_as_float((254u - sc) << 23);  // 2^(127 - byte), exact
#pragma unroll
    for (int k = 0; k < 4; ++k) c[k] = 0u;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float y0 = bf16_bits_to_f32(w[i] & 0xFFFFu) * inv;
        const float y1 = __uint_as_float(w[i] & 0xFFFF0000u) * inv;
        switch (i & 3) {
            case 0: c[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[i >> 2], y0, y1, 1.0f, 0); break;
            case 1: c[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[i >> 2], y0, y1, 1.0f, 1); break;
            case 2: c[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[i >> 2], y0, y1, 1.0f, 2); break;
            default: c[i >> 2] = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c[i >> 2], y0, y1, 1.0f, 3); break;
        }
    }
    return sc;
}

}  // namespace csa2
