// FP4 E2M1 quantization with one E4M3 scale per 16 channels, and the inverse.
//
// One lane owns one 16-channel group: it loads the group's 32 bytes of bf16
// with two 16-byte loads (a wave covers 2 KiB of a row contiguously), finds
// amax, rounds amax/6 to E4M3 (round-to-nearest-even, saturating at 448),
// and picks each E2M1 code by comparing |x| with the scaled rounding
// thresholds t*S, t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}. Each t*S has at
// most 7 significant bits, so it is exact in fp32 and the comparison decides
// exactly as rounding the real quotient x/S would: strict '>' at thresholds
// whose lower neighbour has the even code, '>=' where the upper one does.
// The 16 codes leave as one 8-byte store, the scale as one byte.
#include "device.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kQuantThreads = 256;

__global__ void __launch_bounds__(kQuantThreads)
k_quant(const uint16_t* __restrict__ x, int64_t rows, int32_t gpr, int64_t x_stride, uint8_t* __restrict__ codes,
        int64_t cs, uint8_t* __restrict__ scales, int64_t ss) {
    const int64_t total = rows * gpr;
    for (int64_t gid = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; gid < total;
         gid += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t r = gid / gpr;
        const int32_t g = (int32_t)(gid - r * gpr);
        const uint4* src = reinterpret_cast<const uint4*>(x + r * x_stride + (int64_t)g * 16);
        const uint4 a = ld_stream16(src);
        const uint4 b = ld_stream16(src + 1);
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t amax_bits = 0;                 // |x| of non-NaN bf16 orders like its bits
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            amax_bits = max(amax_bits, w[i] & 0x7FFFu);
            amax_bits = max(amax_bits, (w[i] >> 16) & 0x7FFFu);
        }
        const float amax = bf16_bits_to_f32(amax_bits);
        const uint32_t sc = f32_to_e4m3_sat(__fdiv_rn(amax, 6.0f));
        const float S = e4m3_to_f32(sc);
        uint32_t lo = 0, hi = 0;
        if (S > 0.0f) {
            const float t0 = 0.25f * S, t1 = 0.75f * S, t2 = 1.25f * S, t3 = 1.75f * S;
            const float t4 = 2.5f * S, t5 = 3.5f * S, t6 = 5.0f * S;
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const uint32_t hb = (i & 1) ? (w[i >> 1] >> 16) : (w[i >> 1] & 0xFFFFu);
                const float v = bf16_bits_to_f32(hb & 0x7FFFu);
                uint32_t c = (uint32_t)(v > t0) + (uint32_t)(v >= t1) + (uint32_t)(v > t2) + (uint32_t)(v >= t3) +
                             (uint32_t)(v > t4) + (uint32_t)(v >= t5) + (uint32_t)(v > t6);
                c |= (hb >> 12) & 8u;           // sign bit of the bf16 -> code bit 3
                if (i < 8) lo |= c << (4 * i);
                else hi |= c << (4 * (i - 8));
            }
        }
        *reinterpret_cast<uint2*>(codes + r * cs + (int64_t)g * 8) = make_uint2(lo, hi);
        scales[r * ss + g] = (uint8_t)sc;
    }
}

__global__ void __launch_bounds__(kQuantThreads)
k_dequant(const uint8_t* __restrict__ codes, int64_t cs, const uint8_t* __restrict__ scales, int64_t ss,
          int64_t rows, int32_t gpr, uint16_t* __restrict__ y, int64_t y_stride) {
    const int64_t total = rows * gpr;
    for (int64_t gid = (int64_t)blockIdx.x * kQuantThreads + threadIdx.x; gid < total;
         gid += (int64_t)gridDim.x * kQuantThreads) {
        const int64_t r = gid / gpr;
        const int32_t g = (int32_t)(gid - r * gpr);
        const uint2 c = *reinterpret_cast<const uint2*>(codes + r * cs + (int64_t)g * 8);
        const float S = e4m3_to_f32(scales[r * ss + g]);
        uint32_t o[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t word = (i < 4) ? c.x : c.y;
            const uint32_t byte = (word >> (8 * (i & 3))) & 0xFFu;
            const uint32_t c0 = byte & 0xFu, c1 = byte >> 4;
            // E2M1 * E4M3 is exact in fp32 and in bf16, so the top half is the bf16.
            const uint32_t v0 = __float_as_uint(e2m1_mag_to_f32(c0 & 7u) * S) | ((c0 & 8u) << 28);
            const uint32_t v1 = __float_as_uint(e2m1_mag_to_f32(c1 & 7u) * S) | ((c1 & 8u) << 28);
            o[i] = (v0 >> 16) | (v1 & 0xFFFF0000u);
        }
        uint4* dst = reinterpret_cast<uint4*>(y + r * y_stride + (int64_t)g * 16);
        dst[0] = make_uint4(o[0], o[1], o[2], o[3]);
        dst[1] = make_uint4(o[4], o[5], o[6], o[7]);
    }
}

static unsigned grid_for(int64_t items, int threads) {
    int64_t blocks = (items + threads - 1) / threads;
    const int64_t cap = 256 * 64;               // grid-stride beyond this
    if (blocks > cap) blocks = cap;
    return (unsigned)(blocks < 1 ? 1 : blocks);
}

int launch_quant(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride, uint8_t* codes, int64_t cs,
                 uint8_t* scales, int64_t ss, hipStream_t stream) {
    if (rows == 0) return OK;
    const int32_t gpr = C / 16;
    hipLaunchKernelGGL(k_quant, dim3(grid_for(rows * gpr, kQuantThreads)), dim3(kQuantThreads), 0, stream, x, rows,
                       gpr, x_stride, codes, cs, scales, ss);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_quant");
}

int launch_dequant(const uint8_t* codes, int64_t cs, const uint8_t* scales, int64_t ss, int64_t rows, int32_t C,
                   uint16_t* y, int64_t y_stride, hipStream_t stream) {
    if (rows == 0) return OK;
    const int32_t gpr = C / 16;
    hipLaunchKernelGGL(k_dequant, dim3(grid_for(rows * gpr, kQuantThreads)), dim3(kQuantThreads), 0, stream, codes,
                       cs, scales, ss, rows, gpr, y, y_stride);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_dequant");
}

}  // namespace csa2
