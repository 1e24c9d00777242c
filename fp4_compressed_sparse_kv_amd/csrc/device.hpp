// Device helpers shared by the gfx950 kernels of libcsa2: number formats,
// order-preserving score keys, cross-lane sums and the in-kernel row barrier.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace csa2 {

constexpr int kWave = 64;

// ------------------------------------------------------------------ loads

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: non-temporal hint).
__device__ __forceinline__ uint4 ld_stream16(const void* p) {
    const u32x4 v = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
    return make_uint4(v.x, v.y, v.z, v.w);
}

// ---------------------------------------------------------------- formats

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// E4M3FN byte -> fp32 (exact). Bias 7; exponent field 0 is subnormal (m * 2^-9);
// 0x7F / 0xFF are NaN.
__device__ __forceinline__ float e4m3_to_f32(uint32_t b) {
    const uint32_t e = (b >> 3) & 0xFu, m = b & 7u;
    float v = (e == 0) ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
    if (e == 0xFu && m == 7u) v = __uint_as_float(0x7FC00000u);
    return (b & 0x80u) ? -v : v;
}

// Non-negative finite fp32 -> E4M3FN byte, round-to-nearest-even, saturating
// at 448 (0x7E). Below 2^-6 the E4M3 grid is m * 2^-9 (m = 0..8; m = 8 is the
// smallest normal 0x08), so the code is rint(v * 512), an exact scaling.
__device__ __forceinline__ uint32_t f32_to_e4m3_sat(float v) {
    if (!(v < 448.0f)) return 0x7Eu;
    if (v < 0.015625f) return (uint32_t)rintf(v * 512.0f);
    const uint32_t u = __float_as_uint(v);
    uint32_t r = (((u >> 23) - 120u) << 3) | ((u >> 20) & 7u);   // exponent rebias 127 -> 7
    const uint32_t rest = u & 0xFFFFFu, half = 0x80000u;         // 20 dropped mantissa bits
    if (rest > half || (rest == half && (r & 1u))) r += 1u;     // a carry moves into the exponent
    return r;
}

// E2M1 magnitude code (0..7) -> fp32: {0, .5, 1, 1.5, 2, 3, 4, 6}. For c >= 2 the
// fp32 pattern is (c + 252) << 22 (exponent c>>1 with bias 1, mantissa c&1).
__device__ __forceinline__ float e2m1_mag_to_f32(uint32_t c) {
    const uint32_t bits = (c >= 2u) ? ((c + 252u) << 22) : (c == 1u ? (252u << 22) : 0u);
    return __uint_as_float(bits);
}

// ------------------------------------------------------------ score keys

// Order-preserving map fp32 -> u32 for selection. NaN and -inf map to 0 (never
// selected); -0 maps like +0; every other value maps to >= 0x00800000.
__device__ __forceinline__ uint32_t score_key(float s) {
    uint32_t u = __float_as_uint(s);
    if (s != s || u == 0xFF800000u) return 0u;
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float key_score(uint32_t k) {
    if (k == 0u) return __uint_as_float(0x7FC00000u);
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

// ------------------------------------------------------------ cross-lane

__device__ __forceinline__ double shfl_xor_f64(double v, int mask) {
    const int2 p = *reinterpret_cast<int2*>(&v);
    int2 r;
    r.x = __shfl_xor(p.x, mask);
    r.y = __shfl_xor(p.y, mask);
    return *reinterpret_cast<double*>(&r);
}

// Inclusive prefix sum over the 64 lanes of a wave, in registers: shifts
// within each row of 16 lanes (1, 2, 4, 8), then the last lane of row 0 is
// added to row 1 and of row 2 to row 3, then the last lane of row 1 (by now
// the total of rows 0-1) to rows 2 and 3. Lanes whose source is outside the
// row, and rows outside the row mask, add 0.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, false);   // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, false);   // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, false);   // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, false);   // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false);   // row_bcast:15
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false);   // row_bcast:31
    return v;
}

// Number of set bits of a wave mask in the lanes below this one.
__device__ __forceinline__ uint32_t lanes_below(uint64_t m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Sum over the wave, in every lane: the inclusive scan's last lane, broadcast.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan(v), kWave - 1);
}

// ---------------------------------------------------- device-scope exchange

__device__ __forceinline__ uint32_t ld_acq(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_rlx(const uint32_t* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_rlx(uint32_t* p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_rlx(uint32_t* p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Bounded wait: a wait that does not finish within this many polls gives up,
// flags the status word and lets the kernel run to its end.
constexpr uint32_t kSpinLimit = 1u << 20;
constexpr uint32_t kStatusBarrierTimeout = 1u;

__device__ __forceinline__ void st_rlx_f32(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_rlx_f32(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Raw buffer resources: word 3 of a byte-addressed resource with a 32-bit data
// format; a load past the resource's range returns 0 without a memory access.
// Cache policy sc1 makes a buffer access device-coherent, like the relaxed
// agent-scope atomics above.
constexpr uint32_t kRsrcWord3 = 0x00020000u;
constexpr int kCoherent = 16;

// Wait until every memory operation this wave has issued - including
// non-returning atomics and stores - has completed.
__device__ __forceinline__ void wave_drain() { __builtin_amdgcn_s_waitcnt(0); }

// Cross-workgroup data in this library moves only through device-scope
// atomics and device-scope (coherent, "sc1") loads and stores, never through
// ordinary cached accesses. Publishing therefore needs no L2 write-back and
// consuming no L2 invalidate: a writer drains its own operations (wave_drain)
// before the flag RMW that announces them, and readers read with coherent
// loads. On this multi-XCD part an agent-scope fence costs an L2 write-back
// or invalidate of the whole XCD, which is what this protocol avoids.
//
// Barrier among the S workgroups that share one row. `ctrl` is a counter that
// starts at 0 for the launch; the g-th barrier waits until it reaches g*S.
__device__ __forceinline__ void row_barrier(uint32_t* ctrl, uint32_t S, uint32_t& gen, uint32_t* status) {
    wave_drain();
    __syncthreads();
    gen += 1;
    if (threadIdx.x == 0) {
        add_rlx(ctrl, 1u);
        const uint32_t target = gen * S;
        uint32_t spins = 0;
        while (ld_rlx(ctrl) < target) {
            __builtin_amdgcn_s_sleep(1);
            if (++spins > kSpinLimit) {
                __hip_atomic_fetch_or(status, kStatusBarrierTimeout, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                break;
            }
        }
    }
    __syncthreads();
}

}  // namespace csa2
