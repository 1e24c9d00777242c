// The KV write path: decoder KV rows projected from the encoder's last hidden
// state, C = H W (bf16 inputs, fp32 accumulation on the matrix cores), each
// element rounded to bf16 and quantized to FP4 in the same kernel.
//
// H is [T][D] bf16; W is given transposed, one row of D weights per output
// channel ([256][D]: channels 0..127 are K, 128..255 are V of the one shared
// KV head), so both matrix-core operands are contiguous 16-byte runs along D.
// A workgroup of 8 waves owns 128 tokens and one half of the channels (K or
// V): wave w computes tokens 64 (w / 4) .. + 63 x channels 32 (w % 4) .. + 31
// with v_mfma_f32_32x32x16_bf16 (two 32-token tiles), over k-tiles of 64; two
// waves per SIMD let one wave's matrix work overlap the other's staging (4
// waves of 64 tokens x 64 channels: 53 us at 16384 x 4096; 8 waves of 64
// tokens x 32 channels over all 256 channels: 47 us; this shape, which reads
// half the weights per token: 44 us). Both tiles go through LDS: the H tile
// is shared by the eight waves, and each load instruction of a wave reads 8
// whole 128-byte rows (8 lanes per row; loading each wave's operands straight
// into the matrix-core layout touched 32 rows per instruction, 32 bytes of
// each, and the rows were evicted from L1 before the rest was read: 68 us).
// Three register sets and three LDS buffers rotate: while tile k is
// multiplied from LDS buffer k % 3, tile k+2 is being requested into set
// (k+2) % 3 and tile k+1 is written from its set into LDS buffer (k+1) % 3,
// so every load has two tiles' worth of matrix-core work to arrive. The two
// halves of a token tile run on the same XCD (numbered a tile count apart), so
// the second one's H rows mostly come from L2; W (2 MiB at D = 4096) is read
// by every workgroup and stays in each XCD's L2. The epilogue rounds the
// fp32 sums to bf16 (nearest even) into an LDS tile, then each thread quantizes whole 16-channel groups (E4M3 scale)
// or 32-channel blocks (E8M0 scale) with the same per-group code as
// kv_quant_fp4 / kv_quant_mxfp4, and writes the cache records directly:
// codes [K 64 B | V 64 B], scales [K | V], optionally the bf16 row as well.
#include "fp4q.hpp"
#include "internal.hpp"

namespace csa2 {

typedef __bf16 bf16x8p __attribute__((ext_vector_type(8)));
typedef float f32x16p __attribute__((ext_vector_type(16)));

constexpr int kPjThreads = 512;
constexpr int kPjM = 128;                       // tokens per workgroup
constexpr int kPjN = 128;                       // output channels per workgroup (K or V)
constexpr int kPjK = 64;                        // k-tile
constexpr int kPjRow = kPjK + 8;                // staged row: 64 bf16 + 8 pad
constexpr int kPjCRow = kPjN + 8;               // epilogue row of bf16

struct PjStage {
    uint16_t a[3][kPjM * kPjRow];
    uint16_t b[3][kPjN * kPjRow];               // the weight tile, [channel][k]
};
union PjLds {
    PjStage st;
    uint16_t c[kPjM * kPjCRow];
};

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    const uint32_t u = __float_as_uint(x);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

template <bool MX>
__global__ void __launch_bounds__(kPjThreads)
k_kv_project(const uint16_t* __restrict__ h, int64_t T, int32_t D, int64_t hs, const uint16_t* __restrict__ wt,
             int64_t wsd, uint8_t* __restrict__ codes, int64_t cs, uint8_t* __restrict__ scales, int64_t ss,
             uint16_t* __restrict__ cout, int64_t cos) {
    __shared__ __attribute__((aligned(16))) PjLds lds;
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int ln = lane & 31, g = lane >> 5;
    // both halves of a token tile (K, then V) are numbered a tile count apart,
    // so they run on the same XCD and the second one's H reads hit its L2
    const int64_t ntiles = (T + kPjM - 1) / kPjM;
    const int64_t tile = (int64_t)blockIdx.x % ntiles;
    const int half = (int)((int64_t)blockIdx.x / ntiles);
    const int64_t m0 = tile * kPjM;

    // global -> register loads of one k-tile: thread t takes 16-byte chunk
    // (t & 7) of H rows (t >> 3) and (t >> 3) + 64 and of this half's W^T rows
    // at the same offsets: a wave's load instruction reads 8 whole 128-byte rows
    const int lr = tid >> 3, lk = (tid & 7) * 8;
    const uint16_t* ap0 = h + min(m0 + lr, T - 1) * hs + lk;          // rows past T reload the last one (never stored)
    const uint16_t* ap1 = h + min(m0 + lr + 64, T - 1) * hs + lk;
    const uint16_t* bp = wt + (int64_t)(kPjN * half + lr) * wsd + lk;
    struct Regs {                               // named registers: nothing indexed at run time
        uint4 a0, a1, b0, b1;
    };
    Regs r0, r1, r2;
    auto ld16 = [](const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); };
    auto load = [&](int kt, Regs& r) {
        const int o = kt * kPjK;
        r.a0 = ld16(ap0 + o);
        r.a1 = ld16(ap1 + o);
        r.b0 = ld16(bp + o);
        r.b1 = ld16(bp + (int64_t)64 * wsd + o);
    };
    auto store = [&](int buf, const Regs& r) {
        *reinterpret_cast<uint4*>(&lds.st.a[buf][lr * kPjRow + lk]) = r.a0;
        *reinterpret_cast<uint4*>(&lds.st.a[buf][(lr + 64) * kPjRow + lk]) = r.a1;
        *reinterpret_cast<uint4*>(&lds.st.b[buf][lr * kPjRow + lk]) = r.b0;
        *reinterpret_cast<uint4*>(&lds.st.b[buf][(lr + 64) * kPjRow + lk]) = r.b1;
    };

    // wave w: tokens 64 (w / 4) .. + 63 (two 32-token tiles) x channels 32 (w % 4) .. + 31
    const int tb = wave >> 2, cbw = wave & 3;
    f32x16p acc[2][1];
#pragma unroll
    for (int mi = 0; mi < 2; ++mi) acc[mi][0] = f32x16p{};

    auto compute = [&](int cur) {
#pragma unroll
        for (int s = 0; s < kPjK / 16; ++s) {   // k-step s, lane group g: k = 16 s + 8 g .. + 7
            bf16x8p a[2], bq[1];
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                a[mi] = __builtin_bit_cast(bf16x8p, *reinterpret_cast<const uint4*>(
                                                        &lds.st.a[cur][(64 * tb + 32 * mi + ln) * kPjRow + 16 * s + 8 * g]));
            bq[0] = __builtin_bit_cast(bf16x8p, *reinterpret_cast<const uint4*>(
                                                    &lds.st.b[cur][(32 * cbw + ln) * kPjRow + 16 * s + 8 * g]));
#pragma unroll
            for (int mi = 0; mi < 2; ++mi)
                acc[mi][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[mi], bq[0], acc[mi][0], 0, 0, 0);
        }
    };

    // tile k: LDS buffer and register set k % 3. Loads past the last tile
    // re-read the last one (unconditional loads keep the compiler's wait
    // counts exact) and are never used.
    const int nk = D / kPjK;
    auto step = [&](int k, Regs& rl, Regs& rc, Regs& rs, int bc, int bs) {
        (void)rc;
        load(min(k + 2, nk - 1), rl);           // tile k+2
        compute(bc);                            // tile k
        if (k + 1 < nk) store(bs, rs);          // tile k+1
        __syncthreads();
    };
    load(0, r0);
    load(min(1, nk - 1), r1);
    store(0, r0);
    __syncthreads();
    for (int kt = 0; kt < nk; kt += 3) {
        step(kt, r2, r0, r1, 0, 1);
        if (kt + 1 < nk) step(kt + 1, r0, r1, r2, 1, 2);
        if (kt + 2 < nk) step(kt + 2, r1, r2, r0, 2, 0);
    }
    __syncthreads();                            // the epilogue tile overlays the staging buffers

    // ---- epilogue: bf16 tile in LDS (element i of a 32x32 accumulator is row
    // 8 (i / 4) + 4 g + i % 4, column ln), then whole groups per thread
#pragma unroll
    for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int m = 64 * tb + 32 * mi + 8 * (i / 4) + 4 * g + (i % 4);
            const int n = 32 * cbw + ln;
            lds.c[m * kPjCRow + n] = (uint16_t)bf16_rne_bits(acc[mi][0][i]);
        }
    __syncthreads();
    constexpr int kGroup = MX ? 32 : 16;
    constexpr int kUnits = kPjM * kPjN / kGroup;
#pragma unroll
    for (int j = 0; j < kUnits / kPjThreads; ++j) {
        const int u = tid + kPjThreads * j;
        const int tok = u / (kPjN / kGroup), grp = u % (kPjN / kGroup);
        const int64_t row = m0 + tok;
        const uint4* src = reinterpret_cast<const uint4*>(&lds.c[tok * kPjCRow + grp * kGroup]);
        if (row >= T) continue;
        if constexpr (MX) {
            uint32_t w[16];
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const uint4 v = src[q];
                w[4 * q] = v.x;
                w[4 * q + 1] = v.y;
                w[4 * q + 2] = v.z;
                w[4 * q + 3] = v.w;
            }
            uint32_t c[4];
            const uint32_t sc = quant_block_mx(w, c);
            *reinterpret_cast<uint4*>(codes + row * cs + 64 * half + grp * 16) = make_uint4(c[0], c[1], c[2], c[3]);
            scales[row * ss + 4 * half + grp] = (uint8_t)sc;
            if (cout) {
                uint4* dst = reinterpret_cast<uint4*>(cout + row * cos + kPjN * half + grp * kGroup);
#pragma unroll
                for (int q = 0; q < 4; ++q) dst[q] = src[q];
            }
        } else {
            const uint4 v0 = src[0], v1 = src[1];
            const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
            uint32_t sc;
            const uint2 c = quant_group(w, sc);
            *reinterpret_cast<uint2*>(codes + row * cs + 64 * half + grp * 8) = c;
            scales[row * ss + 8 * half + grp] = (uint8_t)sc;
            if (cout) {
                uint4* dst = reinterpret_cast<uint4*>(cout + row * cos + kPjN * half + grp * kGroup);
                dst[0] = v0;
                dst[1] = v1;
            }
        }
    }
}

int launch_kv_project(const uint16_t* h, int64_t T, int32_t D, int64_t hs, const uint16_t* wt, int64_t wsd, bool mx,
                      uint8_t* codes, int64_t cs, uint8_t* scales, int64_t ss, uint16_t* cout, int64_t cos,
                      hipStream_t stream) {
    if (T == 0) return OK;
    const int64_t groups = 2 * ((T + kPjM - 1) / kPjM);   // token tiles x (K, V)
    if (groups > 0x7FFFFFFFll) return fail(INVALID, "kv projection: too many tokens");
    if (mx)
        hipLaunchKernelGGL(k_kv_project<true>, dim3((unsigned)groups), dim3(kPjThreads), 0, stream, h, T, D, hs, wt, wsd,
                           codes, cs, scales, ss, cout, cos);
    else
        hipLaunchKernelGGL(k_kv_project<false>, dim3((unsigned)groups), dim3(kPjThreads), 0, stream, h, T, D, hs, wt,
                           wsd, codes, cs, scales, ss, cout, cos);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_kv_project");
}

}  // namespace csa2
