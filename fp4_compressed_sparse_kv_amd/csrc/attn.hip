// Sparse softmax attention over gathered FP4 KV rows on gfx950 matrix cores.
//
// One query row (all H <= 16 heads, which share one KV head and one position
// list) is split over NS workgroups of 4 waves; each wave walks blocks of 32
// positions of its slice. Per block, a wave:
//   1. gathers, per lane, the K code bytes and scales it feeds to the matrix
//      core (16 contiguous code bytes of one position) and the V code dword /
//      scale of 8 positions, straight from HBM;
//   2. dequantizes in registers: the FP4 pairs are widened to f16 with the
//      hardware convert at unit scale (exact), then multiplied by the E4M3
//      scale as a packed f16 product (E2M1 x E4M3 has at most 6 significant
//      bits and lies in [2^-10, 2688], so it is exact in f16);
//   3. S^T = K_hat Q^T with 8 MFMA 16x16x32 f16 (M = positions, N = heads,
//      contraction over the 128 channels in a lane-friendly channel order);
//   4. an online softmax per head on the accumulator registers;
//   5. out^T += V_hat^T P^T with 8 more MFMAs. The contraction index of this
//      product is ordered so that each lane's softmax weights are exactly the
//      ones it holds from step 3 (no cross-lane movement), and output channel
//      8m + t of MFMA t lands in accumulator row m, so each lane dequantizes
//      only the 8 channels 8n..8n+7 of its 8 positions.
// The query is converted to f16 once (exact for |q| in [2^-14, 65504]; smaller
// magnitudes round to f16 subnormals, an absolute error below 2^-25). Each
// softmax weight p (fp32) enters the matrix core as two f16 terms hi + lo
// (about 22 significant bits together); accumulation is fp32.
// The 4 waves are merged through LDS; the NS slices of a row are written to
// the workspace and merged in slice order by a second, small kernel, so the
// result does not depend on scheduling.
#include "device.hpp"
#include "internal.hpp"

namespace csa2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kAttnThreads = 256;
constexpr int kAttnWaves = 4;
constexpr int kBlk = 32;
constexpr int kMaxHeads = 16;
constexpr int kD = 128;
constexpr int kAttnWsHeader = 64;               // words; [0] device status word
constexpr int kAttnTargetBlocks = 512;
constexpr int kMaxSplits = 16;                  // slices per query row (bounded for the merge)
constexpr float kLog2e = 1.4426950408889634f;

static int attn_splits(int64_t rows, int32_t K) {
    const int64_t nblk = (K + kBlk - 1) / kBlk;
    int64_t ns = (kAttnTargetBlocks + rows - 1) / (rows > 0 ? rows : 1);
    const int64_t max_ns = (nblk + kAttnWaves - 1) / kAttnWaves;   // at least one block per wave
    if (ns > max_ns) ns = max_ns;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    return (int)ns;
}

size_t attn_workspace_bytes(int64_t rows, int32_t H, int32_t d, int32_t K) {
    const int ns = attn_splits(rows, K);
    const size_t part = (size_t)rows * ns * (size_t)kMaxHeads * (kD + 2);
    (void)H;
    (void)d;
    return (kAttnWsHeader + part) * 4;
}

// 8 FP4 codes (one dword, channel 2j in the low nibble of byte j) times a scale -> 8 f16.
__device__ __forceinline__ f16x8 dq8(uint32_t w, _Float16 s) {
    const f16x2 ss = {s, s};
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * ss;
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * ss;
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * ss;
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * ss;
    return f16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ _Float16 scale_f16(uint32_t b) { return (_Float16)e4m3_to_f32(b); }

__global__ void __launch_bounds__(kAttnThreads)
k_sparse_attn(const uint16_t* __restrict__ q, int32_t rows_per_seq, int32_t H, const uint8_t* __restrict__ k_codes,
              const uint8_t* __restrict__ k_scales, const uint8_t* __restrict__ v_codes,
              const uint8_t* __restrict__ v_scales, int64_t N, int64_t cs, int64_t ss, const int32_t* __restrict__ idx,
              int64_t idx_stride, int32_t K, float scale, float* __restrict__ out, int32_t NS,
              uint32_t* __restrict__ ws, int64_t rows) {
    __shared__ float s_m[kAttnWaves][kMaxHeads];
    __shared__ float s_l[kAttnWaves][kMaxHeads];
    __shared__ float s_acc[kAttnWaves][kMaxHeads][kD + 1];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t row = blockIdx.x / NS;
    const int split = blockIdx.x - (int)(row * NS);
    const int64_t seq = row / rows_per_seq;
    const int nblk = (K + kBlk - 1) / kBlk;
    const int bps = (nblk + NS - 1) / NS;              // blocks per slice
    const int b0 = split * bps, b1 = min(nblk, b0 + bps);
    const float sl2 = scale * kLog2e;

    // query as the B operand of S^T = K_hat Q^T: lane (n, g), k-step s holds
    // q[head n][channel 32g + 8s + i], i = 0..7
    f16x8 qb[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint4 raw = make_uint4(0, 0, 0, 0);
        if (n < H) raw = *reinterpret_cast<const uint4*>(q + (row * H + n) * (int64_t)kD + 32 * g + 8 * s);
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            qb[s][2 * i + 0] = (_Float16)bf16_bits_to_f32(w[i] & 0xFFFFu);
            qb[s][2 * i + 1] = (_Float16)bf16_bits_to_f32(w[i] >> 16);
        }
    }

    const int32_t* ip = idx + row * idx_stride;
    const uint8_t* kc_base = k_codes + seq * N * cs;
    const uint8_t* ks_base = k_scales + seq * N * ss;
    const uint8_t* vc_base = v_codes + seq * N * cs;
    const uint8_t* vs_base = v_scales + seq * N * ss;

    float m_run = -INFINITY, l_run = 0.f;             // per head n, in log2 units of the scaled logits
    f32x4 acc[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int blk = b0 + wave; blk < b1; blk += kAttnWaves) {
        const int jb = blk * kBlk;
        int32_t my_pos = -1;
        if (lane < kBlk && jb + lane < K) {
            const int32_t p = ip[jb + lane];
            my_pos = (p >= 0 && (int64_t)p < N) ? p : -1;
        }
        // K rows: positions n and 16 + n of the block; V rows / softmax columns:
        // positions 4g + i (i < 4) and 16 + 4g + (i - 4) (i >= 4)
        const int32_t kp0 = __shfl(my_pos, n), kp1 = __shfl(my_pos, 16 + n);
        int32_t vp[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) vp[i] = __shfl(my_pos, (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4));

        uint4 kraw[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
        uint32_t ksc[2] = {0, 0};
        if (kp0 >= 0) {
            kraw[0] = *reinterpret_cast<const uint4*>(kc_base + kp0 * cs + 16 * g);
            ksc[0] = (uint32_t)ks_base[kp0 * ss + 2 * g] | ((uint32_t)ks_base[kp0 * ss + 2 * g + 1] << 8);
        }
        if (kp1 >= 0) {
            kraw[1] = *reinterpret_cast<const uint4*>(kc_base + kp1 * cs + 16 * g);
            ksc[1] = (uint32_t)ks_base[kp1 * ss + 2 * g] | ((uint32_t)ks_base[kp1 * ss + 2 * g + 1] << 8);
        }
        uint32_t vraw[8], vsc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            vraw[i] = 0;
            vsc[i] = 0;
            if (vp[i] >= 0) {
                vraw[i] = *reinterpret_cast<const uint32_t*>(vc_base + vp[i] * cs + 4 * n);
                vsc[i] = vs_base[vp[i] * ss + (n >> 1)];
            }
        }

        // ---- S^T = K_hat Q^T
        f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const _Float16 s_lo = scale_f16(ksc[mb] & 0xFFu), s_hi = scale_f16(ksc[mb] >> 8);
            const uint32_t w[4] = {kraw[mb].x, kraw[mb].y, kraw[mb].z, kraw[mb].w};
#pragma unroll
            for (int s = 0; s < 4; ++s)
                sacc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(dq8(w[s], s < 2 ? s_lo : s_hi), qb[s], sacc[mb], 0, 0, 0);
        }

        // ---- online softmax for head n over the 8 positions this lane holds
        float lg[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const float sv = (i < 4) ? sacc[0][i] : sacc[1][i - 4];
            lg[i] = (vp[i] >= 0) ? sv * sl2 : -INFINITY;
        }
        float mx = lg[0];
#pragma unroll
        for (int i = 1; i < 8; ++i) mx = fmaxf(mx, lg[i]);
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float m_new = fmaxf(m_run, mx);
        f16x8 pb_hi, pb_lo;                         // p = hi + lo, both f16: ~22 significant bits
        float psum = 0.f, alpha = 1.f;
        if (m_new != -INFINITY) {
            alpha = exp2f(m_run - m_new);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float p = exp2f(lg[i] - m_new);
                const _Float16 hi = (_Float16)p;
                pb_hi[i] = hi;
                pb_lo[i] = (_Float16)(p - (float)hi);
                psum += p;
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; ++i) pb_hi[i] = pb_lo[i] = (_Float16)0.f;
        }
        psum += __shfl_xor(psum, 16);
        psum += __shfl_xor(psum, 32);
        l_run = l_run * alpha + psum;
        m_run = m_new;

        // ---- out^T += V_hat^T P^T: MFMA t covers channels 8m + t
        f16x2 hv[8][4];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const _Float16 sv = scale_f16(vsc[i]);
            const f16x2 sp = {sv, sv};
            hv[i][0] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vraw[i], 1.0f, 0) * sp;
            hv[i][1] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vraw[i], 1.0f, 1) * sp;
            hv[i][2] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vraw[i], 1.0f, 2) * sp;
            hv[i][3] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(vraw[i], 1.0f, 3) * sp;
        }
#pragma unroll
        for (int t = 0; t < 8; ++t) {
            f16x8 va;
#pragma unroll
            for (int i = 0; i < 8; ++i) va[i] = hv[i][t >> 1][t & 1];
            acc[t] = acc[t] * alpha;
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb_hi, acc[t], 0, 0, 0);
            acc[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(va, pb_lo, acc[t], 0, 0, 0);
        }
    }

    // ---- merge the 4 waves through LDS: lane (n, g) holds out[n][8*(4g+i) + t] in acc[t][i]
    if (g == 0) {
        s_m[wave][n] = m_run;
        s_l[wave][n] = l_run;
    }
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) s_acc[wave][n][8 * (4 * g + i) + t] = acc[t][i];
    __syncthreads();

    const int h = tid >> 4;                              // this thread's head and 8 channels
    const int c0 = (tid & 15) * 8;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, s_m[w][h]);
    float L = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float wt = (s_m[w][h] == -INFINITY) ? 0.f : exp2f(s_m[w][h] - M);
            L += wt * s_l[w][h];
#pragma unroll
            for (int i = 0; i < 8; ++i) o[i] = fmaf(wt, s_acc[w][h][c0 + i], o[i]);
        }
    }

    float* orow = out + row * (int64_t)H * kD;
    if (NS == 1) {
        if (h < H) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) orow[h * kD + c0 + i] = o[i] * inv;
        }
        return;
    }

    // ---- slices -> workspace (plain stores); k_attn_merge combines them in slice order
    float* part = reinterpret_cast<float*>(ws + kAttnWsHeader);
    const int64_t pstride = (int64_t)kMaxHeads * (kD + 2);
    float* mine = part + (row * NS + split) * pstride;
    *reinterpret_cast<float4*>(mine + h * kD + c0) = make_float4(o[0], o[1], o[2], o[3]);
    *reinterpret_cast<float4*>(mine + h * kD + c0 + 4) = make_float4(o[4], o[5], o[6], o[7]);
    if ((tid & 15) == 0) {
        mine[kMaxHeads * kD + 2 * h + 0] = M;
        mine[kMaxHeads * kD + 2 * h + 1] = L;
    }
}

// Merge of the NS slices of each query row (launched after k_sparse_attn on the
// same stream, so the kernel boundary orders the partials before these reads):
// out = sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s, in slice order.
__global__ void __launch_bounds__(kAttnThreads)
k_attn_merge(const uint32_t* __restrict__ ws, int32_t H, int32_t NS, float* __restrict__ out) {
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x;
    const int h = tid >> 4, c0 = (tid & 15) * 8;
    if (h >= H) return;
    const float* part = reinterpret_cast<const float*>(ws + kAttnWsHeader);
    const int64_t pstride = (int64_t)kMaxHeads * (kD + 2);
    const float* base = part + row * NS * pstride;
    float ms[kMaxSplits];
    float MM = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
        ms[s] = (s < NS) ? base[s * pstride + kMaxHeads * kD + 2 * h] : -INFINITY;
        MM = fmaxf(MM, ms[s]);
    }
    float LL = 0.f, oo[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (MM != -INFINITY) {
#pragma unroll 4
        for (int s = 0; s < NS; ++s) {
            const float* b = base + s * pstride;
            const float4 a0 = *reinterpret_cast<const float4*>(b + h * kD + c0);
            const float4 a1 = *reinterpret_cast<const float4*>(b + h * kD + c0 + 4);
            const float ls = b[kMaxHeads * kD + 2 * h + 1];
            const float wt = (ms[s] == -INFINITY) ? 0.f : exp2f(ms[s] - MM);
            LL += wt * ls;
            oo[0] = fmaf(wt, a0.x, oo[0]);
            oo[1] = fmaf(wt, a0.y, oo[1]);
            oo[2] = fmaf(wt, a0.z, oo[2]);
            oo[3] = fmaf(wt, a0.w, oo[3]);
            oo[4] = fmaf(wt, a1.x, oo[4]);
            oo[5] = fmaf(wt, a1.y, oo[5]);
            oo[6] = fmaf(wt, a1.z, oo[6]);
            oo[7] = fmaf(wt, a1.w, oo[7]);
        }
    }
    const float inv = LL > 0.f ? 1.f / LL : 0.f;
    float* orow = out + row * (int64_t)H * kD + h * kD + c0;
    *reinterpret_cast<float4*>(orow) = make_float4(oo[0] * inv, oo[1] * inv, oo[2] * inv, oo[3] * inv);
    *reinterpret_cast<float4*>(orow + 4) = make_float4(oo[4] * inv, oo[5] * inv, oo[6] * inv, oo[7] * inv);
}

int launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (a.rows == 0) return OK;
    const int ns = attn_splits(a.rows, a.K);
    if (ws_bytes < attn_workspace_bytes(a.rows, a.H, a.d, a.K)) return fail(WORKSPACE, "attention workspace too small");
    hipLaunchKernelGGL(k_sparse_attn, dim3((unsigned)(a.rows * ns)), dim3(kAttnThreads), 0, stream, a.q,
                       a.rows_per_seq, a.H, a.k_codes, a.k_scales, a.v_codes, a.v_scales, a.N, a.code_stride,
                       a.scale_stride, a.idx, a.idx_stride, a.K, a.scale, a.out, ns,
                       reinterpret_cast<uint32_t*>(ws), a.rows);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return hip_fail(e, "launch k_sparse_attn");
    if (ns > 1) {
        hipLaunchKernelGGL(k_attn_merge, dim3((unsigned)a.rows), dim3(kAttnThreads), 0, stream,
                           reinterpret_cast<const uint32_t*>(ws), a.H, ns, a.out);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "launch k_attn_merge");
    }
    return OK;
}

}  // namespace csa2
