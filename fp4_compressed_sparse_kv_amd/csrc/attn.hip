// Sparse softmax attention over gathered FP4 KV rows (gather, dequantize, attend).
//
// One query row (all H heads, which share one KV head and one position list)
// is split over NS workgroups, each taking a contiguous slice of the position
// list. A workgroup walks its slice in tiles of 32 positions: 256 lanes each
// gather one 16-channel group of K and of V (8 code bytes + 1 scale byte each),
// dequantize it in registers (E2M1 value times the E4M3 scale, exact in fp32)
// into LDS, then compute the tile's logits and fold the tile into an online
// softmax (running max, running sum, fp32 accumulators). Each slice leaves
// (max, sum, acc) per head in the workspace; the last workgroup of the row to
// finish (device-scope counter) combines the slices in slice order, so the
// result does not depend on scheduling.
#include "device.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kAttnThreads = 256;
constexpr int kTile = 32;
constexpr int kMaxHeads = 16;
constexpr int kD = 128;
constexpr int kAttnWsHeader = 64;             // words; [0] device status word
constexpr int kAttnTargetBlocks = 512;

static int attn_splits(int64_t rows, int32_t K) {
    int64_t ns = (kAttnTargetBlocks + rows - 1) / (rows > 0 ? rows : 1);
    const int64_t max_ns = (K + 63) / 64;
    if (ns > max_ns) ns = max_ns;
    if (ns < 1) ns = 1;
    return (int)ns;
}

size_t attn_workspace_bytes(int64_t rows, int32_t H, int32_t d, int32_t K) {
    const int ns = attn_splits(rows, K);
    const size_t counters = (size_t)((rows + 63) / 64 * 64);
    const size_t part = (size_t)rows * ns * (size_t)H * (d + 2);
    return (kAttnWsHeader + counters + part) * 4;
}

__device__ __forceinline__ void dequant_group16(uint2 c, float S, float* dst) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const uint32_t word = (i < 8) ? c.x : c.y;
        const uint32_t code = (word >> (4 * (i & 7))) & 0xFu;
        const float v = e2m1_mag_to_f32(code & 7u) * S;
        dst[i] = (code & 8u) ? -v : v;
    }
}

__global__ void __launch_bounds__(kAttnThreads)
k_sparse_attn(const uint16_t* __restrict__ q, int32_t rows_per_seq, int32_t H, const uint8_t* __restrict__ k_codes,
              const uint8_t* __restrict__ k_scales, const uint8_t* __restrict__ v_codes,
              const uint8_t* __restrict__ v_scales, int64_t N, int64_t cs, int64_t ss, const int32_t* __restrict__ idx,
              int64_t idx_stride, int32_t K, float scale, float* __restrict__ out, int32_t NS,
              uint32_t* __restrict__ ws, int64_t rows) {
    __shared__ float qf[kMaxHeads][kD];
    __shared__ float kt[kTile][kD + 1];
    __shared__ float vt[kTile][kD];
    __shared__ float pt[kMaxHeads][kTile];
    __shared__ int32_t tpos[kTile];
    __shared__ uint32_t last_flag;

    const int tid = threadIdx.x;
    const int64_t row = blockIdx.x / NS;
    const int split = blockIdx.x - (int)(row * NS);
    const int64_t seq = row / rows_per_seq;
    const int per = (K + NS - 1) / NS;
    const int j0 = split * per;
    const int j1 = min(K, j0 + per);

    for (int i = tid; i < H * kD; i += kAttnThreads)
        qf[i / kD][i % kD] = bf16_bits_to_f32(q[row * (int64_t)H * kD + i]);

    // accumulator ownership: head h = tid/16, channels [c0, c0+8)
    const int h = tid >> 4;
    const int c0 = (tid & 15) * 8;
    float acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    float m_run = -INFINITY, l_run = 0.f;

    const int32_t* ip = idx + row * idx_stride;
    for (int jt = j0; jt < j1; jt += kTile) {
        __syncthreads();
        if (tid < kTile) {
            const int j = jt + tid;
            int32_t pos = (j < j1) ? ip[j] : -1;
            if (pos < 0 || (int64_t)pos >= N) pos = -1;
            tpos[tid] = pos;
        }
        __syncthreads();
        {   // gather + dequant: token tid/8, group tid%8, for K and V
            const int tj = tid >> 3, g = tid & 7;
            const int32_t pos = tpos[tj];
            float kv[16], vv[16];
            if (pos >= 0) {
                const int64_t r = seq * N + pos;
                const uint2 kc = *reinterpret_cast<const uint2*>(k_codes + r * cs + g * 8);
                const uint2 vc = *reinterpret_cast<const uint2*>(v_codes + r * cs + g * 8);
                dequant_group16(kc, e4m3_to_f32(k_scales[r * ss + g]), kv);
                dequant_group16(vc, e4m3_to_f32(v_scales[r * ss + g]), vv);
            } else {
#pragma unroll
                for (int i = 0; i < 16; ++i) kv[i] = vv[i] = 0.f;
            }
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                kt[tj][g * 16 + i] = kv[i];
                vt[tj][g * 16 + i] = vv[i];
            }
        }
        __syncthreads();
        // logits: head h, tokens (tid%16)*2 + {0,1}
        float lg[2];
        if (h < H) {
#pragma unroll
            for (int u = 0; u < 2; ++u) {
                const int tj = (tid & 15) * 2 + u;
                float s = 0.f;
#pragma unroll 8
                for (int c = 0; c < kD; ++c) s = fmaf(qf[h][c], kt[tj][c], s);
                lg[u] = (tpos[tj] >= 0) ? s * scale : -INFINITY;
            }
        } else {
            lg[0] = lg[1] = -INFINITY;
        }
        // tile max over the 16 lanes of this head group
        float mx = fmaxf(lg[0], lg[1]);
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
        const float m_new = fmaxf(m_run, mx);
        float p0 = 0.f, p1 = 0.f, alpha = 1.f;
        if (m_new != -INFINITY) {
            p0 = __expf(lg[0] - m_new);
            p1 = __expf(lg[1] - m_new);
            alpha = __expf(m_run - m_new);
        }
        float ps = p0 + p1;
#pragma unroll
        for (int o = 8; o >= 1; o >>= 1) ps += __shfl_xor(ps, o);
        l_run = l_run * alpha + ps;
        m_run = m_new;
        if (h < H) {
            pt[h][(tid & 15) * 2 + 0] = p0;
            pt[h][(tid & 15) * 2 + 1] = p1;
        }
        __syncthreads();
        if (h < H) {
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] *= alpha;
            for (int tj = 0; tj < kTile; ++tj) {
                const float p = pt[h][tj];
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[i] = fmaf(p, vt[tj][c0 + i], acc[i]);
            }
        }
    }

    float* orow = out + row * (int64_t)H * kD;
    if (NS == 1) {
        if (h < H) {
            const float inv = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
            for (int i = 0; i < 8; ++i) orow[h * kD + c0 + i] = acc[i] * inv;
        }
        return;
    }
    // partials -> workspace; the last workgroup of the row combines them
    uint32_t* counters = ws + kAttnWsHeader;
    const int64_t ncnt = (rows + 63) / 64 * 64;
    float* part = reinterpret_cast<float*>(ws + kAttnWsHeader + ncnt);
    const int64_t pstride = (int64_t)H * (kD + 2);
    float* mine = part + (row * NS + split) * pstride;
    if (h < H) {
#pragma unroll
        for (int i = 0; i < 8; ++i) mine[h * kD + c0 + i] = acc[i];
        if ((tid & 15) == 0) {
            mine[H * kD + 2 * h + 0] = m_run;
            mine[H * kD + 2 * h + 1] = l_run;
        }
    }
    __threadfence();
    __syncthreads();
    if (tid == 0) {
        const uint32_t old = __hip_atomic_fetch_add(&counters[row], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        last_flag = (old == (uint32_t)NS - 1) ? 1u : 0u;
    }
    __syncthreads();
    if (!last_flag) return;
    __threadfence();
    if (h < H) {
        const float* base = part + row * NS * pstride;
        float M = -INFINITY;
        for (int s = 0; s < NS; ++s) M = fmaxf(M, base[s * pstride + H * kD + 2 * h]);
        float L = 0.f, o[8] = {0, 0, 0, 0, 0, 0, 0, 0};
        if (M != -INFINITY) {
            for (int s = 0; s < NS; ++s) {
                const float ms = base[s * pstride + H * kD + 2 * h];
                const float w = (ms == -INFINITY) ? 0.f : __expf(ms - M);
                L += w * base[s * pstride + H * kD + 2 * h + 1];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = fmaf(w, base[s * pstride + h * kD + c0 + i], o[i]);
            }
        }
        const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) orow[h * kD + c0 + i] = o[i] * inv;
    }
    if (tid == 0) st_rlx(&counters[row], 0u);
}

int launch_attn(const AttnArgs& a, void* ws, size_t ws_bytes, hipStream_t stream) {
    if (a.rows == 0) return OK;
    const int ns = attn_splits(a.rows, a.K);
    if (ws_bytes < attn_workspace_bytes(a.rows, a.H, a.d, a.K)) return fail(WORKSPACE, "attention workspace too small");
    hipLaunchKernelGGL(k_sparse_attn, dim3((unsigned)(a.rows * ns)), dim3(kAttnThreads), 0, stream, a.q,
                       a.rows_per_seq, a.H, a.k_codes, a.k_scales, a.v_codes, a.v_scales, a.N, a.code_stride,
                       a.scale_stride, a.idx, a.idx_stride, a.K, a.scale, a.out, ns,
                       reinterpret_cast<uint32_t*>(ws), a.rows);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_sparse_attn");
}

}  // namespace csa2
