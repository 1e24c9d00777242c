// Sparse softmax attention over gathered FP4 KV rows on gfx950 matrix cores.
//
// One query row (all H <= 16 heads, which share one KV head and one position
// list) is split over NS workgroups of W waves (8, or 4 when every row has a
// workgroup of its own); each wave walks
// blocks of 32 positions of its slice, with the next block's gathers (and the
// position list of the block after it) in flight while the current block is
// computed. Per block, a wave:
//   1. gathers, with 16-byte loads, the 64 K code bytes and 64 V code bytes of
//      each of its 32 positions (4 lanes per position and plane) and the
//      position's 8 + 8 E4M3 scale bytes, straight from HBM;
//   2. stages the V codes and all scales in its own LDS area, from which each
//      lane reads the bytes its matrix-core operands need;
//   3. dequantizes in registers: the FP4 pairs are widened to f16 with the
//      hardware convert at unit scale (exact - the instruction applies only
//      the exponent of its scale operand), then multiplied by the E4M3 scale
//      as a packed f16 product (E2M1 x E4M3 has at most 6 significant bits
//      and lies in [2^-10, 2688], so it is exact in f16);
//   4. S^T = K_hat Q^T with 8 MFMA 16x16x32 f16 (M = positions, N = heads,
//      contraction over the 128 channels in a lane-friendly channel order);
//   5. an online softmax per head on the accumulator registers;
//   6. out^T += V_hat^T P^T. The contraction index of this product is ordered
//      so that each lane's softmax weights are exactly the ones it holds from
//      step 4 (no cross-lane movement), and output channel 8m + t of MFMA t
//      lands in accumulator row m, so each lane dequantizes only the 8
//      channels 8n..8n+7 of its 8 positions.
// Each head's query is scaled by a power of two 2^-e (e from the head's
// largest |q|, so that element lands in [2^14, 2^15)) and converted to f16
// once: exact for every element within 2^28 of the head's largest one, any
// finite bf16 magnitude. The logits stay in these scaled units; the factor
// 2^e is applied to the differences (logit - running maximum) inside the
// exponent, so neither huge nor tiny queries overflow or lose the softmax.
// Each softmax weight p (fp32) enters the matrix core as two f16 terms
// hi + lo (about 22 significant bits together); accumulation is fp32.
//
// MXFP4 caches (E2M1 with one E8M0 scale per 32 channels) take the same
// path with bf16 operands: K is widened by the hardware scaled FP4 -> bf16
// convert, which applies the block's power-of-two scale exactly (a lane's 32
// K channels are one block); V by the FP4 -> fp32 convert times each
// position's scale (exact) and the top halves; the query, scaled per head by
// a power of two as below, stays bf16; each softmax weight enters as two bf16
// terms hi + lo (16 bits).
//
// A sliding-window branch (the decoder's window of recent tokens, kept as
// bf16 K and V rows beside the FP4 cache) joins the same softmax: its rows are
// extra blocks of 32 positions after the sparse ones, multiplied on the bf16
// matrix cores (K rows are the operands as loaded; V rows are staged in LDS
// and each lane reads its channel columns back transposed).
//
// The waves of a workgroup are merged through LDS in wave order. With NS > 1
// each workgroup writes its (max, sum, acc) state to the workspace with
// device-coherent stores, and the last workgroup of the row to arrive (one
// device-scope counter per row) merges the NS states in slice order and
// writes the output, then resets the counter. Workgroups are numbered row
// fastest, so all slices of a row run on the same XCD whenever the row count
// is a multiple of 8. The result does not depend on scheduling.
#include "attn_core.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kAttnTargetGroups = 256;          // one workgroup per CU of a 256-CU part
constexpr int kMaxSplits = 8;

// K: positions per row, counting the window's rows too (blocks of 32 each).
static int attn_splits(int64_t rows, int32_t K, int waves) {
    const int64_t nblk = (K + kBlk - 1) / kBlk;
    int64_t ns = (kAttnTargetGroups + rows - 1) / (rows > 0 ? rows : 1);
    const int64_t max_ns = (nblk + waves - 1) / waves;   // at least one block per wave
    if (ns > max_ns) ns = max_ns;
    if (ns > kMaxSplits) ns = kMaxSplits;
    if (ns < 1) ns = 1;
    return (int)ns;
}

// Launch shape: rows that fill the device one workgroup each run 4-wave
// workgroups (more of them resident per CU); rows split over several
// workgroups run 8-wave ones (fewer, shorter slices to merge).
struct AttnShape {
    int waves, ns;
};
static AttnShape attn_shape(int64_t rows, int32_t K) {
    const int ns4 = attn_splits(rows, K, 4);
    if (ns4 == 1) return AttnShape{4, 1};
    return AttnShape{8, attn_splits(rows, K, 8)};
}

static int32_t attn_blocks_positions(int32_t K, int32_t W) {
    return ((K + kBlk - 1) / kBlk + (W + kBlk - 1) / kBlk) * kBlk;
}

size_t attn_data_bytes(int64_t rows, int32_t K, int32_t W) {
    const int ns = attn_shape(rows, attn_blocks_positions(K, W)).ns;
    return ns > 1 ? (size_t)rows * ns * kPartFloats * 4 : 0;
}

template <int W, bool MX>
__global__ void __launch_bounds__(W * kWave, W == 4 ? 2 : 1)
k_sparse_attn(const uint16_t* __restrict__ q, int32_t rows_per_seq, int32_t H, const uint8_t* __restrict__ k_codes,
              const uint8_t* __restrict__ k_scales, const uint8_t* __restrict__ v_codes,
              const uint8_t* __restrict__ v_scales, int64_t N, int64_t cs, int64_t ss, const int32_t* __restrict__ idx,
              int64_t idx_stride, int32_t K, float scale, float* __restrict__ out, int32_t NS,
              uint32_t* __restrict__ counters, float* __restrict__ parts, int64_t rows,
              const uint16_t* __restrict__ win_k, const uint16_t* __restrict__ win_v, int64_t win_rs, int32_t Wn,
              const int32_t* __restrict__ win_len) {
    constexpr int kAttnWaves = W;
    constexpr int kAttnThreads = W * kWave;
    constexpr int kCh = kMaxHeads * kD / kAttnThreads;  // output channels per thread in the merges
    constexpr int kV4 = kCh / 4;
    static_assert(kCh % 4 == 0 && kD % kCh == 0, "merge tiling");
    __shared__ AttnLds<W> lds;
    __shared__ int s_last;

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int n = lane & 15, g = lane >> 4;
    const int64_t row = (int64_t)blockIdx.x % rows;            // row fastest: a row's slices share an XCD
    const int split = (int)((int64_t)blockIdx.x / rows);
    const int64_t seq = row / rows_per_seq;
    const int nblk_s = (K + kBlk - 1) / kBlk;                   // blocks of the sparse positions
    const int nblk = nblk_s + (Wn + kBlk - 1) / kBlk;           // then the window's blocks
    const int bps = (nblk + NS - 1) / NS;                       // blocks per slice
    const int b0 = split * bps, b1 = min(nblk, b0 + bps);
    const float sl2 = scale * kLog2e;

    // the query, loaded after the first block's position list so that the
    // first gathers do not wait for it
    uint4 qraw[4];
    auto load_q = [&]() { load_q_slice(q, row, H, n, g, qraw); };
    typename OpOf<MX>::type qb[4];
    bf16x8 qw[4];                               // the same scaled query in bf16 (window blocks)
    int qe = 0;                                 // head n's query is used as q * 2^-qe
    auto convert_q = [&]() { qe = convert_q_slice<MX>(qraw, H, n, qb, qw); };

    const int32_t* ip = idx + row * idx_stride;
    const KvBase kv{k_codes + seq * N * cs, k_scales + seq * N * ss, v_codes + seq * N * cs,
                    v_scales + seq * N * ss, cs, ss};

    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.f = 1.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- this wave's blocks k = 0 .. nb-1: block first + k*W. Issue order per
    // step k: position list of block k+2, gathers of block k+1, then the math
    // of block k - so two blocks of gathers are in flight and no load is waited
    // for before it is needed. Even and odd blocks use separate registers (the
    // loop is unrolled by two) and every load in the steady-state loop is
    // unconditional, so nothing in flight is copied and the compiler's wait
    // counts stay exact; the last one to three blocks are peeled.
    const int first = b0 + wave;
    const int nb_all = first < b1 ? (b1 - first + kAttnWaves - 1) / kAttnWaves : 0;
    const int b1s = min(b1, nblk_s);
    const int nb = first < b1s ? (b1s - first + kAttnWaves - 1) / kAttnWaves : 0;   // sparse blocks first
    if (nb > 0) {
        BlockRaw r0, r1;
        BlockPos p0 = load_pos(ip, first, K, lane);
        load_q();
        BlockPos p1 = load_pos(ip, first + min(1, nb - 1) * kAttnWaves, K, lane);
        gather<MX>(r0, p0, first, K, kv, N, lane, n, g);
        convert_q();
        st.f = ldexpf(1.f, qe);
        int k = 0;
        for (; k + 3 < nb; k += 2) {
            const int bk = first + k * kAttnWaves;
            p0 = load_pos(ip, bk + 2 * kAttnWaves, K, lane);
            gather<MX>(r1, p1, bk + kAttnWaves, K, kv, N, lane, n, g);
            attend_block<MX>(st, r0, lds.st[wave].sp, qb, sl2, lane, n, g);
            p1 = load_pos(ip, bk + 3 * kAttnWaves, K, lane);
            gather<MX>(r0, p0, bk + 2 * kAttnWaves, K, kv, N, lane, n, g);
            attend_block<MX>(st, r1, lds.st[wave].sp, qb, sl2, lane, n, g);
        }
        const int bk = first + k * kAttnWaves;
        const int rem = nb - k;                 // 1, 2 or 3
        if (rem == 1) {
            attend_block<MX>(st, r0, lds.st[wave].sp, qb, sl2, lane, n, g);
        } else if (rem == 2) {
            gather<MX>(r1, p1, bk + kAttnWaves, K, kv, N, lane, n, g);
            attend_block<MX>(st, r0, lds.st[wave].sp, qb, sl2, lane, n, g);
            attend_block<MX>(st, r1, lds.st[wave].sp, qb, sl2, lane, n, g);
        } else {
            p0 = load_pos(ip, bk + 2 * kAttnWaves, K, lane);
            gather<MX>(r1, p1, bk + kAttnWaves, K, kv, N, lane, n, g);
            attend_block<MX>(st, r0, lds.st[wave].sp, qb, sl2, lane, n, g);
            gather<MX>(r0, p0, bk + 2 * kAttnWaves, K, kv, N, lane, n, g);
            attend_block<MX>(st, r1, lds.st[wave].sp, qb, sl2, lane, n, g);
            attend_block<MX>(st, r0, lds.st[wave].sp, qb, sl2, lane, n, g);
        }
    } else {                                    // no sparse block: the query is needed as it stands
        load_q();
        convert_q();
        st.f = ldexpf(1.f, qe);
    }
    if (nb_all > nb) {                          // then this wave's window blocks
        const uint16_t* wkr = win_k + row * win_rs;
        const uint16_t* wvr = win_v + row * win_rs;
        const int len = win_len ? min(max(win_len[row], 0), Wn) : Wn;
        for (int k = nb; k < nb_all; ++k)
            attend_window_block(st, wkr, wvr, first + k * kAttnWaves - nblk_s, len, lds.st[wave], qw, sl2, n, g);
    }

    // ---- merge the waves in wave order (the staging areas are reused)
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float* dst = &lds.mg.acc[wave][n][8 * (4 * g + i)];
        *reinterpret_cast<f32x4*>(dst) = f32x4{st.acc[0][i], st.acc[1][i], st.acc[2][i], st.acc[3][i]};
        *reinterpret_cast<f32x4*>(dst + 4) = f32x4{st.acc[4][i], st.acc[5][i], st.acc[6][i], st.acc[7][i]};
    }
    if (g == 0) {
        lds.mg.m[wave][n] = st.m * sl2;         // scaled log2 units
        lds.mg.l[wave][n] = st.l;
        if (wave == 0) lds.mg.f[n] = st.f;
    }
    __syncthreads();

    // this thread's head h and channels c0 .. c0 + kCh - 1
    const int h = tid / (kD / kCh);
    const int c0 = (tid % (kD / kCh)) * kCh;
    const float fh = lds.mg.f[h];
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kAttnWaves; ++w) M = fmaxf(M, lds.mg.m[w][h]);
    float L = 0.f;
    f32x4 o[kV4];
#pragma unroll
    for (int v = 0; v < kV4; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < kAttnWaves; ++w) {
            const float mw = lds.mg.m[w][h];
            const float wt = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * fh);
            L += wt * lds.mg.l[w][h];
#pragma unroll
            for (int v = 0; v < kV4; ++v) o[v] += wt * *reinterpret_cast<const f32x4*>(&lds.mg.acc[w][h][c0 + 4 * v]);
        }
    }

    float* orow = out + row * (int64_t)H * kD;
    if (NS == 1) {
        if (h < H) {
            const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
            for (int v = 0; v < kV4; ++v) *reinterpret_cast<f32x4*>(orow + h * kD + c0 + 4 * v) = o[v] * inv;
        }
        return;
    }

    // ---- NS > 1: publish this slice's state, the last slice of the row merges
    uint32_t* ctr = counters + row;
    float* part_row = parts + row * NS * kPartFloats;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(part_row, (short)0, NS * kPartFloats * 4, kRsrcWord3);
    const int mine = split * kPartFloats * 4;
#pragma unroll
    for (int v = 0; v < kV4; ++v)
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[v]), rs, mine + (h * kD + c0 + 4 * v) * 4, 0,
                                               kCoherent);
    if (c0 == 0) {
        const f32x2 ml = {M, L};
        __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), rs,
                                             mine + (kMaxHeads * kD + 2 * h) * 4, 0, kCoherent);
    }
    wave_drain();
    __syncthreads();
    if (tid == 0) s_last = (add_rlx(ctr, 1u) == (uint32_t)(NS - 1));
    __syncthreads();
    if (!s_last) return;

    // slices beyond NS read past the resource's range and return zeros
    u32x4 pa[kMaxSplits][kV4];
    u32x2 pml[kMaxSplits];
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) {
#pragma unroll
        for (int v = 0; v < kV4; ++v)
            pa[s][v] = __builtin_amdgcn_raw_buffer_load_b128(rs, (s * kPartFloats + h * kD + c0 + 4 * v) * 4, 0, kCoherent);
        pml[s] = __builtin_amdgcn_raw_buffer_load_b64(rs, (s * kPartFloats + kMaxHeads * kD + 2 * h) * 4, 0, kCoherent);
    }
    float MM = -INFINITY;
#pragma unroll
    for (int s = 0; s < kMaxSplits; ++s) MM = fmaxf(MM, s < NS ? __uint_as_float(pml[s].x) : -INFINITY);
    float LL = 0.f;
    f32x4 oo[kV4];
#pragma unroll
    for (int v = 0; v < kV4; ++v) oo[v] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (MM != -INFINITY) {
#pragma unroll
        for (int s = 0; s < kMaxSplits; ++s) {
            const float ms = __uint_as_float(pml[s].x);
            const float wt = (s >= NS || ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms - MM) * fh);
            LL += wt * __uint_as_float(pml[s].y);
#pragma unroll
            for (int v = 0; v < kV4; ++v) oo[v] += wt * __builtin_bit_cast(f32x4, pa[s][v]);
        }
    }
    if (h < H) {
        const float inv = LL > 0.f ? 1.f / LL : 0.f;
#pragma unroll
        for (int v = 0; v < kV4; ++v) *reinterpret_cast<f32x4*>(orow + h * kD + c0 + 4 * v) = oo[v] * inv;
    }
    if (tid == 0) st_rlx(ctr, 0u);              // ready for the next launch
}

int launch_attn_scratch(const AttnArgs& a, uint32_t* counters, void* parts, size_t parts_bytes, hipStream_t stream) {
    if (a.rows == 0) return OK;
    const AttnShape sh = attn_shape(a.rows, attn_blocks_positions(a.K, a.Wn));
    const int ns = sh.ns;
    if (parts_bytes < attn_data_bytes(a.rows, a.K, a.Wn)) return fail(WORKSPACE, "attention workspace too small");
    if (ns > 1 && a.rows > kAttnCtrlWords) return fail(INVALID, "attention: split rows exceed the counter table");
    const int64_t groups = a.rows * ns;
    if (groups > 0x7FFFFFFFll) return fail(INVALID, "attention: too many query rows");
    auto fn = a.mx ? (sh.waves == 4 ? k_sparse_attn<4, true> : k_sparse_attn<8, true>)
                   : (sh.waves == 4 ? k_sparse_attn<4, false> : k_sparse_attn<8, false>);
    hipLaunchKernelGGL(fn, dim3((unsigned)groups), dim3(sh.waves * kWave), 0, stream, a.q, a.rows_per_seq,
                       a.H, a.k_codes, a.k_scales, a.v_codes, a.v_scales, a.N, a.code_stride, a.scale_stride, a.idx,
                       a.idx_stride, a.K, a.scale, a.out, ns, counters, reinterpret_cast<float*>(parts), a.rows,
                       a.win_k, a.win_v, a.win_rs, a.Wn, a.win_len);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_sparse_attn");
}

int launch_attn(const AttnArgs& a, void* ws_ctrl, void* ws_data, size_t data_bytes, hipStream_t stream) {
    return launch_attn_scratch(a, reinterpret_cast<uint32_t*>(ws_ctrl) + kAttnCtrlOffsetWords, ws_data, data_bytes,
                               stream);
}

}  // namespace csa2
