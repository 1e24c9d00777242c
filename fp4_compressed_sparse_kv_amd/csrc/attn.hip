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
#include "device.hpp"
#include "internal.hpp"

namespace csa2 {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBlk = 32;
constexpr int kMaxHeads = 16;
constexpr int kD = 128;
constexpr int kAttnTargetGroups = 256;          // one workgroup per CU of a 256-CU part
constexpr int kMaxSplits = 8;
constexpr int kPartFloats = kMaxHeads * kD + 2 * kMaxHeads;   // per (row, slice): acc [16][128], (m, l) [16][2]
constexpr int kVRowBytes = 80;                  // staged V row: 64 code bytes + pad (conflict-free dword reads)
constexpr int kMergeStride = kD + 4;
constexpr float kLog2e = 1.4426950408889634f;

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

// 8 FP4 codes (one dword) of one 32-channel MXFP4 block -> 8 bf16 with the
// block's E8M0 scale (an fp32 whose exponent field is the scale byte).
__device__ __forceinline__ bf16x8 dq8_mx(uint32_t w, float X) {
    const bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, X, 0);
    const bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, X, 1);
    const bf16x2 c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, X, 2);
    const bf16x2 d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, X, 3);
    return bf16x8{a.x, a.y, b.x, b.y, c.x, c.y, d.x, d.y};
}

__device__ __forceinline__ float e8m0_f32(uint32_t b) { return __uint_as_float((b & 0xFFu) << 23); }

// Top halves of two fp32 whose values are exact in bf16, as a bf16 pair.
__device__ __forceinline__ uint32_t pack_hi(float lo, float hi) {
    return (__float_as_uint(lo) >> 16) | (__float_as_uint(hi) & 0xFFFF0000u);
}

__device__ __forceinline__ f32x4 mfma16(const f16x8& a, const f16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const bf16x8& a, const bf16x8& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Matrix-core operand type of a cache format: f16 (E4M3 scales), bf16 (MXFP4).
template <bool MX> struct OpOf { using type = f16x8; };
template <> struct OpOf<true> { using type = bf16x8; };

// Over the four rows of 16 lanes (lanes n, 16 + n, 32 + n, 48 + n): the
// maximum and the sum, in every lane of the group. v_permlane16_swap and
// v_permlane32_swap hand each lane the value of lane ^ 16 and lane ^ 32 as one
// of the pair they return (the other is its own), so op(pair) is the combine
// with that lane; both lanes of a pair compute the same value.
__device__ __forceinline__ float rows_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

struct KvBase {
    const uint8_t *kc, *ks, *vc, *vs;           // this sequence's planes
    int64_t cs, ss;
};

// One lane's loads for a block of 32 positions. Lane (n, g) holds bytes
// 16g..16g+15 of the K and V code rows of positions n and 16 + n; lanes < 32
// hold the K and V scale bytes of position `lane`.
struct BlockRaw {
    uint4 k[2], v[2];
    uint2 ks, vs;
    int32_t pos;                                // lanes < 32: position of entry `lane`, -1 if none
};

struct Stage {                                  // one wave's LDS staging area
    uint8_t v[kBlk][kVRowBytes];
    uint8_t ks[kBlk][8];
    uint8_t vs[kBlk][8];
};

constexpr int kWinRow = kD + 8;                 // staged window V row (bf16): 128 channels + pad
union WaveStage {                               // a wave's area: FP4 blocks, or a window block's V rows
    Stage sp;
    uint16_t wv[kBlk][kWinRow];
};

template <int W>
struct MergeArea {
    float acc[W][kMaxHeads][kMergeStride];
    float m[W][kMaxHeads];
    float l[W][kMaxHeads];
    float f[kMaxHeads];                         // per head: 2^e, the query's scale-back factor
};

template <int W>
union AttnLds {
    WaveStage st[W];
    MergeArea<W> mg;
};

// Raw position-list entries a lane of block `blk` needs: entries n and 16 + n
// (its code rows) and entry lane % 32 (the scale record it loads). Each lane
// loads them itself - lanes with the same entry read the same word - so no
// cross-lane move waits on the list. Entries past K read a clamped in-range
// entry and are discarded later. The loads are unconditional and their values
// are checked only where they are consumed, so they can stay in flight.
struct BlockPos {
    int32_t a, b, s;
};
__device__ __forceinline__ BlockPos load_pos(const int32_t* ip, int blk, int K, int lane) {
    const int n = lane & 15;
    BlockPos p;
    p.a = ip[min(blk * kBlk + n, K - 1)];
    p.b = ip[min(blk * kBlk + 16 + n, K - 1)];
    p.s = ip[min(blk * kBlk + (lane & (kBlk - 1)), K - 1)];
    return p;
}

// Issue the gathers of one block. Every load is unconditional: an entry that
// is padding (past K, negative or >= N) reads position 0 of the sequence
// instead, and its scales are zeroed when the block is staged, so it
// dequantizes to exact zeros and is masked out of the softmax.
template <bool MX>
__device__ __forceinline__ void gather(BlockRaw& r, const BlockPos& bp, int blk, int K, const KvBase& kv, int64_t N,
                                       int lane, int n, int g) {
    const bool ok = lane < kBlk && blk * kBlk + lane < K && bp.s >= 0 && (int64_t)bp.s < N;
    const int32_t safe = ok ? bp.s : 0;
    const int32_t p0 = (blk * kBlk + n < K && bp.a >= 0 && (int64_t)bp.a < N) ? bp.a : 0;
    const int32_t p1 = (blk * kBlk + 16 + n < K && bp.b >= 0 && (int64_t)bp.b < N) ? bp.b : 0;
    r.k[0] = *reinterpret_cast<const uint4*>(kv.kc + p0 * kv.cs + 16 * g);
    r.v[0] = *reinterpret_cast<const uint4*>(kv.vc + p0 * kv.cs + 16 * g);
    r.k[1] = *reinterpret_cast<const uint4*>(kv.kc + p1 * kv.cs + 16 * g);
    r.v[1] = *reinterpret_cast<const uint4*>(kv.vc + p1 * kv.cs + 16 * g);
    if constexpr (MX) {                         // 4 E8M0 bytes per plane (128 channels)
        r.ks = make_uint2(*reinterpret_cast<const uint32_t*>(kv.ks + safe * kv.ss), 0u);
        r.vs = make_uint2(*reinterpret_cast<const uint32_t*>(kv.vs + safe * kv.ss), 0u);
    } else {
        r.ks = *reinterpret_cast<const uint2*>(kv.ks + safe * kv.ss);
        r.vs = *reinterpret_cast<const uint2*>(kv.vs + safe * kv.ss);
    }
    r.pos = ok ? bp.s : -1;
}

struct WaveState {
    float m, l;                                 // head n (same in the 4 lane groups), scaled log2 units
    float f;                                    // head n: 2^e, scaled log2 units -> log2 units
    f32x4 acc[8];                               // acc[t][i] = unnormalized out[n][8*(4g+i) + t]
};

// Two E4M3 bytes (bits 0..15 of w) -> two f16, exactly (the hardware decode
// to fp32 is exact and every E4M3 value is an f16 value).
__device__ __forceinline__ f16x2 e4m3x2_to_f16(uint32_t w) {
    const f32x2 f = __builtin_amdgcn_cvt_pk_f32_fp8(w, false);
    return __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(f.x, f.y));
}

template <bool MX>
__device__ __forceinline__ void attend_block(WaveState& st, const BlockRaw& r, Stage& sg,
                                             const typename OpOf<MX>::type (&qb)[4], float sl2, int lane, int n, int g) {
    using OpT = typename OpOf<MX>::type;
    // ---- stage V codes and scales; this wave alone uses `sg`, and its LDS
    // accesses complete in order, so no barrier is needed
    *reinterpret_cast<uint4*>(&sg.v[n][16 * g]) = r.v[0];
    *reinterpret_cast<uint4*>(&sg.v[16 + n][16 * g]) = r.v[1];
    if (lane < kBlk) {
        *reinterpret_cast<uint2*>(&sg.ks[lane][0]) = r.ks;
        *reinterpret_cast<uint2*>(&sg.vs[lane][0]) = r.vs;
    }
    __builtin_amdgcn_wave_barrier();
    // bit p: position p of the block is a real entry (padding is masked out of
    // the softmax; its codes and scales are those of position 0, all finite)
    const uint32_t vmask = (uint32_t)__builtin_amdgcn_ballot_w64(r.pos >= 0);
    // this lane's softmax columns i: positions 4g + i (i < 4), 16 + 4g + i - 4 (i >= 4);
    // its V channels 8n .. 8n+7 lie in scale group n/2 (16 channels) or block n/4 (32)
    uint32_t vw[8], vsb[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int p = (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4);
        vw[i] = *reinterpret_cast<const uint32_t*>(&sg.v[p][4 * n]);
        vsb[i] = MX ? sg.vs[p][n >> 2] : sg.vs[p][n >> 1];
    }

    // ---- S^T = K_hat Q^T (a lane's K channels 32g .. 32g+31: two E4M3 groups, one MXFP4 block)
    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
        const uint32_t w[4] = {r.k[mb].x, r.k[mb].y, r.k[mb].z, r.k[mb].w};
        if constexpr (MX) {
            const float X = e8m0_f32(sg.ks[16 * mb + n][g]);
#pragma unroll
            for (int s = 0; s < 4; ++s) sacc[mb] = mfma16(dq8_mx(w[s], X), qb[s], sacc[mb]);
        } else {
            const f16x2 ks = e4m3x2_to_f16(*reinterpret_cast<const uint16_t*>(&sg.ks[16 * mb + n][2 * g]));
#pragma unroll
            for (int s = 0; s < 4; ++s) sacc[mb] = mfma16(dq8(w[s], s < 2 ? ks.x : ks.y), qb[s], sacc[mb]);
        }
    }

    // ---- online softmax for head n over the 8 positions this lane holds
    const uint32_t mlo = vmask >> (4 * g), mhi = vmask >> (16 + 4 * g);
    float lg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float sv = (i < 4) ? sacc[0][i] : sacc[1][i - 4];
        const uint32_t bit = (i < 4) ? (mlo >> i) & 1u : (mhi >> (i - 4)) & 1u;
        lg[i] = bit ? sv * sl2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])), fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));
    mx = rows_max(mx);
    const float m_old = st.m;
    const float m_new = fmaxf(m_old, mx);
    // weights 2^((lg - m_new) * 2^e): the hardware exp2 flushes results below
    // 2^-126 to zero, far below what can matter against the maximum weight 1
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f((lg[i] - mref) * st.f);
        psum += p[i];
    }
    uint32_t ph[4], pl[4];                      // p = hi + lo: f16 (~22 bits) or bf16 (16 bits) pairs
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        if constexpr (MX) {
            const float h0 = __uint_as_float(__float_as_uint(p[i]) & 0xFFFF0000u);
            const float h1 = __uint_as_float(__float_as_uint(p[i + 1]) & 0xFFFF0000u);
            ph[i / 2] = pack_hi(h0, h1);
            pl[i / 2] = pack_hi(p[i] - h0, p[i + 1] - h1);
        } else {
            const f16x2 hi = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[i], p[i + 1]));
            const f16x2 lo = __builtin_bit_cast(f16x2, __builtin_amdgcn_cvt_pkrtz(p[i] - (float)hi.x, p[i + 1] - (float)hi.y));
            ph[i / 2] = __builtin_bit_cast(uint32_t, hi);
            pl[i / 2] = __builtin_bit_cast(uint32_t, lo);
        }
    }
    const OpT pb_hi = __builtin_bit_cast(OpT, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const OpT pb_lo = __builtin_bit_cast(OpT, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    psum = rows_sum(psum);
    const float alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - mref) * st.f);
    st.l = st.l * alpha + psum;
    st.m = m_new;
    // the running sums need rescaling only where the maximum grew after the
    // first block (before it they are zero)
    if (__builtin_amdgcn_ballot_w64(m_old != -INFINITY && alpha != 1.f) != 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st.acc[t] = st.acc[t] * alpha;
    }

    // ---- out^T += V_hat^T P^T: MFMA t covers channels 8m + t; its operand
    // element i is channel 8n + t of position column i. Codes of columns
    // 2k and 2k+1 are interleaved nibble-wise so that one convert yields the
    // (column 2k, column 2k+1) pair of a channel, then each value takes its
    // own position's scale: a packed f16 product with the E4M3 scale pair, or
    // fp32 products with the two E8M0 scales (exact) and the bf16 top halves.
    uint32_t va[8][4];                          // va[t][k] = (V[2k][8n+t], V[2k+1][8n+t])
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t wa = vw[2 * k], wb = vw[2 * k + 1];
        const uint32_t ev = (wa & 0x0F0F0F0Fu) | ((wb << 4) & 0xF0F0F0F0u);   // byte j: channel 2j of a | of b
        const uint32_t od = ((wa >> 4) & 0x0F0F0F0Fu) | (wb & 0xF0F0F0F0u);  // byte j: channel 2j+1
        if constexpr (MX) {
            const float X0 = e8m0_f32(vsb[2 * k]), X1 = e8m0_f32(vsb[2 * k + 1]);
            auto pair = [&](f32x2 e) { return pack_hi(e.x * X0, e.y * X1); };
            va[0][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 0));
            va[2][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 1));
            va[4][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 2));
            va[6][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(ev, 1.0f, 3));
            va[1][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 0));
            va[3][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 1));
            va[5][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 2));
            va[7][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f32_fp4(od, 1.0f, 3));
        } else {
            const f16x2 sp = e4m3x2_to_f16(vsb[2 * k] | (vsb[2 * k + 1] << 8));
            auto pair = [&](f16x2 e) { return __builtin_bit_cast(uint32_t, e * sp); };
            va[0][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 0));
            va[2][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 1));
            va[4][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 2));
            va[6][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(ev, 1.0f, 3));
            va[1][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 0));
            va[3][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 1));
            va[5][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 2));
            va[7][k] = pair(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(od, 1.0f, 3));
        }
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        const OpT a = __builtin_bit_cast(OpT, make_uint4(va[t][0], va[t][1], va[t][2], va[t][3]));
        st.acc[t] = mfma16(a, pb_hi, st.acc[t]);
        st.acc[t] = mfma16(a, pb_lo, st.acc[t]);
    }
}

// One block of 32 window rows (rows 32 wb .. of this query row's window; rows
// at or past `len` are masked). Lane (n, g) loads channels 32g..32g+31 of K
// rows n and 16 + n (its S^T operands as they are) and of the same V rows,
// which it stages in LDS; the softmax is attend_block's; each lane then reads
// channels 8n..8n+7 of its 8 position columns and transposes them into the
// PV operands. qw: the query (scaled by 2^-qe like the sparse part) in bf16.
__device__ __forceinline__ void attend_window_block(WaveState& st, const uint16_t* wk, const uint16_t* wv, int wb,
                                                    int len, WaveStage& sg, const bf16x8 (&qw)[4], float sl2,
                                                    int n, int g) {
    const int lim = max(len - 1, 0);
    const int r0 = min(32 * wb + n, lim), r1 = min(32 * wb + 16 + n, lim);
    uint4 kq[2][4], vq[2][4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        kq[0][s] = *reinterpret_cast<const uint4*>(wk + (int64_t)r0 * kD + 32 * g + 8 * s);
        kq[1][s] = *reinterpret_cast<const uint4*>(wk + (int64_t)r1 * kD + 32 * g + 8 * s);
        vq[0][s] = *reinterpret_cast<const uint4*>(wv + (int64_t)r0 * kD + 32 * g + 8 * s);
        vq[1][s] = *reinterpret_cast<const uint4*>(wv + (int64_t)r1 * kD + 32 * g + 8 * s);
    }
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        *reinterpret_cast<uint4*>(&sg.wv[n][32 * g + 8 * s]) = vq[0][s];
        *reinterpret_cast<uint4*>(&sg.wv[16 + n][32 * g + 8 * s]) = vq[1][s];
    }
    __builtin_amdgcn_wave_barrier();
    const int nvalid = min(max(len - 32 * wb, 0), kBlk);
    const uint32_t vmask = nvalid >= kBlk ? 0xFFFFFFFFu : ((1u << nvalid) - 1u);

    f32x4 sacc[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int s = 0; s < 4; ++s) sacc[mb] = mfma16(__builtin_bit_cast(bf16x8, kq[mb][s]), qw[s], sacc[mb]);

    const uint32_t mlo = vmask >> (4 * g), mhi = vmask >> (16 + 4 * g);
    float lg[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float sv = (i < 4) ? sacc[0][i] : sacc[1][i - 4];
        const uint32_t bit = (i < 4) ? (mlo >> i) & 1u : (mhi >> (i - 4)) & 1u;
        lg[i] = bit ? sv * sl2 : -INFINITY;
    }
    float mx = fmaxf(fmaxf(fmaxf(lg[0], lg[1]), fmaxf(lg[2], lg[3])), fmaxf(fmaxf(lg[4], lg[5]), fmaxf(lg[6], lg[7])));
    mx = rows_max(mx);
    const float m_old = st.m;
    const float m_new = fmaxf(m_old, mx);
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    float p[8], psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f((lg[i] - mref) * st.f);
        psum += p[i];
    }
    uint32_t ph[4], pl[4];                      // p = hi + lo as bf16 pairs (16 bits)
#pragma unroll
    for (int i = 0; i < 8; i += 2) {
        const float h0 = __uint_as_float(__float_as_uint(p[i]) & 0xFFFF0000u);
        const float h1 = __uint_as_float(__float_as_uint(p[i + 1]) & 0xFFFF0000u);
        ph[i / 2] = pack_hi(h0, h1);
        pl[i / 2] = pack_hi(p[i] - h0, p[i + 1] - h1);
    }
    const bf16x8 pb_hi = __builtin_bit_cast(bf16x8, make_uint4(ph[0], ph[1], ph[2], ph[3]));
    const bf16x8 pb_lo = __builtin_bit_cast(bf16x8, make_uint4(pl[0], pl[1], pl[2], pl[3]));
    psum = rows_sum(psum);
    const float alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - mref) * st.f);
    st.l = st.l * alpha + psum;
    st.m = m_new;
    if (__builtin_amdgcn_ballot_w64(m_old != -INFINITY && alpha != 1.f) != 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st.acc[t] = st.acc[t] * alpha;
    }

    // V: channels 8n..8n+7 (16 bytes) of each of this lane's 8 position columns
    uint4 vr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int pp = (i < 4) ? (4 * g + i) : (16 + 4 * g + i - 4);
        vr[i] = *reinterpret_cast<const uint4*>(&sg.wv[pp][8 * n]);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) {
        uint32_t va[4];                         // (V[2k][8n+t], V[2k+1][8n+t]) bf16 pairs
        const uint32_t sel = (t & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint4 a = vr[2 * k], b = vr[2 * k + 1];
            const uint32_t wa = (t >> 1) == 0 ? a.x : (t >> 1) == 1 ? a.y : (t >> 1) == 2 ? a.z : a.w;
            const uint32_t wb2 = (t >> 1) == 0 ? b.x : (t >> 1) == 1 ? b.y : (t >> 1) == 2 ? b.z : b.w;
            va[k] = __builtin_amdgcn_perm(wb2, wa, sel);
        }
        const bf16x8 a8 = __builtin_bit_cast(bf16x8, make_uint4(va[0], va[1], va[2], va[3]));
        st.acc[t] = mfma16(a8, pb_hi, st.acc[t]);
        st.acc[t] = mfma16(a8, pb_lo, st.acc[t]);
    }
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

    // query as the B operand of S^T = K_hat Q^T: lane (n, g), k-step s holds
    // q[head n][channel 32g + 8s + i], i = 0..7; heads >= H read head H - 1
    // and are zeroed when converted. Loaded after the first block's position
    // list, so the first gathers do not wait for it.
    uint4 qraw[4];
    auto load_q = [&]() {
#pragma unroll
        for (int s = 0; s < 4; ++s)
            qraw[s] = *reinterpret_cast<const uint4*>(q + (row * H + min(n, H - 1)) * (int64_t)kD + 32 * g + 8 * s);
    };
    typename OpOf<MX>::type qb[4];
    bf16x8 qw[4];                               // the same scaled query in bf16 (window blocks)
    int qe = 0;                                 // head n's query is used as q * 2^-qe
    auto convert_q = [&]() {
        uint32_t mb = 0;                        // largest |q| of this lane's 32 elements (bf16 bits)
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            const uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) mb = max(mb, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
        }
        const float qmax = rows_max(bf16_bits_to_f32(mb));   // over the head's 128 channels
        int ex = 0;
        (void)frexpf(qmax, &ex);                // qmax = m * 2^ex, m in [0.5, 1)
        qe = qmax > 0.f ? ex - 15 : 0;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float a = n < H ? ldexpf(bf16_bits_to_f32(w[i] & 0xFFFFu), -qe) : 0.f;
                const float b = n < H ? ldexpf(bf16_bits_to_f32(w[i] >> 16), -qe) : 0.f;
                w[i] = pack_hi(a, b);           // a bf16 times a power of two: its top half (exact unless subnormal)
                if constexpr (!MX) {
                    qb[s][2 * i + 0] = (_Float16)a;
                    qb[s][2 * i + 1] = (_Float16)b;
                }
            }
            qw[s] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
            if constexpr (MX) qb[s] = qw[s];
        }
    };

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
        lds.mg.m[wave][n] = st.m;
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
