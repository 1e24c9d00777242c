// Building blocks of the sparse FP4 attention shared by its kernels: the
// per-wave gather, dequantize and matrix-core step over a block of 32
// positions, the sliding-window block, the query conversion and the
// merging of partial softmax states. The method and the exactness of each
// step are described where the attention kernel is defined.
#pragma once

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
constexpr int kPartFloats = kMaxHeads * kD + 2 * kMaxHeads;   // per (row, slice): acc [16][128], (m, l) [16][2]
static_assert(kPartFloats == kAttnPartFloats, "partial state size");
constexpr int kVRowBytes = 80;                  // staged V row: 64 code bytes + pad (conflict-free dword reads)
constexpr int kMergeStride = kD + 4;
constexpr float kLog2e = 1.4426950408889634f;

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

struct alignas(16) Stage {                      // one wave's LDS staging area
    uint8_t v[kBlk][kVRowBytes];
    uint8_t ks[kBlk][8];
    uint8_t vs[kBlk][8];
};

constexpr int kWinRow = kD + 8;                 // staged window V row (bf16): 128 channels + pad
union alignas(16) WaveStage {                   // a wave's area: FP4 blocks, or a window block's V rows
    Stage sp;
    uint16_t wv[kBlk][kWinRow];
};

template <int W>
struct alignas(16) MergeArea {
    float acc[W][kMaxHeads][kMergeStride];
    float m[W][kMaxHeads];
    float l[W][kMaxHeads];
    float f[kMaxHeads];                         // per head: 2^e, the query's scale-back factor
};

template <int W>
union alignas(16) AttnLds {                     // 16-byte rows: staged with 16-byte LDS accesses
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
    float m;                                    // head n (same in the 4 lane groups): running maximum score,
                                                // in the units of q * 2^-e (times scale * log2(e): scaled log2 units)
    float l;                                    // running sum of the weights
    float f;                                    // head n: 2^e, scaled log2 units -> log2 units
    f32x4 acc[8];                               // acc[t][i] = unnormalized out[n][8*(4g+i) + t]
};

// Online softmax of one block of 32 positions for head n: lanes n, 16 + n,
// 32 + n and 48 + n hold its scores s (units of q * 2^-e) at positions
// 4g + i (i < 4) and 16 + 4g + i - 4 (i >= 4). Weights p = 2^((s - m) * c)
// with c = scale * log2(e) * 2^e (a product with a power of two: exact); the
// difference is formed before the product, so neither huge nor tiny queries
// overflow. vmask bit p: position p is real (all set: nothing to mask). Sets
// p, their sum over the head's 32 positions, and rescales the running state.
__device__ __forceinline__ void block_softmax(WaveState& st, const f32x4 (&sacc)[2], uint32_t vmask, float sl2, int g,
                                              float (&p)[8], float& psum) {
    float sc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) sc[i] = (i < 4) ? sacc[0][i] : sacc[1][i - 4];
    if (vmask != 0xFFFFFFFFu) {                 // the same in every lane: a block with padding
        const uint32_t mlo = vmask >> (4 * g), mhi = vmask >> (16 + 4 * g);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t bit = (i < 4) ? (mlo >> i) & 1u : (mhi >> (i - 4)) & 1u;
            sc[i] = bit ? sc[i] : -INFINITY;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
    mx = rows_max(mx);
    const float c = sl2 * st.f;
    const float m_old = st.m;
    const float m_new = fmaxf(m_old, mx);
    // the hardware exp2 flushes results below 2^-126 to zero, far below what
    // can matter against the maximum weight 1
    const float mref = m_new == -INFINITY ? 0.f : m_new;
    psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        p[i] = __builtin_amdgcn_exp2f((sc[i] - mref) * c);
        psum += p[i];
    }
    psum = rows_sum(psum);
    const float alpha = m_old == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((m_old - mref) * c);
    st.l = st.l * alpha + psum;
    st.m = m_new;
    // the running sums need rescaling only where the maximum grew after the
    // first block (before it they are zero)
    if (__builtin_amdgcn_ballot_w64(m_old != -INFINITY && alpha != 1.f) != 0) {
#pragma unroll
        for (int t = 0; t < 8; ++t) st.acc[t] = st.acc[t] * alpha;
    }
}

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
    float p[8], psum;
    block_softmax(st, sacc, vmask, sl2, g, p, psum);
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

    float p[8], psum;
    block_softmax(st, sacc, vmask, sl2, g, p, psum);
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


// ------------------------------------------------------------------ query

// The query as the B operand of S^T = K_hat Q^T: lane (n, g), k-step s holds
// q[head n][channel 32g + 8s + i], i = 0..7; heads >= H read head H - 1 (and
// are zeroed when converted).
__device__ __forceinline__ void load_q_slice(const uint16_t* q, int64_t row, int32_t H, int n, int g, uint4 (&qraw)[4]) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
        qraw[s] = *reinterpret_cast<const uint4*>(q + (row * H + min(n, H - 1)) * (int64_t)kD + 32 * g + 8 * s);
}

// Head n's query scaled by 2^-qe (qe from its largest |q|, so that element
// lands in [2^14, 2^15)) in the matrix-core operand type of the cache format
// (qb) and in bf16 (qw); returns qe. Each bf16 times a power of two is exact
// in bf16 unless it falls below the normal range, and exact in f16 within 2^28
// of the head's largest element.
template <bool MX>
__device__ __forceinline__ int convert_q_slice(const uint4 (&qraw)[4], int32_t H, int n, typename OpOf<MX>::type (&qb)[4],
                                               bf16x8 (&qw)[4]) {
    uint32_t mb = 0;                            // largest |q| of this lane's 32 elements (bf16 bits)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) mb = max(mb, max(w[i] & 0x7FFFu, (w[i] >> 16) & 0x7FFFu));
    }
    const float qmax = rows_max(bf16_bits_to_f32(mb));   // over the head's 128 channels
    int ex = 0;
    (void)frexpf(qmax, &ex);                    // qmax = m * 2^ex, m in [0.5, 1)
    const int qe = qmax > 0.f ? ex - 15 : 0;
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        uint32_t w[4] = {qraw[s].x, qraw[s].y, qraw[s].z, qraw[s].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const float a = n < H ? ldexpf(bf16_bits_to_f32(w[i] & 0xFFFFu), -qe) : 0.f;
            const float b = n < H ? ldexpf(bf16_bits_to_f32(w[i] >> 16), -qe) : 0.f;
            w[i] = pack_hi(a, b);               // a bf16 times a power of two: its top half (exact unless subnormal)
            if constexpr (!MX) {
                qb[s][2 * i + 0] = (_Float16)a;
                qb[s][2 * i + 1] = (_Float16)b;
            }
        }
        qw[s] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
        if constexpr (MX) qb[s] = qw[s];
    }
    return qe;
}

// ------------------------------------------------- attention in a selection

// An attention fused into a selection kernel (AttnFuse, internal.hpp): every
// workgroup of a row attends to the positions it selected, publishes its
// partial softmax state, and after a row barrier merges the row's states for
// a share of the heads.

constexpr int kFuseWaves = 8;                   // waves of a workgroup that attend

// This workgroup's partial state for query `row` over the n positions pos[0..n)
// (any address space; position order is the summation order): waves
// 0..kFuseWaves-1 take blocks of 32 (wave w: blocks w, w + kFuseWaves, ...),
// their states are merged in wave order, and the result - per head the
// running maximum and sum (scaled log2 units) and the unnormalized output -
// is written to `part` with device-coherent stores, or (direct: the row has
// no other workgroup) normalized straight to the output. All threads of the
// workgroup (at least kFuseWaves waves) call it; it ends with the stores
// drained. lds.mg.f[h] keeps head h's scale-back factor 2^qe.
__device__ __forceinline__ void fused_attn_partial(const AttnFuse& af, int64_t row, const int32_t* pos, int n,
                                                   AttnLds<kFuseWaves>& lds, float* part, bool direct = false) {
    constexpr int W = kFuseWaves;
    constexpr int kCh = kMaxHeads * kD / (W * kWave);   // output channels per merging thread
    constexpr int kV4 = kCh / 4;
    static_assert(kCh % 4 == 0, "merge tiling");
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int nn = lane & 15, g = lane >> 4;
    const int64_t seq = row / af.rows_per_seq;
    const KvBase kv{af.k_codes + seq * af.N * af.cs, af.k_scales + seq * af.N * af.ss,
                    af.v_codes + seq * af.N * af.cs, af.v_scales + seq * af.N * af.ss, af.cs, af.ss};
    const float sl2 = af.scale * kLog2e;
    WaveState st;
    st.m = -INFINITY;
    st.l = 0.f;
    st.f = 1.f;
#pragma unroll
    for (int t = 0; t < 8; ++t) st.acc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (wave < W) {
        // one block in flight per wave (registers are scarce in a 1024-thread
        // workgroup; a chunk's share is usually one block per wave)
        const int nblk = (n + kBlk - 1) / kBlk;
        uint4 qraw[4];
        f16x8 qb[4];
        bf16x8 qw[4];
        BlockRaw r;
        int b = wave;
        if (b < nblk) {                         // the first gathers, then the query
            const BlockPos bp = load_pos(pos, b, n, lane);
            gather<false>(r, bp, b, n, kv, af.N, lane, nn, g);
        }
        load_q_slice(af.q, row, af.H, nn, g, qraw);
        st.f = ldexpf(1.f, convert_q_slice<false>(qraw, af.H, nn, qb, qw));
        for (; b < nblk; b += W) {
            if (b > wave) {
                const BlockPos bp = load_pos(pos, b, n, lane);
                gather<false>(r, bp, b, n, kv, af.N, lane, nn, g);
            }
            attend_block<false>(st, r, lds.st[wave].sp, qb, sl2, lane, nn, g);
        }
    }
    // merge the waves in wave order (the staging areas are reused)
    __syncthreads();
    if (wave < W) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            float* dst = &lds.mg.acc[wave][nn][8 * (4 * g + i)];
            *reinterpret_cast<f32x4*>(dst) = f32x4{st.acc[0][i], st.acc[1][i], st.acc[2][i], st.acc[3][i]};
            *reinterpret_cast<f32x4*>(dst + 4) = f32x4{st.acc[4][i], st.acc[5][i], st.acc[6][i], st.acc[7][i]};
        }
        if (g == 0) {
            lds.mg.m[wave][nn] = st.m * sl2;    // scaled log2 units
            lds.mg.l[wave][nn] = st.l;
            if (wave == 0) lds.mg.f[nn] = st.f;
        }
    }
    __syncthreads();
    if (tid < W * kWave) {
        const int h = tid / (kD / kCh);
        const int c0 = (tid % (kD / kCh)) * kCh;
        const float fh = lds.mg.f[h];
        float M = -INFINITY;
#pragma unroll
        for (int w = 0; w < W; ++w) M = fmaxf(M, lds.mg.m[w][h]);
        float L = 0.f;
        f32x4 o[kV4];
#pragma unroll
        for (int v = 0; v < kV4; ++v) o[v] = f32x4{0.f, 0.f, 0.f, 0.f};
        if (M != -INFINITY) {
#pragma unroll
            for (int w = 0; w < W; ++w) {
                const float mw = lds.mg.m[w][h];
                const float wt = (mw == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((mw - M) * fh);
                L += wt * lds.mg.l[w][h];
#pragma unroll
                for (int v = 0; v < kV4; ++v) o[v] += wt * *reinterpret_cast<const f32x4*>(&lds.mg.acc[w][h][c0 + 4 * v]);
            }
        }
        if (direct) {
            if (h < af.H) {
                const float inv = L > 0.f ? 1.f / L : 0.f;
#pragma unroll
                for (int v = 0; v < kV4; ++v)
                    *reinterpret_cast<f32x4*>(af.out + (row * af.H + h) * (int64_t)kD + c0 + 4 * v) = o[v] * inv;
            }
        } else {
            const __amdgpu_buffer_rsrc_t rs =
                __builtin_amdgcn_make_buffer_rsrc(part, (short)0, kPartFloats * 4, kRsrcWord3);
#pragma unroll
            for (int v = 0; v < kV4; ++v)
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o[v]), rs, (h * kD + c0 + 4 * v) * 4,
                                                       0, kCoherent);
            if (c0 == 0) {
                const f32x2 ml = {M, L};
                __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, ml), rs, (kMaxHeads * kD + 2 * h) * 4,
                                                     0, kCoherent);
            }
        }
    }
    wave_drain();
}

// After every workgroup of the row has published its partial state: the
// output rows of heads h = first, first + step, ... (< H), each the merge of
// the row's S states in slice order, normalized - in batches of MAXS slices
// whose loads are in flight together, each batch folded into the running
// state with the usual rescale (a fixed order: the result does not depend on
// scheduling). fh: the heads' scale-back factors (those of this workgroup's
// own query conversion; every workgroup converts the same query the same
// way). 32 threads per head, 4 channels each.
template <int MAXS>
__device__ __forceinline__ void fused_attn_merge(const AttnFuse& af, int64_t row, const float* parts_row, int S,
                                                 int first, int step, const float* fh) {
    const int tid = threadIdx.x;
    const int h = first + (tid >> 5) * step;
    const int c0 = (tid & 31) * 4;
    if (h >= af.H || (tid >> 5) * step >= kMaxHeads) return;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(parts_row), (short)0, S * kPartFloats * 4, kRsrcWord3);
    const float f = fh[h];
    float MM = -INFINITY, LL = 0.f;
    f32x4 oo = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int s0 = 0; s0 < S; s0 += MAXS) {
        u32x4 pa[MAXS];
        u32x2 pml[MAXS];
#pragma unroll
        for (int i = 0; i < MAXS; ++i) {        // slices past S read past the resource: zeros, no access
            const int s = s0 + i;
            pa[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (s * kPartFloats + h * kD + c0) * 4, 0, kCoherent);
            pml[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, (s * kPartFloats + kMaxHeads * kD + 2 * h) * 4, 0,
                                                          kCoherent);
        }
        float bm = -INFINITY;
#pragma unroll
        for (int i = 0; i < MAXS; ++i) bm = fmaxf(bm, s0 + i < S ? __uint_as_float(pml[i].x) : -INFINITY);
        const float Mn = fmaxf(MM, bm);
        if (Mn == -INFINITY) continue;          // nothing attended so far
        const float a = MM == -INFINITY ? 0.f : __builtin_amdgcn_exp2f((MM - Mn) * f);
        LL *= a;
        oo *= a;
#pragma unroll
        for (int i = 0; i < MAXS; ++i) {
            const float ms = __uint_as_float(pml[i].x);
            const float wt = (s0 + i >= S || ms == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f((ms - Mn) * f);
            LL += wt * __uint_as_float(pml[i].y);
            oo += wt * __builtin_bit_cast(f32x4, pa[i]);
        }
        MM = Mn;
    }
    const float inv = LL > 0.f ? 1.f / LL : 0.f;
    *reinterpret_cast<f32x4*>(af.out + (row * af.H + h) * (int64_t)kD + c0) = oo * inv;
}

}  // namespace csa2
