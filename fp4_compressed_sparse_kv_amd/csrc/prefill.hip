// Prefill indexer on gfx950 matrix cores: candidate positions for the top-K of
// many queries per sequence (a chunk of Q queries scoring all N keys), for the
// Full layer of a prefill.
//
// The exact score of a position is the dot product of the bf16 indexer query
// and the key, rounded once to fp32; the exact top-K of each query is taken
// by the select kernel over a short candidate list per query. The matrix
// cores only decide which positions are candidates:
//   1. k_pf_kmax: per sequence and channel, the largest |key| (partials).
//   2. k_pf_tiles, dense mode: approximate scores s~ of every query against a
//      sample of the keys (every 64th position); k_pf_rth (or, for longer
//      sample rows, the select kernel) then gives each query's R-th largest
//      sample score t.
//   3. k_pf_thresholds: per query, the margin e = 2^-14 * sum_i |q_i| kmax_i
//      (+ 2^-120), which exceeds four times the error of s~ plus one fp32
//      rounding (the products bf16 x bf16 are exact in fp32 and the 64 terms
//      are summed in fp32: |s~ - S| <= 68 * 2^-23 * sum |q_i k_i| for the
//      exact real dot S), the candidate threshold lo = t - e and the check
//      bound v = t - e/2.
//   4. k_pf_tiles, candidate mode: s~ of every query against every causal
//      position; positions with s~ >= lo are appended, in position order, to
//      one list per (query, key range).
//   5. The select kernel ranks each query's candidates by their exact scores.
//   6. k_pf_verify: a position that is not a candidate has s~ < lo, so its
//      exact fp32 score is below lo + e/2 = v. If the K-th largest exact
//      score among the candidates is above v, no other position can enter
//      the top-K or tie with its last member, so the result is the exact
//      top-K; so it is too when the lists hold every causal position. Queries
//      that fail both tests, whose lists overflowed, or with more candidates
//      than the select holds (its LDS is sized for the candidates a query
//      nominates, not for every list slot), are queued for the
//      exact full-scan select (all of them: the first 64 by the multi-
//      workgroup select, any further ones by k_pf_repair_rest).
// Matrix-core tiles: a workgroup of 4 waves owns 128 queries of one sequence
// and one key range; wave w owns query rows 32w..32w+31 and runs
// v_mfma_f32_32x32x16_bf16 over 128-key tiles staged in LDS as bf16 (E4M3
// keys convert exactly), one 64-key half at a time, three workgroups per CU
// (the candidate appends are the VALU-bound part; more resident waves hide
// them behind each other's matrix-core work). The K dimension is permuted (lane group g holds
// channels 32g..32g+31) so each lane reads 32 contiguous key bytes; the dot
// product does not depend on the order of its terms beyond the bound above.
#include "dot.hpp"
#include "internal.hpp"

namespace csa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kPfThreads = 256;
constexpr int kPfRows = 128;                    // query rows per workgroup
constexpr int kPfKeys = 128;                    // keys per LDS tile
constexpr int kPfDim = 64;                      // indexer dim of this path
constexpr int kPfLdsStride = 72;                // bf16 per staged key row (64 + 8: conflict-free reads)
constexpr int kKmaxBlocks = 64;                 // partial-max blocks per sequence

// ------------------------------------------------------------------ kmax

template <int KT>
__global__ void __launch_bounds__(256) k_pf_kmax(const uint8_t* __restrict__ k, int64_t N, float* __restrict__ partial) {
    // thread t reads 16 channels (16 * elem bytes) of keys t/4, t/4 + 64, ...
    constexpr int EB = ElemBytes<KT>::v;
    __shared__ float red[256][16];
    const int seq = blockIdx.y, blk = blockIdx.x, t = threadIdx.x;
    const int cg = t & 3;
    const int64_t per = (N + kKmaxBlocks - 1) / kKmaxBlocks;
    const int64_t t0 = blk * per, t1 = min(N, t0 + per);
    float m[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) m[i] = 0.f;
    const uint8_t* base = k + (size_t)seq * N * kPfDim * EB;
    // four rows per step (r, r + 64, r + 128, r + 192; past the range the last
    // row again, which leaves a maximum unchanged), their loads in flight together
    static_assert(EB == 1 || EB == 2, "E4M3 or bf16 keys");
    constexpr int W = EB;                       // 16-byte words per thread and row
    for (int64_t r = t0 + (t >> 2); r < t1; r += 256) {
        uint4 w[4][W];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int64_t rr = min(r + 64 * u, t1 - 1);
            const uint8_t* p = base + (size_t)rr * kPfDim * EB + cg * 16 * EB;
#pragma unroll
            for (int v = 0; v < W; ++v) w[u][v] = *reinterpret_cast<const uint4*>(p + 16 * v);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            if constexpr (KT == kE4M3) {
                const uint32_t ws[4] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const f32x2 a = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[j], false);
                    const f32x2 b = __builtin_amdgcn_cvt_pk_f32_fp8((int)ws[j], true);
                    m[4 * j + 0] = fmaxf(m[4 * j + 0], fabsf(a.x));
                    m[4 * j + 1] = fmaxf(m[4 * j + 1], fabsf(a.y));
                    m[4 * j + 2] = fmaxf(m[4 * j + 2], fabsf(b.x));
                    m[4 * j + 3] = fmaxf(m[4 * j + 3], fabsf(b.y));
                }
            } else {
                const uint32_t ws[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w,
                                        w[u][W - 1].x, w[u][W - 1].y, w[u][W - 1].z, w[u][W - 1].w};
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    m[2 * j + 0] = fmaxf(m[2 * j + 0], fabsf(__uint_as_float(ws[j] << 16)));
                    m[2 * j + 1] = fmaxf(m[2 * j + 1], fabsf(__uint_as_float(ws[j] & 0xFFFF0000u)));
                }
            }
        }
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) red[t][i] = m[i];
    __syncthreads();
    if (t < kPfDim) {
        const int g = t / 16, i = t % 16;
        float r = 0.f;
        for (int u = g; u < 256; u += 4) r = fmaxf(r, red[u][i]);
        partial[((size_t)seq * kKmaxBlocks + blk) * kPfDim + t] = r;
    }
}

// ----------------------------------------------------------------- tiles

struct PfTileArgs {
    const uint16_t* q;                          // [rows][64] bf16 indexer queries
    const uint8_t* k;                           // [seqs][N][64] keys
    int64_t N;
    int32_t Q;                                  // queries per sequence (row = seq * Q + i)
    const int64_t* q_pos;                       // [rows] causal limit
    int64_t key_off, key_stride, nkeys;         // key j of the set is position key_off + j * key_stride
    int32_t nranges;
    int64_t range_len;                          // dense mode: keys per range (a multiple of kPfKeys)
    float* dense;                               // dense mode: [rows][nkeys] scores (s~, -inf past q_pos)
    const float* thr;                           // candidate mode: [rows][2] (lo, v)
    int32_t* cand;                              // [rows][nranges][cap] positions
    int32_t cap;
    uint32_t* cnt;                              // [rows][nranges] candidates found (may exceed cap)
};

// Raw bytes of one thread's share of a 128-key tile: half (t & 1) of key t / 2.
template <int KT>
struct TileRaw {
    static constexpr int W = 2 * ElemBytes<KT>::v;   // 16-byte words (32 channels)
    uint4 w[W];
};

template <int KT, bool DENSE>
__global__ void __launch_bounds__(kPfThreads, 3) k_pf_tiles(PfTileArgs a) {
    constexpr int EB = ElemBytes<KT>::v;
    __shared__ __attribute__((aligned(16))) uint16_t tile[2][kPfKeys * kPfLdsStride];
    __shared__ int32_t s_qp[kPfThreads / kWave][32];     // causal limit of each query row of a wave
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int g = lane >> 5, ln = lane & 31;
    const int qtiles = (a.Q + kPfRows - 1) / kPfRows;
    const int seq = blockIdx.x / qtiles, qt = blockIdx.x - seq * qtiles;
    const int range = blockIdx.y;
    const int q0 = qt * kPfRows + wave * 32;    // this wave's first query (within the sequence)
    const int64_t rbase = (int64_t)seq * a.Q;

    // A operand: query q0 + ln, channels 32g + 8s .. 32g + 8s + 7 for k-step s
    bf16x8 qa[4];
    {
        const int qi = min(q0 + ln, a.Q - 1);
        const uint4* p = reinterpret_cast<const uint4*>(a.q + (rbase + qi) * kPfDim + 32 * g);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            uint4 w = p[s];
            if (q0 + ln >= a.Q) w = make_uint4(0, 0, 0, 0);
            qa[s] = __builtin_bit_cast(bf16x8, w);
        }
    }
    // accumulator element i of this lane is query row rr(i) = 8*(i/4) + 4g + i%4 of the wave
    float tlo[16];
    uint32_t curv[16];                          // list length of this lane's row rr(i) (uniform per lane group)
    int32_t qmin = INT32_MAX, qmax = -1;        // over this wave's valid rows
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int qi = q0 + 8 * (i / 4) + 4 * g + (i % 4);
        const bool ok = qi < a.Q;
        const int64_t r = rbase + (ok ? qi : 0);
        const int64_t pq = a.q_pos ? a.q_pos[r] : INT64_MAX;
        const int32_t qpi = ok ? (int32_t)(pq < 0 ? -1 : (pq >= a.N ? a.N - 1 : pq)) : -1;
        if (ok) {
            qmin = min(qmin, qpi);
            qmax = max(qmax, qpi);
        }
        if (ln == 0) s_qp[wave][8 * (i / 4) + 4 * g + (i % 4)] = qpi;
        if constexpr (!DENSE) tlo[i] = ok ? a.thr[2 * r + 0] : INFINITY;
        curv[i] = 0u;
    }
    for (int o = 32; o >= 1; o >>= 1) {
        qmin = min(qmin, __shfl_xor(qmin, o));
        qmax = max(qmax, __shfl_xor(qmax, o));
    }

    const uint8_t* kbase = a.k + (size_t)seq * a.N * kPfDim * EB;
    // candidate list of row rr(i): clist + (8*(i/4) + i%4) * row_step (32-bit offsets: the
    // launcher keeps 32 * nranges * cap below 2^31)
    const uint32_t row_step = (uint32_t)a.nranges * (uint32_t)a.cap;
    int32_t* const clist = a.cand + ((size_t)(rbase + q0 + 4 * g) * a.nranges + range) * a.cap;
    // Candidate mode: the ranges split the causal span of this workgroup's 128
    // queries, [0, largest q_pos], not the whole context, so every query's
    // candidates spread over all of its lists wherever the chunk sits.
    int64_t range_len = a.range_len;
    if constexpr (!DENSE) {
        int32_t tmax = -1;
        for (int u = lane; u < kPfRows; u += kWave) {
            const int qi = qt * kPfRows + u;
            if (qi < a.Q) {
                const int64_t pq = a.q_pos ? a.q_pos[rbase + qi] : a.N - 1;
                tmax = max(tmax, (int32_t)(pq < 0 ? -1 : (pq >= a.N ? a.N - 1 : pq)));
            }
        }
        for (int o = 32; o >= 1; o >>= 1) tmax = max(tmax, __shfl_xor(tmax, o));
        const int64_t span = min(a.nkeys, (int64_t)tmax + 1);
        range_len = (span + a.nranges - 1) / a.nranges;
        range_len = (range_len + kPfKeys - 1) / kPfKeys * kPfKeys;
    }
    const int64_t j0 = (int64_t)range * range_len;
    const int64_t j1 = min(a.nkeys, j0 + range_len);
    const int64_t ntile = j1 > j0 ? (j1 - j0 + kPfKeys - 1) / kPfKeys : 0;

    // Loads are unconditional (a tile past the range reloads the last one) so
    // the compiler's wait counts stay exact across the two register sets.
    auto load_raw = [&](int64_t t, TileRaw<KT>& r) {
        const int64_t tt = t < ntile ? t : ntile - 1;
        const int64_t j = j0 + tt * kPfKeys + (tid >> 1);
        const int64_t pos = j < j1 ? a.key_off + j * a.key_stride : 0;
        const uint8_t* src = kbase + (size_t)pos * kPfDim * EB + (tid & 1) * 32 * EB;
#pragma unroll
        for (int u = 0; u < TileRaw<KT>::W; ++u) r.w[u] = *reinterpret_cast<const uint4*>(src + 16 * u);
    };
    auto stage = [&](const TileRaw<KT>& r, uint16_t* buf) {
        uint4* dst = reinterpret_cast<uint4*>(&buf[(tid >> 1) * kPfLdsStride + (tid & 1) * 32]);
        if constexpr (KT == kE4M3) {
            const uint32_t ws[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w, r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
            uint32_t o[16];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                // E4M3 values are exact in bf16; the scale 1.0 leaves them as they are
                o[2 * u + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[u], 1.0f, false));
                o[2 * u + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(ws[u], 1.0f, true));
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) dst[u] = make_uint4(o[4 * u], o[4 * u + 1], o[4 * u + 2], o[4 * u + 3]);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) dst[u] = r.w[u];
        }
    };
    auto compute = [&](const uint16_t* buf, int64_t t) {
        const int64_t jt = j0 + t * kPfKeys;
        const int64_t p_first = a.key_off + jt * a.key_stride;
        const int64_t p_last = a.key_off + min(jt + kPfKeys - 1, j1 - 1) * a.key_stride;
        if (!DENSE && p_first > (int64_t)qmax) return;           // no causal key for any row of the wave
        const bool masked = p_last > (int64_t)qmin;              // some key is past some row's limit
        const bool full = jt + kPfKeys <= j1;                    // every key of the tile is in the range
        // the tile in two halves of 64 keys: the two 32-key blocks' MFMA chains
        // interleaved (independent accumulators), then their candidates - half
        // the accumulators live at a time, so three workgroups fit on a CU
        constexpr int NC = 2;                   // 32-key blocks per half tile
#pragma unroll
        for (int hh = 0; hh < kPfKeys / 64; ++hh) {
            f32x16 accs[NC];
#pragma unroll
            for (int c = 0; c < NC; ++c) accs[c] = f32x16{};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                bf16x8 bop[NC];
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    bop[c] = __builtin_bit_cast(
                        bf16x8, *reinterpret_cast<const uint4*>(&buf[(64 * hh + 32 * c + ln) * kPfLdsStride + 32 * g + 8 * s]));
#pragma unroll
                for (int c = 0; c < NC; ++c) accs[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa[s], bop[c], accs[c], 0, 0, 0);
            }
#pragma unroll
            for (int c = 0; c < NC; ++c) {
                const f32x16 acc = accs[c];
                const int64_t jk = jt + 64 * hh + 32 * c + ln;
                const bool kvalid = jk < j1;
                const int32_t pos = (int32_t)(a.key_off + jk * a.key_stride);
                if constexpr (DENSE) {
                    if (kvalid) {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const int qi = q0 + 8 * (i / 4) + 4 * g + (i % 4);
                            if (qi < a.Q)
                                a.dense[(size_t)(rbase + qi) * a.nkeys + jk] =
                                    pos <= s_qp[wave][8 * (i / 4) + 4 * g + (i % 4)] ? acc[i] : -INFINITY;
                        }
                    }
                } else {
                    // lanes 0..31 hold row rr(i) of lane group 0, lanes 32..63 that of group 1;
                    // each half appends its passing keys in lane (= position) order
                    auto emit = [&](int i, uint64_t m, bool pass) {
                        const uint32_t mlo = (uint32_t)m, mhi = (uint32_t)(m >> 32);
                        // the list length plus the passing lanes below this one in its half
                        const uint32_t slot = __builtin_amdgcn_mbcnt_hi(mhi, __builtin_amdgcn_mbcnt_lo(g ? 0u : mlo, curv[i]));
                        if (pass && slot < (uint32_t)a.cap)
                            clist[(8 * (i / 4) + (i % 4)) * row_step + slot] = pos;
                        curv[i] += (uint32_t)__popc(g ? mhi : mlo);
                    };
                    if (full && !masked) {          // every key valid and causal for every row: one compare each
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const bool pass = acc[i] >= tlo[i];
                            const uint64_t m = __ballot(pass);
                            if (__builtin_expect(m != 0ull, 0)) emit(i, m, pass);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < 16; ++i) {
                            const bool pass = (int)kvalid & (int)(pos <= s_qp[wave][8 * (i / 4) + 4 * g + (i % 4)]) &
                                              (int)(acc[i] >= tlo[i]);
                            const uint64_t m = __ballot(pass);
                            if (__builtin_expect(m != 0ull, 0)) emit(i, m, pass);
                        }
                    }
                }
            }
        }
    };

    // Pipeline: tile t is computed from LDS buffer t & 1 while the raw bytes
    // of tile t + 2 load into one register set and those of tile t + 1 (loaded
    // one tile earlier, in the other set) are converted into the other buffer.
    if (ntile > 0) {
        TileRaw<KT> r0, r1;
        load_raw(0, r0);
        load_raw(1, r1);
        stage(r0, tile[0]);
        __syncthreads();
        for (int64_t t = 0; t < ntile; t += 2) {
            load_raw(t + 2, r0);
            compute(tile[0], t);
            if (t + 1 < ntile) stage(r1, tile[1]);
            __syncthreads();
            if (t + 1 >= ntile) break;
            load_raw(t + 3, r1);
            compute(tile[1], t + 1);
            if (t + 2 < ntile) stage(r0, tile[0]);
            __syncthreads();
        }
    }
    if constexpr (!DENSE) {
        if (ln == 0) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int qi = q0 + 8 * (i / 4) + 4 * g + (i % 4);
                if (qi < a.Q) a.cnt[(size_t)(rbase + qi) * a.nranges + range] = curv[i];
            }
        }
    }
}

// ------------------------------------------------------- sample threshold

// The R-th largest of each row's n sample scores, exactly (-inf when fewer
// than R are finite): the row's order-preserving keys stay in registers (256
// threads, up to kRthPer keys each) and three radix passes over 11, 11 and 10
// key bits narrow the bin that holds the R-th key, counting from the top.
// With R <= 256 the first pass counts only the keys at or above a floor: the
// lower edge of the 11-bit bin that holds the R-th largest of the threads'
// maxima. Those maxima are R distinct keys at or above the floor, so the R-th
// largest key of the row is too, and every key below the floor ranks after
// it; the floor leaves out most of the row, whose keys would otherwise crowd
// a few histogram bins with conflicting atomic adds.
constexpr int kRthThreads = 256;
constexpr int kRthPer = 64;                     // rows of up to 16384 samples

// Over nb = 2^w bins h[0..nb) scanned from the top: the bin holding the
// need-th key and how many of its keys are still needed (res[0], res[1]);
// returns the total count. Every thread calls it; it ends with a barrier.
__device__ __forceinline__ uint32_t rth_find(const uint32_t* hist, int nb, uint32_t need, uint32_t* wsum,
                                             uint32_t* res) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    // thread t owns bins top - per + 1 .. top (top = nb - 1 - per * t), scanned from the top
    const int per = nb / kRthThreads;
    const int top = nb - 1 - tid * per;
    uint32_t sum = 0;
    for (int i = 0; i < per; ++i) sum += hist[top - i];
    const uint32_t inc = wave_incl_scan(sum);
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = inc - sum, total = 0;
#pragma unroll
    for (int v = 0; v < kRthThreads / kWave; ++v) {
        total += wsum[v];
        if (v < wave) before += wsum[v];
    }
    if (before < need && need <= before + sum) {
        uint32_t c = before;
        for (int i = 0; i < per; ++i) {
            const uint32_t h = hist[top - i];
            if (c + h >= need) {
                res[0] = (uint32_t)(top - i);
                res[1] = need - c;
                break;
            }
            c += h;
        }
    }
    __syncthreads();
    return total;
}

__global__ void __launch_bounds__(kRthThreads)
k_pf_rth(const float* __restrict__ dense, int32_t n, int32_t R, float* __restrict__ tval) {
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t wsum[kRthThreads / kWave];
    __shared__ uint32_t res[2];
    const int tid = threadIdx.x;
    const float* p = dense + (size_t)blockIdx.x * n;
    uint32_t kv[kRthPer];                       // the order of a row's keys does not matter here
    if ((n & 3) == 0) {                         // 16-byte rows: thread t holds entries 4(256j + t) .. + 3
#pragma unroll
        for (int j = 0; j < kRthPer / 4; ++j) {
            const int i = 4 * (j * kRthThreads + tid);
            const float4 v = i < n ? *reinterpret_cast<const float4*>(p + i) : make_float4(NAN, NAN, NAN, NAN);
            kv[4 * j + 0] = score_key(v.x);
            kv[4 * j + 1] = score_key(v.y);
            kv[4 * j + 2] = score_key(v.z);
            kv[4 * j + 3] = score_key(v.w);
        }
    } else {
#pragma unroll
        for (int j = 0; j < kRthPer; ++j) {
            const int i = j * kRthThreads + tid;
            kv[j] = i < n ? score_key(p[i]) : 0u;
        }
    }
    uint32_t floor_key = 1u;                    // key 0 (NaN, -inf, padding) never counts
    if (R <= kRthThreads) {
        uint32_t mx = 0u;
#pragma unroll
        for (int j = 0; j < kRthPer; ++j) mx = max(mx, kv[j]);
        for (int b = tid; b < 2048; b += kRthThreads) hist[b] = 0u;
        __syncthreads();
        if (mx != 0u) atomicAdd(&hist[mx >> 21], 1u);
        __syncthreads();
        const uint32_t tot = rth_find(hist, 2048, (uint32_t)R, wsum, res);
        // fewer than R nonzero maxima: no floor beyond the nonzero keys
        if (tot >= (uint32_t)R && res[0] != 0u) floor_key = res[0] << 21;
        __syncthreads();                        // res is rewritten by the first pass
    }
    uint32_t prefix = 0, need = (uint32_t)R;
#pragma unroll
    for (int d = 0; d < 3; ++d) {
        const int lo = d == 0 ? 21 : (d == 1 ? 10 : 0);
        const int w = d == 2 ? 10 : 11;
        const int nb = 1 << w;
        for (int b = tid; b < nb; b += kRthThreads) hist[b] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < kRthPer; ++j) {
            const uint32_t k = kv[j];
            if (d == 0 ? k >= floor_key : (k != 0u && (k >> (lo + w)) == prefix))
                atomicAdd(&hist[(k >> lo) & (uint32_t)(nb - 1)], 1u);
        }
        __syncthreads();
        const uint32_t total = rth_find(hist, nb, need, wsum, res);
        if (d == 0 && total < need) {           // the same for every thread
            if (tid == 0) tval[blockIdx.x] = -INFINITY;
            return;
        }
        prefix = (prefix << w) | res[0];
        need = res[1];
        __syncthreads();                        // hist, wsum and res are rewritten by the next pass
    }
    if (tid == 0) tval[blockIdx.x] = key_score(prefix);
}

// ------------------------------------------------------------ thresholds

// One thread per query row: t = R-th largest sample score (the minimum of the
// select's R outputs; -inf if fewer than R samples are causal), the margin
// from the query and the per-channel key maxima, lo and v. The key maxima of
// the (at most two) sequences a workgroup's rows belong to are reduced from
// the partials once per workgroup, in LDS; with fewer than 256 queries per
// sequence each thread reduces its own.
constexpr int kThrThreads = 256;

__global__ void __launch_bounds__(kThrThreads)
k_pf_thresholds(const uint16_t* __restrict__ q, int64_t rows, int32_t Q, const float* __restrict__ sel, int32_t R,
                const float* __restrict__ kmax_partial, float* __restrict__ thr, uint32_t* __restrict__ repair_count) {
    __shared__ float part[kThrThreads / kPfDim][kPfDim];
    __shared__ float skm[2][kPfDim];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.x * kThrThreads;
    const int64_t r = r0 + tid;
    if (r == 0) *repair_count = 0u;
    const int64_t seq0 = r0 / Q;
    const int64_t nseq = r0 < rows ? (min(rows, r0 + kThrThreads) - 1) / Q - seq0 + 1 : 0;
    const bool shared_km = nseq >= 1 && nseq <= 2;      // the same in every thread
    if (shared_km) {
        const int c = tid % kPfDim, gq = tid / kPfDim;
        for (int sq = 0; sq < nseq; ++sq) {
            const float* kp = kmax_partial + (size_t)(seq0 + sq) * kKmaxBlocks * kPfDim;
            float m = 0.f;
            for (int b = gq; b < kKmaxBlocks; b += kThrThreads / kPfDim) m = fmaxf(m, kp[b * kPfDim + c]);
            part[gq][c] = m;
            __syncthreads();
            if (tid < kPfDim) {
                float km = 0.f;
#pragma unroll
                for (int u = 0; u < kThrThreads / kPfDim; ++u) km = fmaxf(km, part[u][tid]);
                skm[sq][tid] = km;
            }
            __syncthreads();
        }
    }
    if (r >= rows) return;
    const int64_t seq = r / Q;
    float t = INFINITY;
    int n = 0;
    for (int j = 0; j < R; ++j) {
        const float v = sel[r * R + j];
        if (v == v) {                           // the select pads with NaN
            t = fminf(t, v);
            ++n;
        }
    }
    if (n < R) t = -INFINITY;
    const float* kp = kmax_partial + (size_t)seq * kKmaxBlocks * kPfDim;
    const uint4* qr = reinterpret_cast<const uint4*>(q + r * kPfDim);
    double s = 0.0;
#pragma unroll
    for (int v = 0; v < kPfDim / 8; ++v) {
        const uint4 w = qr[v];
        const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
        for (int h = 0; h < 8; ++h) {
            const int i = 8 * v + h;
            float km;
            if (shared_km) {
                km = skm[seq - seq0][i];
            } else {
                km = 0.f;
                for (int b = 0; b < kKmaxBlocks; ++b) km = fmaxf(km, kp[b * kPfDim + i]);
            }
            const uint32_t bits = (h & 1) ? (ws[h >> 1] >> 16) : (ws[h >> 1] & 0xFFFFu);
            s += fabs((double)bf16_bits_to_f32(bits)) * (double)km;
        }
    }
    const double e = s * 0x1p-14 + 0x1p-120;
    thr[2 * r + 0] = t == -INFINITY ? -INFINITY : (float)((double)t - e);
    thr[2 * r + 1] = t == -INFINITY ? -INFINITY : (float)((double)t - 0.5 * e);
}

// ----------------------------------------------------------------- verify

// See step 6 above; sel holds the exact scores the select returned ([rows][K],
// NaN past the selected ones). One wave per query row.
__global__ void __launch_bounds__(256)
k_pf_verify(int64_t rows, int32_t nranges, int32_t cap, int64_t dense_cap, const uint32_t* __restrict__ cnt,
            const float* __restrict__ sel,
            const float* __restrict__ thr, const int64_t* __restrict__ q_pos, int64_t N, int32_t K,
            int32_t* __restrict__ repair_rows, uint32_t* __restrict__ repair_count, int32_t repair_cap,
            uint32_t* __restrict__ status) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (r >= rows) return;
    float sk = INFINITY;
    uint32_t n = 0;
    for (int j = lane; j < K; j += 64) {
        const float v = sel[r * K + j];
        if (v == v) {
            sk = fminf(sk, v);
            ++n;
        }
    }
    for (int o = 32; o >= 1; o >>= 1) {
        sk = fminf(sk, __shfl_xor(sk, o));
        n += __shfl_xor(n, o);
    }
    if (lane != 0) return;
    const int64_t pq = q_pos ? q_pos[r] : N - 1;
    const int64_t valid = pq < 0 ? 0 : (pq >= N ? N : pq + 1);
    int64_t total = 0;
    bool overflow = false;
    for (int j = 0; j < nranges; ++j) {
        const uint32_t c = cnt[r * nranges + j];
        total += c;
        overflow = overflow || c > (uint32_t)cap;
    }
    overflow = overflow || total > dense_cap;  // more candidates than the exact select holds: it left the row alone
    const bool ok = !overflow && (total == valid || (n == (uint32_t)K && sk > thr[2 * r + 1]));
    if (!ok) {
        const uint32_t slot = atomicAdd(repair_count, 1u);
        if (slot < (uint32_t)repair_cap) repair_rows[slot] = (int32_t)r;   // the queue holds every row
    }
}

// Repair map for one launch of the exact select: slots [first, first + n) of
// the repair list, -1 where the list is shorter.
__global__ void k_pf_repair_map(const int32_t* __restrict__ repair_rows, const uint32_t* __restrict__ repair_count,
                                int32_t first, int32_t n, int32_t* __restrict__ map) {
    const int i = threadIdx.x;
    if (i < n) map[i] = (uint32_t)(first + i) < *repair_count ? repair_rows[first + i] : -1;
}

// ------------------------------------------------- exact repair, any count

// Queued queries past the fast repair pass (queue slots first .. count-1):
// one workgroup per query, grid-stride over the queue, so every queued query
// gets its exact top-K whatever the count (a count within the fast pass makes
// this kernel return at once). A query's exact scores over its causal range
// [0, q_pos] are recomputed in each of four passes instead of being stored:
// three radix passes (11, 11, 10 key bits) narrow the threshold key T and the
// number of keys equal to T to take, and the last pass writes the selected
// positions in ascending order (keys above T, then the lowest-positioned
// keys equal to T), then -1 padding. Only degenerate inputs (mass ties at a
// query's threshold) queue more queries than the fast pass holds.
constexpr int kRepThreads = 512;
constexpr int kRepQuads = kRepThreads / 4;
constexpr int kRepU = 8;                        // keys per quad in flight
constexpr int kRepTile = kRepQuads * kRepU;     // keys per iteration

// Bin holding the need-th largest key of a 2048-bin histogram (counted from
// the top): returns the bin; `above` = keys in higher bins. need >= 1 and
// the histogram holds at least need keys.
__device__ uint32_t rep_find(const uint32_t* hist, int nb, uint32_t need, uint32_t& above, uint32_t* sm) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    constexpr int kPer = 2048 / kRepThreads;
    // thread t owns bins nb-1-kPer*t .. nb-kPer*(t+1) (top down); nb <= 2048
    uint32_t c[kPer], tot = 0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = nb - 1 - kPer * tid - i;
        c[i] = b >= 0 ? hist[b] : 0u;
        tot += c[i];
    }
    const uint32_t inc = wave_incl_scan(tot);
    if (lane == 63) sm[wave] = inc;
    __syncthreads();
    uint32_t before = inc - tot;
    for (int w = 0; w < wave; ++w) before += sm[w];
    uint32_t run = before;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int b = nb - 1 - kPer * tid - i;
        if (b >= 0 && run < need && run + c[i] >= need) {
            sm[16] = (uint32_t)b;
            sm[17] = run;
        }
        run += c[i];
    }
    __syncthreads();
    const uint32_t bin = sm[16];
    above = sm[17];
    __syncthreads();
    return bin;
}

template <int KT>
__global__ void __launch_bounds__(kRepThreads)
k_pf_repair_rest(const uint16_t* __restrict__ q, const uint8_t* __restrict__ k, int64_t N, int32_t Q,
                 const int64_t* __restrict__ q_pos, const int32_t* __restrict__ repair_rows,
                 const uint32_t* __restrict__ repair_count, int32_t first, int32_t K, int32_t* __restrict__ idx_out) {
    using KS = KeySlice<KT, kPfDim, kBF16>;
    __shared__ uint32_t hist[2048];
    __shared__ uint32_t sm[32];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int quad = tid >> 2, lq = tid & 3;
    const uint32_t count = *repair_count;
    for (uint32_t slot = (uint32_t)first + blockIdx.x; slot < count; slot += gridDim.x) {
        const int64_t row = repair_rows[slot];
        const int64_t seq = row / Q;
        const int64_t pq = q_pos ? q_pos[row] : N - 1;
        const int64_t L = pq < 0 ? 0 : (pq >= N ? N : pq + 1);
        double qd[kPfDim / 4];
        load_query_slice<kBF16, kPfDim>(q + row * kPfDim, lq, qd);
        const uint8_t* kb = k + (size_t)seq * N * KS::ROW_BYTES;
        // keys[u] of this quad: position base + u * kRepQuads + quad (0 = padding / not selectable)
        auto scan = [&](auto&& visit) {
            for (int64_t base = 0; base < L; base += kRepTile) {
                KS sl[kRepU];
#pragma unroll
                for (int u = 0; u < kRepU; ++u) {
                    const int64_t t = base + u * kRepQuads + quad;
                    if (t < L) sl[u].load(kb + t * KS::ROW_BYTES, lq);
                    else for (int j = 0; j < KS::RAW; ++j) sl[u].raw[j] = make_uint4(0, 0, 0, 0);
                }
#pragma unroll
                for (int u = 0; u < kRepU; ++u) {
                    const int64_t t = base + u * kRepQuads + quad;
                    const auto v = quad_sum(sl[u].dot(qd));
                    visit(t, t < L ? score_key(round_score(v)) : 0u, u);
                }
            }
        };
        // ---- pass 1: top 11 bits, and the number of selectable keys
        for (int i = tid; i < 2048; i += kRepThreads) hist[i] = 0u;
        if (tid == 0) sm[18] = 0u;
        __syncthreads();
        uint32_t nvalid = 0;
        scan([&](int64_t, uint32_t key, int) {
            if (lq == 0 && key) {
                atomicAdd(&hist[key >> 21], 1u);
                ++nvalid;
            }
        });
        atomicAdd(&sm[18], nvalid);
        __syncthreads();
        const uint32_t need = min((uint32_t)K, sm[18]);
        uint32_t T = 0xFFFFFFFFu, take_eq = 0;
        if (need > 0) {
            uint32_t above = 0, rem = need;
            const uint32_t b1 = rep_find(hist, 2048, rem, above, sm);
            rem -= above;
            // ---- pass 2: bits 10..20 of the keys in bin b1
            for (int i = tid; i < 2048; i += kRepThreads) hist[i] = 0u;
            __syncthreads();
            scan([&](int64_t, uint32_t key, int) {
                if (lq == 0 && key && (key >> 21) == b1) atomicAdd(&hist[(key >> 10) & 0x7FFu], 1u);
            });
            __syncthreads();
            const uint32_t b2 = rep_find(hist, 2048, rem, above, sm);
            rem -= above;
            const uint32_t pre = (b1 << 11) | b2;
            // ---- pass 3: bits 0..9 of the keys with that 22-bit prefix
            for (int i = tid; i < 2048; i += kRepThreads) hist[i] = 0u;
            __syncthreads();
            scan([&](int64_t, uint32_t key, int) {
                if (lq == 0 && key && (key >> 10) == pre) atomicAdd(&hist[key & 0x3FFu], 1u);
            });
            __syncthreads();
            const uint32_t b3 = rep_find(hist, 1024, rem, above, sm);
            rem -= above;
            T = (pre << 10) | b3;
            take_eq = rem;                      // keys equal to T to take, lowest positions first
        }
        // ---- pass 4: selected positions in ascending order
        int32_t* orow = idx_out + row * (int64_t)K;
        uint32_t run_sel = 0, run_eq = 0;       // over the positions already visited (uniform)
        if (need > 0) {
            scan([&](int64_t t, uint32_t key, int) {
                // positions of this step are base + u*kRepQuads + quad: ascending in (quad) for fixed u
                const bool is_eq = lq == 0 && key == T;
                const uint64_t me = __ballot(is_eq);
                if (lane == 63) sm[wave] = (uint32_t)__popcll(me);
                __syncthreads();
                uint32_t eq_before = run_eq, eq_tot = 0;
                for (int w = 0; w < kRepThreads / 64; ++w) {
                    if (w < wave) eq_before += sm[w];
                    eq_tot += sm[w];
                }
                eq_before += lanes_below(me);
                // eq_before: this key's rank among the keys equal to T, in position order
                const bool sel = lq == 0 && key != 0u && (key > T || (is_eq && eq_before < take_eq));
                __syncthreads();
                const uint64_t ms = __ballot(sel);
                if (lane == 63) sm[wave] = (uint32_t)__popcll(ms);
                __syncthreads();
                uint32_t sel_before = run_sel, sel_tot = 0;
                for (int w = 0; w < kRepThreads / 64; ++w) {
                    if (w < wave) sel_before += sm[w];
                    sel_tot += sm[w];
                }
                sel_before += lanes_below(ms);
                if (sel && sel_before < (uint32_t)K) orow[sel_before] = (int32_t)t;
                run_sel += sel_tot;
                run_eq += eq_tot;
                __syncthreads();
            });
        }
        for (int i = (int)need + tid; i < K; i += kRepThreads) orow[i] = -1;
        __syncthreads();
    }
}

// ------------------------------------------------------------------- host

size_t pf_kmax_floats(int32_t B) { return (size_t)B * kKmaxBlocks * kPfDim; }

int launch_pf_kmax(const uint8_t* k, int k_dtype, int32_t B, int64_t N, float* partial, hipStream_t stream) {
    const dim3 grid(kKmaxBlocks, (unsigned)B);
    if (k_dtype == kE4M3) hipLaunchKernelGGL(k_pf_kmax<kE4M3>, grid, dim3(256), 0, stream, k, N, partial);
    else hipLaunchKernelGGL(k_pf_kmax<kBF16>, grid, dim3(256), 0, stream, k, N, partial);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_kmax");
}

int launch_pf_tiles(const PfTiles& t, int k_dtype, bool dense, hipStream_t stream) {
    PfTileArgs a;
    a.q = t.q;
    a.k = t.k;
    a.N = t.N;
    a.Q = t.Q;
    a.q_pos = t.q_pos;
    a.key_off = t.key_off;
    a.key_stride = t.key_stride;
    a.nkeys = t.nkeys;
    a.nranges = t.nranges;
    a.range_len = (t.nkeys + t.nranges - 1) / t.nranges;
    a.range_len = (a.range_len + kPfKeys - 1) / kPfKeys * kPfKeys;
    a.dense = t.dense;
    a.thr = t.thr;
    a.cand = t.cand;
    a.cap = t.cap;
    a.cnt = t.cnt;
    // the kernel addresses a row's lists with 32-bit offsets of up to 32 * nranges * cap
    if (!dense && (int64_t)32 * t.nranges * t.cap >= ((int64_t)1 << 31))
        return fail(INVALID, "prefill candidate lists: nranges * cap too large");
    const int qtiles = (t.Q + kPfRows - 1) / kPfRows;
    const dim3 grid((unsigned)((int64_t)t.B * qtiles), (unsigned)t.nranges);
    if (k_dtype == kE4M3) {
        if (dense) hipLaunchKernelGGL((k_pf_tiles<kE4M3, true>), grid, dim3(kPfThreads), 0, stream, a);
        else hipLaunchKernelGGL((k_pf_tiles<kE4M3, false>), grid, dim3(kPfThreads), 0, stream, a);
    } else {
        if (dense) hipLaunchKernelGGL((k_pf_tiles<kBF16, true>), grid, dim3(kPfThreads), 0, stream, a);
        else hipLaunchKernelGGL((k_pf_tiles<kBF16, false>), grid, dim3(kPfThreads), 0, stream, a);
    }
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_tiles");
}

int launch_pf_rth(const float* dense, int64_t rows, int32_t n, int32_t R, float* tval, hipStream_t stream) {
    if (rows == 0) return OK;
    if (n > kRthThreads * kRthPer || R < 1) return fail(INVALID, "prefill: sample row too long for the threshold kernel");
    hipLaunchKernelGGL(k_pf_rth, dim3((unsigned)rows), dim3(kRthThreads), 0, stream, dense, n, R, tval);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_rth");
}

int launch_pf_thresholds(const uint16_t* q, int64_t rows, int32_t Q, const float* sel, int32_t R,
                         const float* kmax_partial, float* thr, uint32_t* repair_count, hipStream_t stream) {
    const unsigned blocks = (unsigned)((rows + 255) / 256);
    hipLaunchKernelGGL(k_pf_thresholds, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, q, rows, Q, sel, R,
                       kmax_partial, thr, repair_count);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_thresholds");
}

int launch_pf_verify(int64_t rows, int32_t nranges, int32_t cap, int64_t dense_cap, const uint32_t* cnt, const float* sel,
                     const float* thr, const int64_t* q_pos, int64_t N, int32_t K, int32_t* repair_rows,
                     uint32_t* repair_count, int32_t repair_cap, uint32_t* status, hipStream_t stream) {
    const unsigned blocks = (unsigned)((rows + 3) / 4);
    hipLaunchKernelGGL(k_pf_verify, dim3(blocks > 0 ? blocks : 1), dim3(256), 0, stream, rows, nranges, cap, dense_cap, cnt, sel,
                       thr, q_pos, N, K, repair_rows, repair_count, repair_cap, status);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_verify");
}

int launch_pf_repair_rest(const uint16_t* q, const uint8_t* k, int k_dtype, int64_t N, int32_t Q,
                          const int64_t* q_pos, const int32_t* repair_rows, const uint32_t* repair_count, int32_t first,
                          int32_t K, int32_t* idx_out, hipStream_t stream) {
    DeviceInfo di;
    if (int e = device_info(&di)) return e;
    const dim3 grid((unsigned)(di.num_cus > 0 ? di.num_cus : 1));
    if (k_dtype == kE4M3)
        hipLaunchKernelGGL(k_pf_repair_rest<kE4M3>, grid, dim3(kRepThreads), 0, stream, q, k, N, Q, q_pos, repair_rows,
                           repair_count, first, K, idx_out);
    else
        hipLaunchKernelGGL(k_pf_repair_rest<kBF16>, grid, dim3(kRepThreads), 0, stream, q, k, N, Q, q_pos, repair_rows,
                           repair_count, first, K, idx_out);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_repair_rest");
}

int launch_pf_repair_map(const int32_t* repair_rows, const uint32_t* repair_count, int32_t first, int32_t n,
                         int32_t* map, hipStream_t stream) {
    hipLaunchKernelGGL(k_pf_repair_map, dim3(1), dim3(256), 0, stream, repair_rows, repair_count, first, n, map);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_pf_repair_map");
}

}  // namespace csa2
