// Top-K / top-P selection on gfx950: a multi-workgroup radix select with the
// scores resident in LDS.
//
// Each row (one query's score list) is cut into S chunks; one workgroup of
// 1024 threads owns one chunk and keeps its order-preserving u32 score keys
// in LDS for the whole kernel. The keys come from one of four sources:
//   SrcScores - precomputed fp32 scores in HBM (the standalone top-K call);
//   SrcScan   - indexer keys streamed from HBM and scored in the kernel (a
//               Full layer: scan and select fused, scores never leave LDS);
//   SrcPool   - indexer keys gathered at candidate-pool positions and scored
//               (a Reindex layer);
//   SrcCand   - indexer keys gathered at the prefill indexer's candidate
//               positions and scored exactly.
// The source also builds the chunk's histogram of the top 11 key bits while
// it writes the keys. The histograms of a row's chunks are summed in the
// workspace with device-scope atomics, and each chunk also publishes the
// suffix sums of its own histogram; after a barrier of the row's S
// workgroups (all resident at once: a launch never holds more workgroups
// than CUs, and the kernel fits one per CU) every chunk knows the bin b1 that
// holds the M-th largest key, and every chunk's count of keys above b1 and
// in it.
//   List path (S > 1 and at most kListCap keys in bin b1 row-wide): each
//     wave first copies its keys in bin b1 or above (a few percent of them)
//     with their indices, in index order, to the start of its own LDS span;
//     the later steps visit only these. Each chunk writes its bin-b1 keys to
//     its segment of a per-row list (segments in chunk order, placed by those
//     counts). After a second barrier every chunk reads the short list and
//     resolves the exact threshold key T, how many entries equal to T are
//     taken, and the counts of entries > T and == T in earlier chunks and in
//     all chunks, with no further exchange. A list of up to kListBatch
//     entries stays in registers for all of these passes; a longer one is
//     read again, batch by batch, in each pass.
//   Radix path (otherwise): two more radix passes over the LDS keys (11 and
//     10 bits), each with a row-wide histogram exchange, then an exchange of
//     the per-chunk counts of keys > T and == T.
// Ties at T go to the lowest entry index (chunks in order, entries in order
// within a chunk). Each chunk compacts its selected entries in index order
// straight into the output, so the output is sorted without a sort. Up to
// two targets (pool size P and K) are selected from the same keys in one
// launch. The last workgroup of a row to leave resets the row's counters and
// histograms, so the workspace is ready for the next launch without a memset.
//
// A Full layer's attention can run in the same launch (scan source, FA): each
// chunk also writes its positions of the last target to LDS in output order,
// attends to them with the attention's per-block step once the keys' LDS
// area is free, publishes its partial softmax state, and after one more row
// barrier writes heads split, split + S, ... as the merge of the row's states
// in slice order (a row of one chunk writes its output directly).
#include "attn_core.hpp"
#include "dot.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kB1 = 2048, kB2 = 2048, kB3 = 1024;   // radix digits 11 | 11 | 10 bits
constexpr int kRowHdr = 16;                          // control words of a row: [0] barrier, [1] exit
constexpr int kListCap = 32768;                      // list entries per (row, target)
constexpr int kListBatch = 16384;                    // list entries held in registers at once
constexpr int kMaxS = 256;                           // chunks per row (<= CUs)
constexpr int kScratchWords = 256;
constexpr int kLdsFixedWords = kB1 + 2 * kB2 + 4 * kMaxS + kScratchWords;
constexpr int kMaxChunk = 32768;
constexpr int kPadTo = 256;                          // keys per wave step of the count/compaction passes
constexpr int kMaxSteps = kMaxChunk / kSelWaves / kPadTo;   // steps per wave (8)
// LDS words the fused attention needs at the start of the keys' area, and the
// most positions its list (the histogram area lh2) holds.
constexpr int kFuseLdsWords = (int)((sizeof(AttnLds<kFuseWaves>) + 255) / 256 * 64);
constexpr int kFuseMaxK = 2 * kB2;

struct SelDev {
    int64_t n;
    int32_t S, chunk, chunk_pad, row0, nt, row_words;
    int32_t pos_lds;                            // the source keeps each key's position in LDS
    int32_t skew;                               // even chunks chunk + skew entries, odd ones chunk - skew
    uint32_t* ctrl;                             // workspace control region
    uint32_t* data;                             // this call's data region
    const int32_t* rowmap;                      // launch row -> row (-1: nothing to do), or null
};

static_assert(kRowHdr + kB1 + 2 * kB2 + 2 * kB3 <= kSelCtrlRowWords, "select control words per row");
static_assert(kMaxS <= kSelCtrlRows, "select rows per launch");

struct SelTgt {
    int32_t* idx;
    float* score;
    int64_t stride;
    int32_t M;
};

__device__ __forceinline__ void put_key(uint32_t* keys, uint32_t* hist, int i, uint32_t key) {
    keys[i] = key;
    if (key) atomicAdd(&hist[key >> 21], 1u);
}

__device__ __forceinline__ void pad_keys(uint32_t* keys, int cnt, int cpad) {
    for (int i = cnt + (int)threadIdx.x; i < cpad; i += kSelThreads) keys[i] = 0u;
}

// ------------------------------------------------------------------ sources

struct SrcScores {
    const float* scores;
    int64_t stride;
    const int32_t* cand;
    int64_t n;

    static constexpr bool kPosLds = false;
    __device__ __forceinline__ int fill(int64_t row, int64_t begin, int cnt, int cpad, uint32_t* keys,
                                        uint32_t* hist, uint32_t*) const {
        const float* p = scores + row * stride + begin;
        for (int i = threadIdx.x; i < cnt; i += kSelThreads) put_key(keys, hist, i, score_key(p[i]));
        pad_keys(keys, cnt, cpad);
        __syncthreads();
        return cnt;
    }
    __device__ __forceinline__ int32_t position(int64_t row, int64_t i) const {
        return cand ? cand[row * n + i] : (int32_t)i;
    }
};

template <int KT, int QT, int D>
struct SrcScan {
    const void* q;
    const uint8_t* k;
    int64_t N;
    int32_t rows_per_seq;
    const int64_t* q_pos;

    static constexpr bool kPosLds = false;       // position = index
    __device__ __forceinline__ int fill(int64_t row, int64_t begin, int cnt, int cpad, uint32_t* keys,
                                        uint32_t* hist, uint32_t*) const {
        using KS = KeySlice<KT, D, QT>;
        constexpr int QB = (QT == kBF16) ? 2 : 4;
        constexpr int U = KS::RAW >= 4 ? 1 : 4 / KS::RAW;   // 64 bytes in flight per lane
        const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
        double qd[D / 4];
        load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
        const int64_t seq = row / rows_per_seq;
        const uint8_t* kb = k + (seq * N + begin) * (int64_t)KS::ROW_BYTES;
        int lim = cnt;                                      // entries >= lim are causally masked
        if (q_pos) {
            const int64_t v = q_pos[row] - begin + 1;
            lim = (int)(v < 0 ? 0 : (v > cnt ? cnt : v));
        }
        if constexpr (KS::RAW == 1) {
            // One 16-byte load per lane and key: batches of 1024 keys, key
            // base + 256u + quad in slot u of its quad's lanes; after the
            // transposed reduction lane lq owns key base + 256 lq + quad. Whole
            // unmasked batches run software-pipelined over three register
            // sets: while a batch is scored the loads of the next two are in
            // flight. The loads are streaming buffer loads bounded by the
            // chunk's causal limit, so the look-ahead past the last batch
            // returns zeros without touching memory, and every load is
            // unconditional (the compiler's wait counts stay exact). The
            // rest is predicated.
            constexpr int kB = kSelThreads;
            constexpr int kStreaming = 2;       // cache policy: non-temporal
            const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint8_t*>(kb), (short)0, lim * KS::ROW_BYTES, kRsrcWord3);
            const int qoff = quad * KS::ROW_BYTES + lq * (KS::ROW_BYTES / 4);
            const uint8_t* kq = kb + (int64_t)quad * KS::ROW_BYTES + lq * (KS::ROW_BYTES / 4);
            const int nfull = lim / kB;
            auto load_batch = [&](int bi, uint4 (&r)[4]) {
#pragma unroll
                for (int u = 0; u < 4; ++u)
                    r[u] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(
                                                         kr, (bi * kB + u * 256) * KS::ROW_BYTES + qoff, 0, kStreaming));
            };
            auto score_batch = [&](const uint4 (&r)[4], int base, bool masked) {
                typename KS::Part acc[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    KS sl;
                    sl.raw[0] = r[u];
                    acc[u] = sl.dot(qd);
                }
                const auto v = quad_transpose_sum(acc, lq);
                const int i = base + lq * 256 + quad;
                if (!masked) put_key(keys, hist, i, score_key(round_score(v)));
                else if (i < cnt) put_key(keys, hist, i, (i < lim) ? score_key(round_score(v)) : 0u);
            };
            if (nfull > 0) {
                uint4 ra[4], rb[4], rc[4];
                load_batch(0, ra);
                load_batch(1, rb);
                int bi = 0;
                for (; bi + 3 <= nfull; bi += 3) {
                    load_batch(bi + 2, rc);
                    score_batch(ra, bi * kB, false);
                    load_batch(bi + 3, ra);
                    score_batch(rb, (bi + 1) * kB, false);
                    load_batch(bi + 4, rb);
                    score_batch(rc, (bi + 2) * kB, false);
                }
                if (bi < nfull) score_batch(ra, bi * kB, false);
                if (bi + 1 < nfull) score_batch(rb, (bi + 1) * kB, false);
            }
            for (int base = nfull * kB; base < cnt; base += kB) {
                uint4 r[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int i = base + u * 256 + quad;
                    r[u] = (i < lim) ? ld_stream16(kq + (int64_t)(base + u * 256) * KS::ROW_BYTES) : make_uint4(0, 0, 0, 0);
                }
                score_batch(r, base, true);
            }
            pad_keys(keys, cnt, cpad);
            __syncthreads();
            return cnt;
        }
        for (int base = 0; base < cnt; base += (kSelThreads / 4) * U) {
            KS s[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * (kSelThreads / 4) + quad;
                if (i < lim) s[u].load(kb + (int64_t)i * KS::ROW_BYTES, lq);
                else for (int j = 0; j < KS::RAW; ++j) s[u].raw[j] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * (kSelThreads / 4) + quad;
                const auto v = quad_sum(s[u].dot(qd));
                if (lq == 0 && i < cnt) put_key(keys, hist, i, (i < lim) ? score_key(round_score(v)) : 0u);
            }
        }
        pad_keys(keys, cnt, cpad);
        __syncthreads();
        return cnt;
    }
    __device__ __forceinline__ int32_t position(int64_t, int64_t i) const { return (int32_t)i; }
};

template <int KT, int QT, int D>
struct SrcPool {
    const void* q;
    const uint8_t* k;
    int64_t N;
    const int32_t* pool;
    int64_t P;
    int32_t rows_per_seq;                        // row r reads sequence r / rows_per_seq

    static constexpr bool kPosLds = true;        // positions come from the pool: kept in LDS when they fit
    __device__ __forceinline__ int fill(int64_t row, int64_t begin, int cnt, int cpad, uint32_t* keys,
                                        uint32_t* hist, uint32_t* posl) const {
        using KS = KeySlice<KT, D, QT>;
        constexpr int QB = (QT == kBF16) ? 2 : 4;
        constexpr int U = KS::RAW >= 4 ? 1 : 4 / KS::RAW;
        const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
        double qd[D / 4];
        load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
        const uint8_t* kb = k + (row / rows_per_seq) * N * (int64_t)KS::ROW_BYTES;
        const int32_t* pr = pool + row * P + begin;
        for (int base = 0; base < cnt; base += (kSelThreads / 4) * U) {
            KS s[U];
            bool ok[U];
            int32_t pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * (kSelThreads / 4) + quad;
                pv[u] = (i < cnt) ? pr[i] : -1;
                ok[u] = pv[u] >= 0 && (int64_t)pv[u] < N;
                if (ok[u]) s[u].load(kb + (int64_t)pv[u] * KS::ROW_BYTES, lq);
                else for (int j = 0; j < KS::RAW; ++j) s[u].raw[j] = make_uint4(0, 0, 0, 0);
            }
            if constexpr (U == 4) {
                // transposed quad reduction: lane lq ends with the sum of slot lq's key
                typename KS::Part acc[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) acc[u] = s[u].dot(qd);
                const auto v = quad_transpose_sum(acc, lq);
                const int i = base + lq * (kSelThreads / 4) + quad;
                const bool okl = lq == 0 ? ok[0] : lq == 1 ? ok[1] : lq == 2 ? ok[2] : ok[3];
                const int32_t pvl = lq == 0 ? pv[0] : lq == 1 ? pv[1] : lq == 2 ? pv[2] : pv[3];
                if (i < cnt) {
                    put_key(keys, hist, i, okl ? score_key(round_score(v)) : 0u);
                    if (posl) posl[i] = (uint32_t)pvl;
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const int i = base + u * (kSelThreads / 4) + quad;
                    const auto v = quad_sum(s[u].dot(qd));
                    if (lq == 0 && i < cnt) {
                        put_key(keys, hist, i, ok[u] ? score_key(round_score(v)) : 0u);
                        if (posl) posl[i] = (uint32_t)pv[u];
                    }
                }
            }
        }
        pad_keys(keys, cnt, cpad);
        __syncthreads();
        return cnt;
    }
    __device__ __forceinline__ int32_t position(int64_t row, int64_t i) const { return pool[row * P + i]; }
};

// Candidate lists of the prefill indexer: entry i of a row is slot i % cap of
// list i / cap, valid below that list's count; entries are in position order.
// When positions are kept in LDS the chunk's valid entries are stored densely
// (key v = the v-th valid entry, still in position order) and the select runs
// over those only; otherwise key i is entry begin + i.
template <int KT, int QT, int D>
struct SrcCand {
    const void* q;
    const uint8_t* k;
    int64_t N;
    int32_t rows_per_seq;
    const int32_t* cand;
    const uint32_t* cnt;
    int32_t nranges, cap;

    __device__ __forceinline__ int32_t entry(int64_t row, int i) const {
        const int r = i / cap, sl = i - r * cap;
        const uint32_t c = cnt[row * nranges + r];
        return (uint32_t)sl < (c < (uint32_t)cap ? c : (uint32_t)cap) ? cand[(row * nranges + r) * cap + sl] : -1;
    }

    // Only the valid slots are visited: the chunk's keys start at 0 (padding)
    // and each valid slot (list r, slot sl) writes its key at entry r*cap + sl.
    static constexpr bool kPosLds = true;        // positions come from the lists: kept in LDS when they fit
    __device__ __forceinline__ int fill(int64_t row, int64_t begin, int cnt_, int cpad, uint32_t* keys,
                                        uint32_t* hist, uint32_t* posl) const {
        using KS = KeySlice<KT, D, QT>;
        constexpr int QB = (QT == kBF16) ? 2 : 4;
        constexpr int U = KS::RAW >= 4 ? 2 : 8 / KS::RAW;
        constexpr int kMaxLists = 16;
        const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
        const bool dense = posl != nullptr;
        double qd[D / 4];
        load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
        const uint8_t* kb = k + (row / rows_per_seq) * N * (int64_t)KS::ROW_BYTES;
        // entries [begin, begin + cnt_) of the row cover lists r0 .. r1 - 1 (a chunk is whole lists or a part of one)
        uint32_t lo[kMaxLists], nv[kMaxLists];  // per list: first valid entry, number of valid entries in this chunk
        uint32_t total = 0;
#pragma unroll
        for (int r = 0; r < kMaxLists; ++r) {
            lo[r] = 0u;
            nv[r] = 0u;
            if (r < nranges) {
                const uint32_t c = cnt[row * nranges + r];
                const int64_t e0 = (int64_t)r * cap, e1 = e0 + (c < (uint32_t)cap ? c : (uint32_t)cap);
                const int64_t a0 = e0 > begin ? e0 : begin, a1 = e1 < begin + cnt_ ? e1 : begin + cnt_;
                if (a1 > a0) {
                    lo[r] = (uint32_t)(a0 - begin);
                    nv[r] = (uint32_t)(a1 - a0);
                }
            }
            total += nv[r];
        }
        // more valid entries than the dense LDS area holds (its size may be below the chunk's):
        // the row is left alone, every thread returns -1 (total is the same in all of them)
        if (dense && total > (uint32_t)cpad) return -1;
        {
            const int zfrom = dense ? (int)total : 0;
            const int zto = dense ? (int)((total + kPadTo - 1) / kPadTo * kPadTo) : cpad;
            for (int i = zfrom + (int)threadIdx.x; i < zto; i += kSelThreads) keys[i] = 0u;
        }
        if (dense) {
            // Pass 1: every list's valid positions to LDS (independent, coalesced loads).
            // Pass 2: quads take U entries each, read their positions from LDS, issue
            // all U key loads, then score them.
            uint32_t v0 = 0;
#pragma unroll
            for (int r = 0; r < kMaxLists; ++r) {
                const int32_t* lst = cand + (row * nranges + r) * (int64_t)cap + (int64_t)(begin + lo[r] - (int64_t)r * cap);
                for (uint32_t sl = threadIdx.x; sl < nv[r]; sl += kSelThreads) posl[v0 + sl] = (uint32_t)lst[sl];
                v0 += nv[r];
            }
            __syncthreads();
            for (uint32_t base = 0; base < total; base += (kSelThreads / 4) * U) {
                KS sk[U];
                int32_t pv[U];
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t v = base + u * (kSelThreads / 4) + quad;
                    pv[u] = v < total ? (int32_t)posl[v] : -1;
                    if (pv[u] >= 0 && (int64_t)pv[u] < N) sk[u].load(kb + (int64_t)pv[u] * KS::ROW_BYTES, lq);
                    else for (int j = 0; j < KS::RAW; ++j) sk[u].raw[j] = make_uint4(0, 0, 0, 0);
                }
                if constexpr (U == 8) {
                    // two groups of four slots, transposed quad reduction: lane lq writes slot 4h + lq
                    auto group = [&](const KS& a, const KS& b, const KS& c, const KS& d, int32_t p0, int32_t p1,
                                     int32_t p2, int32_t p3, int h) {
                        const typename KS::Part acc[4] = {a.dot(qd), b.dot(qd), c.dot(qd), d.dot(qd)};
                        const auto sv = quad_transpose_sum(acc, lq);
                        const int32_t p = lq == 0 ? p0 : lq == 1 ? p1 : lq == 2 ? p2 : p3;
                        const uint32_t v = base + (4 * h + lq) * (kSelThreads / 4) + quad;
                        if (v < total)          // an entry without a valid position is padding (key 0)
                            put_key(keys, hist, (int)v, (p >= 0 && (int64_t)p < N) ? score_key(round_score(sv)) : 0u);
                    };
                    group(sk[0], sk[1], sk[2], sk[3], pv[0], pv[1], pv[2], pv[3], 0);
                    group(sk[4], sk[5], sk[6], sk[7], pv[4], pv[5], pv[6], pv[7], 1);
                } else {
#pragma unroll
                    for (int u = 0; u < U; ++u) {
                        const auto sv = quad_sum(sk[u].dot(qd));
                        const uint32_t v = base + u * (kSelThreads / 4) + quad;
                        if (lq == 0 && v < total)
                            put_key(keys, hist, (int)v, (pv[u] >= 0 && (int64_t)pv[u] < N) ? score_key(round_score(sv)) : 0u);
                    }
                }
            }
            __syncthreads();
            return (int)total;
        }
        __syncthreads();                        // the zero fill is complete before valid keys land
        for (uint32_t base = 0; base < total; base += (kSelThreads / 4) * U) {
            KS s[U];
            int32_t ent[U], pv[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const uint32_t v = base + u * (kSelThreads / 4) + quad;     // v-th valid entry of the chunk
                ent[u] = -1;
                int32_t pos = -1;
                if (v < total) {
                    uint32_t rest = v;
#pragma unroll
                    for (int r = 0; r < kMaxLists; ++r) {
                        if (ent[u] < 0 && rest < nv[r]) ent[u] = (int32_t)(lo[r] + rest);
                        else if (ent[u] < 0) rest -= nv[r];
                    }
                    const int64_t e = begin + ent[u];
                    const int r = (int)(e / cap), sl = (int)(e - (int64_t)r * cap);
                    pos = cand[(row * nranges + r) * cap + sl];
                }
                pv[u] = pos;
                if (pos >= 0 && (int64_t)pos < N) {
                    s[u].load(kb + (int64_t)pos * KS::ROW_BYTES, lq);
                } else {
                    for (int j = 0; j < KS::RAW; ++j) s[u].raw[j] = make_uint4(0, 0, 0, 0);
                    ent[u] = -1;                // no position: the entry stays padding
                }
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const auto sv = quad_sum(s[u].dot(qd));
                const uint32_t v = base + u * (kSelThreads / 4) + quad;
                if (lq != 0) continue;
                if (dense) {
                    if (v < total) {            // an entry without a valid position is padding (key 0)
                        put_key(keys, hist, (int)v, ent[u] >= 0 ? score_key(round_score(sv)) : 0u);
                        posl[v] = (uint32_t)pv[u];
                    }
                } else if (ent[u] >= 0) {
                    put_key(keys, hist, ent[u], score_key(round_score(sv)));
                }
            }
        }
        __syncthreads();
        return dense ? (int)total : cnt_;
    }
    __device__ __forceinline__ int32_t position(int64_t row, int64_t i) const { return entry(row, (int)i); }
};

// ------------------------------------------------------------ block helpers

struct Found {
    uint32_t bin, rem, total;
};

// Walk the histogram from the highest bin down and find the bin where the
// running count reaches `need` (1 <= need <= total is required for bin/rem
// to be meaningful); rem = how many entries of that bin are needed.
__device__ Found block_find(const uint32_t* hist, int nb, uint32_t need, uint32_t* sm) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int per = nb / kSelThreads;
    const int top = nb - 1 - tid * per;
    uint32_t s = 0;
    for (int j = 0; j < per; ++j) s += hist[top - j];
    const uint32_t inc = wave_incl_scan(s);
    if (lane == kWave - 1) sm[wave] = inc;
    __syncthreads();
    uint32_t before = inc - s, total = 0;
    for (int w = 0; w < kSelWaves; ++w) {
        const uint32_t t = sm[w];
        total += t;
        if (w < wave) before += t;
    }
    if (before < need && need <= before + s) {
        uint32_t c = before;
        for (int j = 0; j < per; ++j) {
            const uint32_t h = hist[top - j];
            if (c + h >= need) {
                sm[kSelWaves] = (uint32_t)(top - j);
                sm[kSelWaves + 1] = need - c;
                break;
            }
            c += h;
        }
    }
    __syncthreads();
    Found f{sm[kSelWaves], sm[kSelWaves + 1], total};
    __syncthreads();
    return f;
}

// block_find over NT histograms at once (histogram j at hist + j * hstride,
// target need[j]; need[j] = 0 skips it) with two block barriers. The
// histograms are not read after the second one, and a later call rewrites the
// scratch words only after its own first barrier, when every thread has read
// this call's result.
template <int NT>
__device__ __forceinline__ void block_find_multi(const uint32_t* hist, int nb, int hstride, const uint32_t (&need)[2],
                                                 uint32_t* sm, Found (&out)[2]) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int per = nb / kSelThreads;
    const int top = nb - 1 - tid * per;
    uint32_t s[2] = {0u, 0u}, inc[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        for (int i = 0; i < per; ++i) s[j] += hist[j * hstride + top - i];
        inc[j] = wave_incl_scan(s[j]);
        if (lane == kWave - 1) sm[j * kSelWaves + wave] = inc[j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        uint32_t before = inc[j] - s[j], total = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const uint32_t t = sm[j * kSelWaves + w];
            total += t;
            if (w < wave) before += t;
        }
        out[j].total = total;
        if (before < need[j] && need[j] <= before + s[j]) {
            uint32_t c = before;
            for (int i = 0; i < per; ++i) {
                const uint32_t h = hist[j * hstride + top - i];
                if (c + h >= need[j]) {
                    sm[2 * kSelWaves + 2 * j] = (uint32_t)(top - i);
                    sm[2 * kSelWaves + 2 * j + 1] = need[j] - c;
                    break;
                }
                c += h;
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        out[j].bin = sm[2 * kSelWaves + 2 * j];
        out[j].rem = sm[2 * kSelWaves + 2 * j + 1];
    }
}

__device__ __forceinline__ void push_hist(const uint32_t* lh, uint32_t* gh, int nb) {
    for (int b = threadIdx.x; b < nb; b += kSelThreads) {
        const uint32_t c = lh[b];
        if (c) add_rlx(&gh[b], c);
    }
}

template <int NB>
__device__ __forceinline__ void pull_hist(uint32_t* lh, const uint32_t* gh) {
    static_assert(NB % kSelThreads == 0, "whole bins per thread");
    constexpr int P = NB / kSelThreads;
    uint32_t v[P];
#pragma unroll
    for (int i = 0; i < P; ++i) v[i] = ld_rlx(&gh[threadIdx.x + i * kSelThreads]);   // all in flight
#pragma unroll
    for (int i = 0; i < P; ++i) lh[threadIdx.x + i * kSelThreads] = v[i];
    __syncthreads();
}

// ------------------------------------------------------------------ kernel

enum : int { kPathAll = 0, kPathList = 1, kPathRadix = 2 };

// Element j of a per-target pair, as a select on values (an indexed access
// would force the pair into scratch memory).
template <int NT, class T>
__device__ __forceinline__ T pick(T a0, T a1, int j) {
    return (NT > 1 && j) ? a1 : a0;
}

template <class Src, int NT, bool FA>
__global__ void __launch_bounds__(kSelThreads) k_select(Src src, SelDev g, SelTgt t0, SelTgt t1, AttnFuse af) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int S = g.S;
    const int lrow = blockIdx.x / S;
    const int split = blockIdx.x - lrow * S;
    const int64_t row = g.rowmap ? (int64_t)g.rowmap[g.row0 + lrow] : (int64_t)g.row0 + lrow;
    if (row < 0) return;                        // the same for every workgroup of the launch row
    // chunk s starts at s * chunk, plus skew when s is odd (an even chunk before it took skew more)
    const int64_t begin = (int64_t)split * g.chunk + ((split & 1) ? g.skew : 0);
    int cnt = (int)min((int64_t)g.chunk + ((split & 1) ? -g.skew : g.skew), g.n - begin);
    int cpad = g.chunk_pad;                     // LDS key area; after the fill: the keys written, rounded up
    const bool multi = S > 1;

    uint32_t* keys = lds;                       // [cpad] score keys, 0 past cnt
    const bool pos_lds = Src::kPosLds && g.pos_lds;
    uint32_t* posl = pos_lds ? lds + cpad : nullptr;     // [cpad] positions of the keys (sources that keep them)
    // (the fused attention reuses the keys' area, at least kFuseLdsWords)
    uint32_t* lh1 = lds + (pos_lds ? 2 * cpad : (FA && cpad < kFuseLdsWords ? kFuseLdsWords : cpad));   // [kB1] this chunk's top-digit histogram
    uint32_t* lh2 = lh1 + kB1;                  // [2*kB2] row histogram, then later histograms
    uint32_t* cnts = lh2 + 2 * kB2;             // [S][2 targets][> T, == T]
    uint32_t* sm = cnts + 4 * kMaxS;            // scratch
    uint32_t* status = g.ctrl;
    uint32_t* rc = g.ctrl + kSelCtrlOffsetWords + (size_t)lrow * kSelCtrlRowWords;   // zero between calls
    uint32_t* ctrl = rc;
    uint32_t* exitc = rc + 1;
    uint32_t* gh1 = rc + kRowHdr;
    uint32_t* gh2 = gh1 + kB1;
    uint32_t* gh3 = gh2 + 2 * kB2;
    uint32_t* rw = g.data + (size_t)lrow * g.row_words;                              // data, any content
    uint32_t* gcnt = rw;                        // [S][2][> T, == T]
    uint32_t* gsuf = gcnt + 4 * S;              // [S][kB1] per-chunk suffix sums of the top-digit histogram
    uint32_t* glist = gsuf + (size_t)S * kB1;  // [2][kListCap] bin-b1 keys, one segment per chunk in chunk order
    uint32_t gen = 0;

    const uint32_t M[2] = {(uint32_t)t0.M, (uint32_t)t1.M};

    for (int i = tid; i < kB1; i += kSelThreads) lh1[i] = 0u;
    if (tid < 4) sm[204 + tid] = 0u;          // list slot cursors and tie counters of the two targets
    __syncthreads();
    cnt = src.fill(row, begin, cnt, cpad, keys, lh1, posl);   // keys + lh1 (+ positions); ends with a block barrier
    if (cnt < 0) return;                        // a row over the dense capacity (one chunk per row): left to the caller
    cpad = (cnt + kPadTo - 1) / kPadTo * kPadTo;

    // ---- row histogram of the top 11 bits; each chunk also publishes the
    // suffix sums of its own histogram (keys at or above each bin)
    const uint32_t* G = lh1;
    if (multi) {
        push_hist(lh1, gh1, kB1);
        {
            // bins 2047 - 2*tid and 2046 - 2*tid, scanned from the top
            const int hi = kB1 - 1 - 2 * tid;
            const uint32_t a = lh1[hi], b = lh1[hi - 1];
            const uint32_t inc = wave_incl_scan(a + b);
            if (lane == kWave - 1) sm[wave] = inc;
            __syncthreads();
            uint32_t before = inc - (a + b);
            for (int w = 0; w < wave; ++w) before += sm[w];
            uint32_t* mine = gsuf + (size_t)split * kB1;
            st_rlx(&mine[hi], before + a);
            st_rlx(&mine[hi - 1], before + a + b);
        }
        row_barrier(ctrl, S, gen, status);
        {
            // both loads in flight before either is stored (a loop would wait on each)
            static_assert(kB1 == 2 * kSelThreads, "two row-histogram bins per thread");
            const uint32_t h0 = ld_rlx(&gh1[tid]), h1 = ld_rlx(&gh1[tid + kSelThreads]);
            lh2[tid] = h0;
            lh2[tid + kSelThreads] = h1;
        }
        __syncthreads();
        G = lh2;
    }
    int path[2] = {kPathAll, kPathAll};
    uint32_t b1[2] = {0, 0}, rem[2] = {0, 0}, C[2] = {0, 0}, T[2] = {0, 0}, need[2] = {0, 0};
    {
        Found f[2];
        block_find_multi<NT>(G, kB1, 0, M, sm, f);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (f[j].total > M[j]) {
                b1[j] = f[j].bin;
                rem[j] = f[j].rem;
                C[j] = G[f[j].bin];
                path[j] = (multi && C[j] <= (uint32_t)kListCap) ? kPathList : kPathRadix;
            }
        }
    }
    __syncthreads();                            // G (lh2) may be overwritten below
    const bool any_list = path[0] == kPathList || (NT > 1 && path[1] == kPathList);
    const bool any_radix = path[0] == kPathRadix || (NT > 1 && path[1] == kPathRadix);
    const bool any_other = path[0] != kPathList || (NT > 1 && path[1] != kPathList);

    // ---- each wave owns a contiguous span of kPadTo-key steps; its lanes keep
    // the span's keys in registers for the passes below: component u of lane
    // l's word for step t is the key of chunk index w0 + t*kPadTo + 64u + l,
    // so one ballot per component covers 64 consecutive indices in order
    int span = (cpad + kSelWaves - 1) / kSelWaves;
    span = (span + kPadTo - 1) / kPadTo * kPadTo;
    const int w0 = min(cpad, wave * span), w1 = min(cpad, w0 + span);
    const int nst = (w1 - w0) / kPadTo;         // steps of this wave (<= kMaxSteps)
    static_assert(kPadTo == 4 * kWave, "four components of 64 keys per step");
    uint4 kreg[kMaxSteps];
    auto load_kreg = [&]() {
#pragma unroll
        for (int t = 0; t < kMaxSteps; ++t) {
            const uint32_t* kp = &keys[w0 + t * kPadTo + lane];
            kreg[t] = (t < nst) ? make_uint4(kp[0], kp[kWave], kp[2 * kWave], kp[3 * kWave]) : make_uint4(0, 0, 0, 0);
        }
    };
    uint32_t* wcnt = sm + 64;                   // [2][16][gt, eq] per-wave counts of this chunk

    // ---- extraction: when every target takes the list path, each wave copies
    // its keys in bin min(b1) or above - the only keys any later step needs -
    // as (key, chunk index) pairs in index order to the start of its own LDS
    // span. A wave whose pairs would not fit its span restores the span and
    // keeps working on all its keys (ext = false); so do all waves on the
    // other paths, which read the LDS keys of the whole chunk.
    // cnts[s][j] = (keys above b1, keys in b1) of chunk s, from the suffix
    // sums at b1 and b1 + 1 (S * NT <= 512 pairs, one per thread); the loads
    // stay in flight during the extraction pass
    const int si = tid / NT, sj = tid - si * NT;
    const bool sl = any_list && tid < S * NT && pick<NT>(path[0], path[1], sj) == kPathList;
    // (bin b1 + 1 exists: the largest score key, that of +inf, is in bin
    // 0xFF800000 >> 21 = 2044; the values are used as loaded, so nothing
    // here waits for the loads)
    static_assert((0xFF800000u >> 21) + 1 < (uint32_t)kB1, "a bin above every score key's");
    uint32_t s_at = 0u, s_ab = 0u;
    if (sl) {
        const uint32_t bj = pick<NT>(b1[0], b1[1], sj);
        const uint32_t* su = gsuf + (size_t)si * kB1;
        s_at = ld_rlx(&su[bj]);
        s_ab = ld_rlx(&su[min(bj + 1, (uint32_t)kB1 - 1)]);
    }
    uint2* pairs = reinterpret_cast<uint2*>(keys + w0);
    uint32_t npair = 0;                         // wave-uniform
    bool ext = false;
    if (any_list && !any_other) {
        load_kreg();
        const uint32_t bmin = (NT > 1 && b1[1] < b1[0]) ? b1[1] : b1[0];
        const uint32_t lowk = (bmin << 21) > 1u ? (bmin << 21) : 1u;
        const uint32_t cap = (uint32_t)(w1 - w0) >> 1;
#pragma unroll
        for (int t = 0; t < kMaxSteps; ++t) {
            if (t >= nst) break;
            const int ib = w0 + t * kPadTo + lane;
            const uint32_t kv[4] = {kreg[t].x, kreg[t].y, kreg[t].z, kreg[t].w};
            // candidates of component u (indices ib + 64u over the lanes) take
            // consecutive slots in lane order: slots follow index order
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const bool c = kv[u] >= lowk;
                const uint64_t m = __ballot(c);
                const uint32_t slot = npair + lanes_below(m);
                if (c && slot < cap) pairs[slot] = make_uint2(kv[u], (uint32_t)(ib + kWave * u));
                npair += (uint32_t)__popcll(m);
            }
        }
        ext = npair <= cap;
        if (!ext) {
#pragma unroll
            for (int t = 0; t < kMaxSteps; ++t) {
                if (t >= nst) continue;
                uint32_t* kp = &keys[w0 + t * kPadTo + lane];
                kp[0] = kreg[t].x;
                kp[kWave] = kreg[t].y;
                kp[2 * kWave] = kreg[t].z;
                kp[3 * kWave] = kreg[t].w;
            }
        }
    }
    // Visit this wave's keys in index order, 64 at a time: f(key, chunk index,
    // valid) is called by every lane with wave-uniform control flow.
    auto for_keys = [&](auto&& f) {
        if (ext) {
            for (uint32_t i0 = 0; i0 < npair; i0 += kWave) {
                const uint32_t i = i0 + (uint32_t)lane;
                const uint2 pr = i < npair ? pairs[i] : make_uint2(0u, 0u);
                f(pr.x, pr.y, i < npair);
            }
        } else {
            load_kreg();
#pragma unroll
            for (int t = 0; t < kMaxSteps; ++t) {
                if (t >= nst) break;
                const uint32_t ib = (uint32_t)(w0 + t * kPadTo + lane);
                f(kreg[t].x, ib, true);
                f(kreg[t].y, ib + kWave, true);
                f(kreg[t].z, ib + 2u * kWave, true);
                f(kreg[t].w, ib + 3u * kWave, true);
            }
        }
    };

    // ---- list path, part 1: every chunk's counts above bin b1 and in it come
    // from the published suffix sums, so each chunk knows its segment of the
    // row's list (chunks in order) without an atomic; its waves reserve slots
    // inside the segment and write their bin-b1 keys there.
    if (any_list) {
        uint32_t inb[2] = {0u, 0u};
        for_keys([&](uint32_t k, uint32_t, bool v) {
#pragma unroll
            for (int j = 0; j < NT; ++j) inb[j] += (uint32_t)__popcll(__ballot(v && k != 0u && (k >> 21) == b1[j]));
        });
        uint32_t off[2] = {0u, 0u};             // this wave's first slot in the chunk's segment
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] == kPathList && lane == 0 && inb[j]) off[j] = atomicAdd(&sm[204 + j], inb[j]);
            off[j] = (uint32_t)__builtin_amdgcn_readfirstlane((int)off[j]);
        }
        if (sl) {
            cnts[(si * 2 + sj) * 2 + 0] = s_ab;
            cnts[(si * 2 + sj) * 2 + 1] = s_at - s_ab;
        }
        __syncthreads();
        uint32_t lo[2] = {0u, 0u}, hi[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] != kPathList) continue;
            uint32_t b = 0;
            for (int s = lane; s < split; s += kWave) b += cnts[(s * 2 + j) * 2 + 1];
            lo[j] = wave_sum(b);
            hi[j] = lo[j] + cnts[(split * 2 + j) * 2 + 1];
            if (wave == 0 && lane == 0) {
                sm[200 + 2 * j] = lo[j];        // this chunk's range [lo, hi) of the row's list
                sm[201 + 2 * j] = hi[j];
            }
        }
        uint32_t run[2] = {lo[0] + off[0], lo[1] + off[1]};
        for_keys([&](uint32_t k, uint32_t, bool v) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (path[j] != kPathList) continue;
                const bool c = v && k != 0u && (k >> 21) == b1[j];
                const uint64_t m = __ballot(c);
                const uint32_t slot = run[j] + lanes_below(m);
                if (c && slot < hi[j] && slot < (uint32_t)kListCap)   // holds: the waves' counts sum to hi - lo
                    st_rlx(&glist[(size_t)j * kListCap + slot], k);
                run[j] += (uint32_t)__popcll(m);
            }
        });
    }

    // ---- radix path: two more digit passes over the LDS keys with row exchanges
    if (any_radix) {
        for (int i = tid; i < 2 * kB2; i += kSelThreads) lh2[i] = 0u;
        __syncthreads();
        for (int i = tid; i < cnt; i += kSelThreads) {
            const uint32_t k = keys[i];
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix && (k >> 21) == b1[j]) atomicAdd(&lh2[j * kB2 + ((k >> 10) & 2047u)], 1u);
        }
        __syncthreads();
        if (multi) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix) push_hist(lh2 + j * kB2, gh2 + j * kB2, kB2);
            row_barrier(ctrl, S, gen, status);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix) pull_hist<kB2>(lh2 + j * kB2, gh2 + j * kB2);
        }
        uint32_t pre2[2] = {0, 0};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] != kPathRadix) continue;
            const Found f = block_find(lh2 + j * kB2, kB2, rem[j], sm);
            pre2[j] = (b1[j] << 11) | f.bin;
            rem[j] = f.rem;
        }
        for (int i = tid; i < 2 * kB2; i += kSelThreads) lh2[i] = 0u;
        __syncthreads();
        for (int i = tid; i < cnt; i += kSelThreads) {
            const uint32_t k = keys[i];
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix && (k >> 10) == pre2[j]) atomicAdd(&lh2[j * kB3 + (k & 1023u)], 1u);
        }
        __syncthreads();
        if (multi) {
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix) push_hist(lh2 + j * kB3, gh3 + j * kB3, kB3);
            row_barrier(ctrl, S, gen, status);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                if (path[j] == kPathRadix) pull_hist<kB3>(lh2 + j * kB3, gh3 + j * kB3);
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] != kPathRadix) continue;
            const Found f = block_find(lh2 + j * kB3, kB3, rem[j], sm);
            T[j] = (pre2[j] << 10) | f.bin;
            need[j] = f.rem;
        }
    }

    // ---- list path, part 2: after the row barrier every chunk reads the
    // row's lists, resolves T and the tie count, and counts the entries > T
    // and == T before its own segment and in all segments
    uint32_t lgt_all[2] = {0u, 0u}, leq_all[2] = {0u, 0u};   // list entries > T and == T (list targets)
    if (any_list) {
        row_barrier(ctrl, S, gen, status);
        constexpr int R = kListBatch / kSelThreads;
        uint32_t ent[2][R];
        int rn[2] = {0, 0};                     // list slots per thread in use in the current batch (uniform)
        int nbat = 0;                           // batches of the longest list (uniform)
#pragma unroll
        for (int j = 0; j < NT; ++j)
            if (path[j] == kPathList) nbat = max(nbat, (int)((C[j] + kListBatch - 1) / kListBatch));
        // Batch bi of the list targets: entry tid + r * kSelThreads of the batch
        // is list entry bi * kListBatch + tid + r * kSelThreads. Coherent buffer
        // loads: entries past the list's end read 0 (a padding key) without a
        // branch, so all of a thread's loads are in flight together; ent[j][r]
        // is read only for r < rn[j] and left unset otherwise, so the loads need
        // no merge with a default.
        auto ld_batch = [&](int bi) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                const uint32_t cj = path[j] == kPathList ? C[j] : 0u;
                const uint32_t base = (uint32_t)bi * kListBatch;
                const uint32_t nb = cj > base ? min(cj - base, (uint32_t)kListBatch) : 0u;
                rn[j] = (int)((nb + kSelThreads - 1) / kSelThreads);
                const __amdgpu_buffer_rsrc_t lr = __builtin_amdgcn_make_buffer_rsrc(
                    glist + (size_t)j * kListCap + base, (short)0, (int)(nb * 4u), kRsrcWord3);
#pragma unroll
                for (int r = 0; r < R; ++r)
                    if (r < rn[j])              // uniform
                        ent[j][r] = __builtin_amdgcn_raw_buffer_load_b32(lr, (tid + r * kSelThreads) * 4, 0, kCoherent);
            }
        };
        // a pass over the list: one batch in registers is reused, longer lists are read again
        auto reload = [&](int bi) {
            if (nbat > 1) ld_batch(bi);
        };
        ld_batch(0);
        // both targets' digit histograms side by side: bits 10..20, then bits 0..9
        uint32_t nd[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < NT; ++j) nd[j] = path[j] == kPathList ? rem[j] : 0u;
        for (int i = tid; i < NT * kB2; i += kSelThreads) lh2[i] = 0u;
        __syncthreads();
        for (int bi = 0; bi < nbat; ++bi) {
            if (bi > 0) ld_batch(bi);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r >= rn[j]) break;
                    const uint32_t k = ent[j][r];
                    if (k) atomicAdd(&lh2[j * kB2 + ((k >> 10) & 2047u)], 1u);
                }
            }
        }
        __syncthreads();
        Found f2[2];
        block_find_multi<NT>(lh2, kB2, kB2, nd, sm, f2);
        // The entries of bin (b1, b2) - usually a handful - are collected and
        // ranked directly: T is the key k with (# > k) < rem <= (# >= k). A
        // target with more of them than one per thread takes a histogram of
        // the low 10 bits instead.
        uint32_t* tie = lh2;                    // [2][kSelThreads] (the histogram is no longer read)
        for (int bi = 0; bi < nbat; ++bi) {
            reload(bi);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r >= rn[j]) break;
                    const uint32_t k = ent[j][r];
                    if (k && ((k >> 10) & 2047u) == f2[j].bin) {
                        const uint32_t slot = atomicAdd(&sm[206 + j], 1u);
                        if (slot < (uint32_t)kSelThreads) tie[j * kSelThreads + slot] = k;
                    }
                }
            }
        }
        __syncthreads();
        uint32_t ntie[2] = {0u, 0u};
        bool big = false;
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            ntie[j] = sm[206 + j];
            big = big || (path[j] == kPathList && ntie[j] > (uint32_t)kSelThreads);
        }
        uint32_t tbin[2] = {0u, 0u}, gt_t[2] = {0u, 0u}, eq_t[2] = {0u, 0u};   // in bin (b1, b2): > T, == T
        if (!big) {
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (path[j] != kPathList || (uint32_t)tid >= ntie[j]) continue;
                const uint32_t k = tie[j * kSelThreads + tid];
                uint32_t gt = 0, ge = 0;
                for (uint32_t i = 0; i < ntie[j]; ++i) {
                    const uint32_t v = tie[j * kSelThreads + i];
                    gt += (uint32_t)(v > k);
                    ge += (uint32_t)(v >= k);
                }
                if (gt < f2[j].rem && f2[j].rem <= ge) {   // every thread holding T writes the same values
                    sm[208 + 4 * j] = k & 1023u;
                    sm[209 + 4 * j] = f2[j].rem - gt;
                    sm[210 + 4 * j] = gt;
                    sm[211 + 4 * j] = ge - gt;
                }
            }
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                tbin[j] = sm[208 + 4 * j];
                need[j] = sm[209 + 4 * j];
                gt_t[j] = sm[210 + 4 * j];
                eq_t[j] = sm[211 + 4 * j];
            }
        } else {
            Found f3[2];
            for (int i = tid; i < NT * kB3; i += kSelThreads) lh2[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NT; ++j) nd[j] = path[j] == kPathList ? f2[j].rem : 0u;
            for (int bi = 0; bi < nbat; ++bi) {
                reload(bi);
#pragma unroll
                for (int j = 0; j < NT; ++j) {
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        if (r >= rn[j]) break;
                        const uint32_t k = ent[j][r];
                        if (k && ((k >> 10) & 2047u) == f2[j].bin) atomicAdd(&lh2[j * kB3 + (k & 1023u)], 1u);
                    }
                }
            }
            __syncthreads();
            block_find_multi<NT>(lh2, kB3, kB3, nd, sm, f3);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                tbin[j] = f3[j].bin;
                need[j] = f3[j].rem;
                gt_t[j] = nd[j] - f3[j].rem;
                eq_t[j] = path[j] == kPathList ? lh2[j * kB3 + f3[j].bin] : 0u;
            }
        }
        __syncthreads();                        // lh2 is rewritten below
        // Entries > T and == T in the whole list follow from the finds (bins
        // above b2, then the ranking inside it); those before this chunk's
        // segment (earlier chunks) are counted by list position with ballots.
        // The per-wave sums go to lh2 (free once T is known).
        uint32_t gt_before[2] = {0u, 0u}, eq_before[2] = {0u, 0u};
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] != kPathList) continue;
            T[j] = (b1[j] << 21) | (f2[j].bin << 10) | tbin[j];
            lgt_all[j] = (rem[j] - f2[j].rem) + gt_t[j];
            leq_all[j] = eq_t[j];
        }
        for (int bi = 0; bi < nbat; ++bi) {
            const uint32_t base = (uint32_t)bi * kListBatch;
            bool more = false;                  // entries of earlier chunks left in this batch (uniform)
#pragma unroll
            for (int j = 0; j < NT; ++j) more = more || (path[j] == kPathList && sm[200 + 2 * j] > base);
            if (!more) break;
            reload(bi);
#pragma unroll
            for (int j = 0; j < NT; ++j) {
                if (path[j] != kPathList) continue;
                const uint32_t lo = sm[200 + 2 * j];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    if (r >= rn[j] || base + (uint32_t)(r * kSelThreads) >= lo) break;
                    const uint32_t e = base + (uint32_t)(tid + r * kSelThreads);
                    const uint32_t k = ent[j][r];
                    const bool b = e < lo;
                    gt_before[j] += (uint32_t)__popcll(__ballot(b && k > T[j]));   // padding keys are 0 < T
                    eq_before[j] += (uint32_t)__popcll(__ballot(b && k == T[j]));
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            if (path[j] == kPathList && lane == 0) {
                uint32_t* agg = lh2 + (j * kSelWaves + wave) * 2;
                agg[0] = gt_before[j];
                agg[1] = eq_before[j];
            }
        }
    }

    // ---- per-wave counts of keys > T and == T for every target; targets not
    // resolved from a list then exchange their per-chunk counts
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        uint32_t gt = 0, eq = 0;
        const uint32_t Tj = T[j];
        for_keys([&](uint32_t k, uint32_t, bool v) {
            gt += (uint32_t)__popcll(__ballot(v && k > Tj));
            eq += (uint32_t)__popcll(__ballot(v && k == Tj && k != 0u));
        });
        if (lane == 0) {
            wcnt[(j * kSelWaves + wave) * 2 + 0] = gt;
            wcnt[(j * kSelWaves + wave) * 2 + 1] = eq;
        }
    }
    __syncthreads();
    if (any_other) {
        if (tid < NT && pick<NT>(path[0], path[1], tid) != kPathList) {
            uint32_t gt = 0, eq = 0;
            for (int w = 0; w < kSelWaves; ++w) {
                gt += wcnt[(tid * kSelWaves + w) * 2 + 0];
                eq += wcnt[(tid * kSelWaves + w) * 2 + 1];
            }
            if (multi) {
                st_rlx(&gcnt[(split * 2 + tid) * 2 + 0], gt);
                st_rlx(&gcnt[(split * 2 + tid) * 2 + 1], eq);
            } else {
                cnts[tid * 2 + 0] = gt;
                cnts[tid * 2 + 1] = eq;
            }
        }
        if (multi) {
            row_barrier(ctrl, S, gen, status);
            for (int i = tid; i < S * 2; i += kSelThreads) {
                const int j = i & 1;
                if (j < NT && pick<NT>(path[0], path[1], j) != kPathList) {
                    const uint32_t gt = ld_rlx(&gcnt[i * 2 + 0]), eq = ld_rlx(&gcnt[i * 2 + 1]);
                    cnts[i * 2 + 0] = gt;
                    cnts[i * 2 + 1] = eq;
                }
            }
        }
        __syncthreads();
    }

    // ---- offsets: this chunk's output base and its share of the == T entries.
    // Wave j works out target j with its 64 lanes (lane s: chunk s, lane w:
    // wave w of this chunk), by wave sums and scans in registers.
    uint32_t* wbase = sm + 128;                 // [2][16][base, eq_before]
    uint32_t* tinfo = sm + 192;                 // [2][take_eq, total_sel, eq_chunk, -]
    static_assert(kSelWaves <= kWave, "one lane per wave of the workgroup");
    if (wave < NT) {
        const int j = wave;
        const uint32_t nj = pick<NT>(need[0], need[1], j);
        uint32_t off = 0, total_sel = 0, my_take = 0, my_eq = 0;
        const bool lw = lane < kSelWaves;
        const uint32_t wgt = lw ? wcnt[(j * kSelWaves + lane) * 2 + 0] : 0u;   // this chunk's wave `lane`
        const uint32_t weq = lw ? wcnt[(j * kSelWaves + lane) * 2 + 1] : 0u;
        if (pick<NT>(path[0], path[1], j) == kPathList) {
            // keys above bin b1 per chunk (cnts), plus the list counts by position;
            // ties are taken in chunk order, so only the totals before this
            // chunk and over all chunks matter
            uint32_t ab_before = 0, ab_all = 0;
            for (int s = lane; s < S; s += kWave) {
                const uint32_t a = cnts[(s * 2 + j) * 2 + 0];
                ab_all += a;
                if (s < split) ab_before += a;
            }
            ab_before = wave_sum(ab_before);
            ab_all = wave_sum(ab_all);
            const uint32_t lg_before = wave_sum(lw ? lh2[(j * kSelWaves + lane) * 2 + 0] : 0u);
            const uint32_t le_before = wave_sum(lw ? lh2[(j * kSelWaves + lane) * 2 + 1] : 0u);
            const uint32_t lg_all = pick<NT>(lgt_all[0], lgt_all[1], j);
            const uint32_t le_all = pick<NT>(leq_all[0], leq_all[1], j);
            my_eq = wave_sum(weq);
            off = ab_before + lg_before + (le_before < nj ? le_before : nj);
            my_take = nj > le_before ? nj - le_before : 0u;
            if (my_take > my_eq) my_take = my_eq;
            total_sel = ab_all + lg_all + (le_all < nj ? le_all : nj);
        } else {
            // chunks in order: chunk s takes min(eq_s, nj - (ties in chunks before s)) of its ties
            uint32_t run_eq = 0;
            for (int s0 = 0; s0 < S; s0 += kWave) {
                const int s = s0 + lane;
                const uint32_t gt = s < S ? cnts[(s * 2 + j) * 2 + 0] : 0u;
                const uint32_t eq = s < S ? cnts[(s * 2 + j) * 2 + 1] : 0u;
                const uint32_t inc = wave_incl_scan(eq);
                const uint32_t before = run_eq + inc - eq;
                const uint32_t left = nj > before ? nj - before : 0u;
                const uint32_t take = eq < left ? eq : left;
                const uint32_t sel = gt + take;
                off += wave_sum(s < split ? sel : 0u);
                total_sel += wave_sum(sel);
                if (split >= s0 && split < s0 + kWave) {   // uniform
                    my_take = (uint32_t)__builtin_amdgcn_readlane((int)take, split - s0);
                    my_eq = (uint32_t)__builtin_amdgcn_readlane((int)eq, split - s0);
                }
                run_eq += (uint32_t)__builtin_amdgcn_readlane((int)inc, kWave - 1);
            }
        }
        // wave w of this chunk: base = off + the entries its earlier waves select,
        // where wave w takes min(eq_w, my_take - ties of earlier waves) of its ties
        const uint32_t einc = wave_incl_scan(weq);
        const uint32_t web = einc - weq;
        const uint32_t left = my_take > web ? my_take - web : 0u;
        const uint32_t sel = wgt + (weq < left ? weq : left);
        const uint32_t sinc = wave_incl_scan(sel);
        if (lw) {
            wbase[(j * kSelWaves + lane) * 2 + 0] = off + sinc - sel;
            wbase[(j * kSelWaves + lane) * 2 + 1] = web;
        }
        if (lane == 0) {
            tinfo[j * 4 + 0] = my_take;
            tinfo[j * 4 + 1] = total_sel;
            tinfo[j * 4 + 2] = my_eq;
        }
    }
    __syncthreads();

    // ---- compaction in index order: the selected entries of the wave's keys
    // get consecutive output slots from the wave's base
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const SelTgt& t = j ? t1 : t0;
        const uint32_t Tj = T[j];
        const uint32_t take_eq = tinfo[j * 4 + 0];
        const bool eq_all = take_eq >= tinfo[j * 4 + 2];
        uint32_t run_sel = wbase[(j * kSelWaves + wave) * 2 + 0];
        uint32_t run_eq = wbase[(j * kSelWaves + wave) * 2 + 1];
        int32_t* out_idx = t.idx + row * t.stride;
        float* out_sc = t.score ? t.score + row * t.stride : nullptr;
        // fused attention: this chunk's positions of the last target, in output order, from its first slot
        const bool fa_j = FA && j == NT - 1;
        int32_t* apos = reinterpret_cast<int32_t*>(lh2);
        const uint32_t cbase = wbase[(j * kSelWaves) * 2 + 0];
        // 64 consecutive entries in index order, one per lane (v: the entry exists)
        auto emit = [&](uint32_t k, uint32_t ci, bool v) {
            bool s = v && k > Tj;
            if (eq_all) {
                s = s || (v && k == Tj && k != 0u);
            } else if (take_eq) {               // ties at T split inside this chunk: ranked in index order
                const bool e = v && k == Tj && k != 0u;
                const uint64_t me = __ballot(e);
                s = s || (e && run_eq + lanes_below(me) < take_eq);
                run_eq += (uint32_t)__popcll(me);
            }
            const uint64_t m = __ballot(s);
            const uint32_t slot = run_sel + lanes_below(m);
            if (s && slot < M[j]) {             // the bound holds whenever the counts agree
                const int32_t pos = pos_lds ? (int32_t)posl[ci] : src.position(row, begin + (int64_t)ci);
                out_idx[slot] = pos;
                if (out_sc) out_sc[slot] = key_score(k);
                if (fa_j) apos[slot - cbase] = pos;
            }
            run_sel += (uint32_t)__popcll(m);
        };
        for_keys(emit);
        // the last wave ends at the chunk's last slot: the number of positions it selected
        if (fa_j && wave == kSelWaves - 1 && lane == 0) sm[216] = min(run_sel, M[j]) - cbase;
        if (split == S - 1) {
            for (uint32_t s = tinfo[j * 4 + 1] + tid; s < M[j]; s += kSelThreads) {
                out_idx[s] = -1;
                if (out_sc) out_sc[s] = __uint_as_float(0x7FC00000u);
            }
        }
    }

    // ---- fused attention over this chunk's positions, then the merge
    if constexpr (FA) {
        __syncthreads();                        // positions and count written; the keys' area is free
        const int nsel = (int)sm[216];
        AttnLds<kFuseWaves>& al = *reinterpret_cast<AttnLds<kFuseWaves>*>(lds);
        float* parts_row = af.parts + (size_t)lrow * S * kPartFloats;
        fused_attn_partial(af, row, reinterpret_cast<const int32_t*>(lh2), nsel, al,
                           parts_row + (size_t)split * kPartFloats, !multi);
        if (multi) {
            row_barrier(ctrl, S, gen, status);
            fused_attn_merge<8>(af, row, parts_row, S, split, S, al.mg.f);
        }
    }

    // ---- the last workgroup of the row to leave resets the row's exchange area
    if (multi) {
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = add_rlx(exitc, 1u);
            sm[0] = (old == (uint32_t)S - 1) ? 1u : 0u;
        }
        __syncthreads();
        if (sm[0]) {
            const int nz = any_radix ? kB1 + 2 * kB2 + 2 * kB3 : kB1;
            for (int i = tid; i < nz; i += kSelThreads) st_rlx(&gh1[i], 0u);
            if (tid == 0) {
                st_rlx(ctrl, 0u);
                st_rlx(exitc, 0u);
            }
        }
    }
}

// ------------------------------------------------------------------- host

size_t select_fused_part_bytes(const SelPlan& p) {
    return p.S > 1 ? (size_t)p.rows_per_launch * p.S * kPartFloats * 4 : 0;
}

int plan_select(int64_t rows, int64_t n, int32_t min_chunk, SelPlan* out) {
    DeviceInfo di;
    if (int e = device_info(&di)) return e;
    if (rows < 0 || n < 1 || n >= (int64_t(1) << 31)) return fail(INVALID, "select: n must be in [1, 2^31)");
    int64_t cap = (int64_t)(di.max_lds / 4) - kLdsFixedWords;
    cap = cap / 1024 * 1024;
    if (di.num_cus > kMaxS) return fail(INVALID, "select: more CUs than the kernel's chunk table holds");
    if (cap > kMaxChunk) cap = kMaxChunk;
    if (cap < 1024) return fail(INVALID, "select: device LDS too small");
    const int64_t s_min = (n + cap - 1) / cap;
    const int64_t s_fill = rows > 0 ? (di.num_cus + rows - 1) / rows : 1;
    const int64_t s_fine = n / (min_chunk > 0 ? min_chunk : 1);
    int64_t S = s_fill < s_fine ? s_fill : s_fine;
    if (S < s_min) S = s_min;
    if (S < 1) S = 1;
    int64_t chunk = (n + S - 1) / S;
    chunk = (chunk + 63) / 64 * 64;
    S = (n + chunk - 1) / chunk;
    if (S > di.num_cus) return fail(INVALID, "select: a row needs more workgroups than the device can hold at once");
    SelPlan p;
    p.rows = rows;
    p.n = n;
    p.S = (int32_t)S;
    p.chunk = (int32_t)chunk;
    // rows of one chunk need no co-residency (no row barrier): one launch holds them all
    p.rows_per_launch = S == 1 ? (int32_t)(rows < (int64_t(1) << 24) ? rows : (int64_t(1) << 24)) : (int32_t)(di.num_cus / S);
    if (rows > 0 && p.rows_per_launch > rows) p.rows_per_launch = (int32_t)rows;
    if (p.rows_per_launch < 1) p.rows_per_launch = 1;
    p.launches = rows > 0 ? (int32_t)((rows + p.rows_per_launch - 1) / p.rows_per_launch) : 0;
    p.row_words = S == 1 ? 0 : 4 * (int32_t)S + (int32_t)S * kB1 + 2 * kListCap;
    p.row_words = (p.row_words + 63) / 64 * 64;
    // Workgroup w of a launch runs on XCD w mod 8, and the odd XCDs of this part stream keys 12-25%
    // slower than the even ones (measured per XCD). With S a multiple of 8 every row's chunk s runs on
    // XCD s mod 8, so even chunks take 7.5% more entries and odd ones 7.5% fewer, where LDS and the
    // last chunk leave room (rows of 16 or more chunks: at 8 chunks of 32,768 keys LDS is full).
    int64_t skew = 0;
    if (S >= 16 && S % 8 == 0) {
        skew = chunk * 3 / 40 / 64 * 64;
        if (chunk + skew > cap || n <= (S - 1) * chunk + skew) skew = 0;
    }
    p.skew = (int32_t)skew;
    p.chunk_pad = (int32_t)((chunk + skew + kPadTo - 1) / kPadTo * kPadTo);
    p.lds_bytes = (size_t)(p.chunk_pad + kLdsFixedWords) * 4;
    if (S > 1 && p.rows_per_launch > kSelCtrlRows) return fail(INVALID, "select: too many rows per launch");
    p.data_bytes = (size_t)p.rows_per_launch * p.row_words * 4;
    p.ws_bytes = kCtrlBytes + p.data_bytes;
    *out = p;
    return OK;
}

int64_t plan_select_dense(SelPlan* p) {
    DeviceInfo di;
    // several chunks per row, or keys and positions that fit for the whole chunk: a row holds all n
    if (device_info(&di) != OK || p->S != 1) return p->n;
    if ((size_t)(2 * p->chunk_pad + kLdsFixedWords) * 4 <= di.max_lds) return p->n;
    int64_t cap = ((int64_t)(di.max_lds / 4) - kLdsFixedWords) / 2;
    cap = cap / kPadTo * kPadTo;
    if (cap < kPadTo) return p->chunk;
    p->dense_cap = (int32_t)cap;
    p->lds_bytes = (size_t)(2 * cap + kLdsFixedWords) * 4;
    return cap;
}

namespace {

template <class Src, bool CAN_FA = false>
int launch_rows(const SelPlan& p, const Src& src, const SelOutput* out, int nt, void* ws_ctrl, void* ws_data,
                hipStream_t stream, const int32_t* rowmap = nullptr, const AttnFuse* attn = nullptr) {
    const bool fa = CAN_FA && attn != nullptr;
    const void* fn;
    if constexpr (CAN_FA) {
        fn = fa ? (nt == 2 ? reinterpret_cast<const void*>(&k_select<Src, 2, true>)
                           : reinterpret_cast<const void*>(&k_select<Src, 1, true>))
                : (nt == 2 ? reinterpret_cast<const void*>(&k_select<Src, 2, false>)
                           : reinterpret_cast<const void*>(&k_select<Src, 1, false>));
    } else {
        fn = nt == 2 ? reinterpret_cast<const void*>(&k_select<Src, 2, false>)
                     : reinterpret_cast<const void*>(&k_select<Src, 1, false>);
    }
    const int ki = (nt - 1) + (fa ? 2 : 0);
    static bool attr_set[4] = {false, false, false, false};
    if (!attr_set[ki]) {
        DeviceInfo di;
        if (int e = device_info(&di)) return e;
        hipError_t he = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)di.max_lds);
        if (he != hipSuccess) return hip_fail(he, "hipFuncSetAttribute(select)");
        attr_set[ki] = true;
    }
    if (fa && out[nt - 1].M > kFuseMaxK) return fail(INVALID, "select: fused attention takes at most 4096 positions");
    // Sources whose positions are indirect keep them in LDS next to the keys when both fit.
    DeviceInfo dinfo;
    if (int e = device_info(&dinfo)) return e;
    // A dense capacity below the chunk (one chunk per row, a source that stores its valid entries
    // densely) sizes the key and position areas for that many entries.
    const bool use_dense = Src::kPosLds && p.dense_cap > 0 && p.S == 1 && !fa;
    const int32_t chunk_pad = use_dense && p.dense_cap < p.chunk_pad ? p.dense_cap : p.chunk_pad;
    const bool pos_lds = Src::kPosLds && (size_t)(2 * chunk_pad + kLdsFixedWords) * 4 <= dinfo.max_lds;
    if (chunk_pad < p.chunk_pad && !pos_lds) return fail(INVALID, "select: dense capacity does not fit in LDS");
    const int key_words = fa && chunk_pad < kFuseLdsWords ? kFuseLdsWords : chunk_pad;
    const size_t lds_bytes = (size_t)(pos_lds ? 2 * chunk_pad : key_words) * 4 + (size_t)kLdsFixedWords * 4;
    SelTgt t[2];
    for (int j = 0; j < 2; ++j) {
        const SelOutput& o = out[j < nt ? j : 0];
        t[j] = SelTgt{o.idx, o.score, o.stride, o.M};
    }
    SelDev g;
    g.n = p.n;
    g.S = p.S;
    g.chunk = p.chunk;
    g.skew = p.skew;
    g.chunk_pad = chunk_pad;
    g.pos_lds = pos_lds ? 1 : 0;
    g.nt = nt;
    g.row_words = p.row_words;
    g.ctrl = reinterpret_cast<uint32_t*>(ws_ctrl);
    g.data = reinterpret_cast<uint32_t*>(ws_data);
    g.rowmap = rowmap;
    // The workgroups of a row wait for each other, so every workgroup of a
    // launch must be resident at once. A launch holds at most rows_per_launch
    // * S <= #CUs workgroups; check that the kernel fits one workgroup per CU
    // with this LDS size (the occupancy query accounts for registers too).
    // Kernels on one stream run one after another, so the CUs are free when
    // the launch starts; a wait that still cannot finish gives up after a
    // bounded number of polls and flags the workspace status word.
    static size_t checked_lds[4] = {0, 0, 0, 0};
    if (checked_lds[ki] != lds_bytes) {
        int per_cu = 0;
        hipError_t he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kSelThreads, lds_bytes);
        if (he != hipSuccess) return hip_fail(he, "hipOccupancyMaxActiveBlocksPerMultiprocessor(select)");
        if (per_cu < 1) return fail(INVALID, "select: kernel does not fit on a CU with this LDS size");
        checked_lds[ki] = lds_bytes;
    }
    AttnFuse af{};
    if (fa) af = *attn;
    Src s = src;
    for (int64_t r0 = 0; r0 < p.rows; r0 += p.rows_per_launch) {
        const int64_t nr = (p.rows - r0) < p.rows_per_launch ? (p.rows - r0) : p.rows_per_launch;
        g.row0 = (int32_t)r0;
        void* args[] = {&s, &g, &t[0], &t[1], &af};
        hipError_t he = hipLaunchKernel(fn, dim3((unsigned)(nr * p.S)), dim3(kSelThreads), args,
                                        (unsigned)lds_bytes, stream);
        if (he != hipSuccess) return hip_fail(he, "hipLaunchKernel(select)");
    }
    return OK;
}

template <int KT, int QT, int D>
int run_scan_typed(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* wc,
                   void* wd, hipStream_t stream) {
    if (source == SRC_SCAN) {
        SrcScan<KT, QT, D> s{a.q, a.k, a.N, a.rows_per_seq, a.q_pos};
        return launch_rows<SrcScan<KT, QT, D>, true>(p, s, out, nt, wc, wd, stream, a.rowmap, a.attn);
    }
    if (source == SRC_CAND) {
        if constexpr (D == 64 && KT != kF32 && QT == kBF16) {      // the matrix-core prefill path's inputs
            SrcCand<KT, QT, D> s{a.q, a.k, a.N, a.rows_per_seq, a.cand, a.cnt, a.nranges, a.cap};
            return launch_rows(p, s, out, nt, wc, wd, stream);
        } else {
            return fail(INVALID, "candidate select needs bf16 queries, 64 channels and E4M3 or bf16 keys");
        }
    }
    SrcPool<KT, QT, D> s{a.q, a.k, a.N, a.pool, p.n, a.rows_per_seq};
    return launch_rows(p, s, out, nt, wc, wd, stream);
}

template <int KT, int QT>
int run_scan_d(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* wc,
               void* wd, hipStream_t stream) {
    if (a.d_idx == 64) return run_scan_typed<KT, QT, 64>(p, source, a, out, nt, wc, wd, stream);
    if (a.d_idx == 128) return run_scan_typed<KT, QT, 128>(p, source, a, out, nt, wc, wd, stream);
    return fail(INVALID, "d_idx must be 64 or 128");
}

template <int KT>
int run_scan_q(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* wc,
               void* wd, hipStream_t stream) {
    if (a.q_dtype == kF32) return run_scan_d<KT, kF32>(p, source, a, out, nt, wc, wd, stream);
    if (a.q_dtype == kBF16) return run_scan_d<KT, kBF16>(p, source, a, out, nt, wc, wd, stream);
    return fail(DTYPE, "indexer query dtype must be F32 or BF16");
}

}  // namespace

int run_select(const SelPlan& p, int source, const ScanArgs& scan, const ScoresArgs& sc, const SelOutput* out,
               int nt, void* ws_ctrl, void* ws_data, hipStream_t stream) {
    if (p.rows == 0) return OK;
    if (source == SRC_SCORES) {
        SrcScores s{sc.scores, sc.stride, sc.cand, p.n};
        return launch_rows(p, s, out, nt, ws_ctrl, ws_data, stream);
    }
    switch (scan.k_dtype) {
        case kF32: return run_scan_q<kF32>(p, source, scan, out, nt, ws_ctrl, ws_data, stream);
        case kBF16: return run_scan_q<kBF16>(p, source, scan, out, nt, ws_ctrl, ws_data, stream);
        case kE4M3: return run_scan_q<kE4M3>(p, source, scan, out, nt, ws_ctrl, ws_data, stream);
        default: return fail(DTYPE, "indexer key dtype must be F32, BF16 or E4M3");
    }
}

}  // namespace csa2
