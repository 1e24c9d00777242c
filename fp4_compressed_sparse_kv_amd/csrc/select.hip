// Top-K / top-P selection on gfx950: a multi-workgroup radix select with the
// scores resident in LDS.
//
// Each row (one query's score list) is cut into S chunks; one workgroup of
// 1024 threads owns one chunk and keeps its order-preserving u32 score keys
// in LDS for the whole kernel. The keys come from one of three sources:
//   SrcScores - precomputed fp32 scores in HBM (the standalone top-K call);
//   SrcScan   - indexer keys streamed from HBM and scored in the kernel (a
//               Full layer: scan and select fused, scores never leave LDS);
//   SrcPool   - indexer keys gathered at candidate-pool positions and scored
//               (a Reindex layer).
// The K-th largest key T is found with three radix passes over the LDS keys
// (digits of 11, 11 and 10 bits). Each pass builds a per-chunk histogram with
// LDS atomics, adds it into the row's histogram in the workspace with
// device-scope atomics, waits at a barrier of the row's S workgroups (all
// resident at once: a launch never holds more workgroups than CUs, and the
// kernel fits one per CU) and reads the row total back. Ties at
// T are resolved by position: every chunk publishes its counts of keys > T and
// == T, and chunks take their share of the ==T entries in chunk order. Each
// chunk then compacts its selected entries in position order straight into
// the output, so the output is sorted by position without a sort. Up to two
// targets (pool size P and K) are selected from the same keys in one launch.
//
// The last workgroup of a row to leave zeroes the row's histograms and
// counters, so the workspace is ready for the next launch without a memset.
#include "dot.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kSelThreads = 1024;
constexpr int kSelWaves = kSelThreads / kWave;
constexpr int kB1 = 2048, kB2 = 2048, kB3 = 1024;   // radix digits 11 | 11 | 10 bits
constexpr int kRowHdr = 16;                          // [0] barrier counter, [1] exit counter
constexpr int kRowFixed = kRowHdr + kB1 + 2 * kB2 + 2 * kB3;
constexpr int kWsHeaderWords = 64;                   // [0] device status word
constexpr int kScratchWords = 256;
constexpr int kLdsFixedWords = kB1 + 2 * kB2 + kScratchWords;
constexpr int kMaxChunk = 32768;

struct SelDev {
    int64_t n;
    int32_t S, chunk, row0, nt, row_words;
    uint32_t* ws;
};

struct SelTgt {
    int32_t* idx;
    float* score;
    int64_t stride;
    int32_t M;
};

// ------------------------------------------------------------------ sources

struct SrcScores {
    const float* scores;
    int64_t stride;
    const int32_t* cand;
    int64_t n;

    __device__ __forceinline__ void fill(int64_t row, int64_t begin, int cnt, uint32_t* keys) const {
        const float* p = scores + row * stride + begin;
        for (int i = threadIdx.x; i < cnt; i += kSelThreads) keys[i] = score_key(p[i]);
        __syncthreads();
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

    __device__ __forceinline__ void fill(int64_t row, int64_t begin, int cnt, uint32_t* keys) const {
        using KS = KeySlice<KT, D>;
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
                const double v = quad_sum(s[u].dot(qd));
                if (lq == 0 && i < cnt) keys[i] = (i < lim) ? score_key((float)v) : 0u;
            }
        }
        __syncthreads();
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

    __device__ __forceinline__ void fill(int64_t row, int64_t begin, int cnt, uint32_t* keys) const {
        using KS = KeySlice<KT, D>;
        constexpr int QB = (QT == kBF16) ? 2 : 4;
        constexpr int U = KS::RAW >= 4 ? 1 : 4 / KS::RAW;
        const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
        double qd[D / 4];
        load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
        const uint8_t* kb = k + row * N * (int64_t)KS::ROW_BYTES;
        const int32_t* pr = pool + row * P + begin;
        for (int base = 0; base < cnt; base += (kSelThreads / 4) * U) {
            KS s[U];
            bool ok[U];
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * (kSelThreads / 4) + quad;
                const int32_t pos = (i < cnt) ? pr[i] : -1;
                ok[u] = pos >= 0 && (int64_t)pos < N;
                if (ok[u]) s[u].load(kb + (int64_t)pos * KS::ROW_BYTES, lq);
                else for (int j = 0; j < KS::RAW; ++j) s[u].raw[j] = make_uint4(0, 0, 0, 0);
            }
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int i = base + u * (kSelThreads / 4) + quad;
                const double v = quad_sum(s[u].dot(qd));
                if (lq == 0 && i < cnt) keys[i] = ok[u] ? score_key((float)v) : 0u;
            }
        }
        __syncthreads();
    }
    __device__ __forceinline__ int32_t position(int64_t row, int64_t i) const { return pool[row * P + i]; }
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

__device__ __forceinline__ void push_hist(const uint32_t* lh, uint32_t* gh, int nb) {
    for (int b = threadIdx.x; b < nb; b += kSelThreads) {
        const uint32_t c = lh[b];
        if (c) add_rlx(&gh[b], c);
    }
}

__device__ __forceinline__ void pull_hist(uint32_t* lh, const uint32_t* gh, int nb) {
    for (int b = threadIdx.x; b < nb; b += kSelThreads) lh[b] = ld_rlx(&gh[b]);
    __syncthreads();
}

// ------------------------------------------------------------------ kernel

template <class Src>
__global__ void __launch_bounds__(kSelThreads) k_select(Src src, SelDev g, SelTgt t0, SelTgt t1) {
    extern __shared__ uint32_t lds[];
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int lrow = blockIdx.x / g.S;
    const int split = blockIdx.x - lrow * g.S;
    const int64_t row = (int64_t)g.row0 + lrow;
    const int64_t begin = (int64_t)split * g.chunk;
    const int cnt = (int)min((int64_t)g.chunk, g.n - begin);
    const int nt = g.nt;
    const bool multi = g.S > 1;

    uint32_t* keys = lds;
    uint32_t* lh1 = lds + g.chunk;
    uint32_t* lh2 = lh1 + kB1;                 // [2][kB2]; pass 3 reuses it as [2][kB3]
    uint32_t* sm = lh2 + 2 * kB2;
    uint32_t* status = g.ws;
    uint32_t* rw = g.ws + kWsHeaderWords + (size_t)lrow * g.row_words;
    uint32_t* ctrl = rw;
    uint32_t* exitc = rw + 1;
    uint32_t* gh1 = rw + kRowHdr;
    uint32_t* gh2 = gh1 + kB1;
    uint32_t* gh3 = gh2 + 2 * kB2;
    uint32_t* gcnt = gh3 + 2 * kB3;             // [S][2 targets][gt, eq]
    uint32_t gen = 0;

    const uint32_t M[2] = {(uint32_t)t0.M, (uint32_t)t1.M};

    for (int i = tid; i < kB1 + 2 * kB2; i += kSelThreads) lh1[i] = 0u;
    src.fill(row, begin, cnt, keys);            // ends with a block barrier

    // ---- pass 1: bits 31..21
    for (int i = tid; i < cnt; i += kSelThreads) {
        const uint32_t k = keys[i];
        if (k) atomicAdd(&lh1[k >> 21], 1u);
    }
    __syncthreads();
    if (multi) {
        push_hist(lh1, gh1, kB1);
        row_barrier(ctrl, g.S, gen, status);
        pull_hist(lh1, gh1, kB1);
    }
    bool all[2] = {true, true};
    uint32_t b1[2] = {0, 0}, rem[2] = {0, 0}, T[2] = {0, 0}, need[2] = {0, 0};
    for (int j = 0; j < nt; ++j) {
        const Found f = block_find(lh1, kB1, M[j], sm);
        all[j] = f.total <= M[j];
        b1[j] = f.bin;
        rem[j] = f.rem;
    }
    const bool any_pass = !all[0] || (nt > 1 && !all[1]);
    if (any_pass) {
        // ---- pass 2: bits 20..10 within the chosen top digit
        for (int i = tid; i < cnt; i += kSelThreads) {
            const uint32_t k = keys[i];
            for (int j = 0; j < nt; ++j)
                if (!all[j] && (k >> 21) == b1[j]) atomicAdd(&lh2[j * kB2 + ((k >> 10) & 2047u)], 1u);
        }
        __syncthreads();
        if (multi) {
            for (int j = 0; j < nt; ++j)
                if (!all[j]) push_hist(lh2 + j * kB2, gh2 + j * kB2, kB2);
            row_barrier(ctrl, g.S, gen, status);
            for (int j = 0; j < nt; ++j)
                if (!all[j]) pull_hist(lh2 + j * kB2, gh2 + j * kB2, kB2);
        }
        uint32_t pre2[2] = {0, 0};
        for (int j = 0; j < nt; ++j) {
            if (all[j]) continue;
            const Found f = block_find(lh2 + j * kB2, kB2, rem[j], sm);
            pre2[j] = (b1[j] << 11) | f.bin;
            rem[j] = f.rem;
        }
        // ---- pass 3: bits 9..0 within the chosen 22-bit prefix
        for (int i = tid; i < 2 * kB2; i += kSelThreads) lh2[i] = 0u;
        __syncthreads();
        for (int i = tid; i < cnt; i += kSelThreads) {
            const uint32_t k = keys[i];
            for (int j = 0; j < nt; ++j)
                if (!all[j] && (k >> 10) == pre2[j]) atomicAdd(&lh2[j * kB3 + (k & 1023u)], 1u);
        }
        __syncthreads();
        if (multi) {
            for (int j = 0; j < nt; ++j)
                if (!all[j]) push_hist(lh2 + j * kB3, gh3 + j * kB3, kB3);
            row_barrier(ctrl, g.S, gen, status);
            for (int j = 0; j < nt; ++j)
                if (!all[j]) pull_hist(lh2 + j * kB3, gh3 + j * kB3, kB3);
        }
        for (int j = 0; j < nt; ++j) {
            if (all[j]) continue;
            const Found f = block_find(lh2 + j * kB3, kB3, rem[j], sm);
            T[j] = (pre2[j] << 10) | f.bin;
            need[j] = f.rem;                   // entries equal to T that are taken, row-wide
        }
    }

    // ---- counts of > T and == T per wave (each wave owns a contiguous span)
    int span = (cnt + kSelWaves - 1) / kSelWaves;
    span = (span + kWave - 1) & ~(kWave - 1);
    const int w0 = min(cnt, wave * span), w1 = min(cnt, w0 + span);
    uint32_t* wcnt = sm + 32;                   // [2][16][gt, eq]
    for (int j = 0; j < nt; ++j) {
        uint32_t gt = 0, eq = 0;
        for (int i = w0 + lane; i < w1; i += kWave) {
            const uint32_t k = keys[i];
            gt += k > T[j];
            eq += (k == T[j]) && k != 0u;
        }
        gt = wave_sum(gt);
        eq = wave_sum(eq);
        if (lane == 0) {
            wcnt[(j * kSelWaves + wave) * 2 + 0] = gt;
            wcnt[(j * kSelWaves + wave) * 2 + 1] = eq;
        }
    }
    __syncthreads();
    if (tid < nt) {
        uint32_t gt = 0, eq = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            gt += wcnt[(tid * kSelWaves + w) * 2 + 0];
            eq += wcnt[(tid * kSelWaves + w) * 2 + 1];
        }
        if (multi) {
            st_rlx(&gcnt[(split * 2 + tid) * 2 + 0], gt);
            st_rlx(&gcnt[(split * 2 + tid) * 2 + 1], eq);
        }
        sm[16 + tid * 2 + 0] = gt;
        sm[16 + tid * 2 + 1] = eq;
    }
    if (multi) row_barrier(ctrl, g.S, gen, status);
    else __syncthreads();

    // ---- offsets: this chunk's output base and its share of the == T entries.
    // The counts of all chunks are staged in LDS by one lane each (the pass-2/3
    // histogram space is free now), so no lane walks them with serial loads.
    uint32_t* cnts = lh2;                       // [S][2 targets][gt, eq]
    if (multi) {
        for (int i = tid; i < g.S * 4; i += kSelThreads) cnts[i] = ld_rlx(&gcnt[i]);
    } else if (tid < 4) {
        cnts[tid] = sm[16 + tid];
    }
    __syncthreads();
    uint32_t* wbase = sm + 128;                 // [2][16][base, eq_before]
    uint32_t* tinfo = sm + 192;                 // [2][take_eq, total_sel]
    if (tid < nt) {
        const int j = tid;
        uint32_t off = 0, eq_before = 0, total_sel = 0, my_take = 0;
        for (int s = 0; s < g.S; ++s) {
            const uint32_t gt = cnts[(s * 2 + j) * 2 + 0], eq = cnts[(s * 2 + j) * 2 + 1];
            const uint32_t left = need[j] > eq_before ? need[j] - eq_before : 0u;
            const uint32_t take = eq < left ? eq : left;
            if (s < split) off += gt + take;
            if (s == split) my_take = take;
            total_sel += gt + take;
            eq_before += eq;
        }
        uint32_t wb = off, web = 0;
        for (int w = 0; w < kSelWaves; ++w) {
            const uint32_t gt = wcnt[(j * kSelWaves + w) * 2 + 0], eq = wcnt[(j * kSelWaves + w) * 2 + 1];
            const uint32_t left = my_take > web ? my_take - web : 0u;
            wbase[(j * kSelWaves + w) * 2 + 0] = wb;
            wbase[(j * kSelWaves + w) * 2 + 1] = web;
            wb += gt + (eq < left ? eq : left);
            web += eq;
        }
        tinfo[j * 2 + 0] = my_take;
        tinfo[j * 2 + 1] = total_sel;
    }
    __syncthreads();

    // ---- compaction in position order
    const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (kWave - lane));
    for (int j = 0; j < nt; ++j) {
        const SelTgt& t = j ? t1 : t0;
        const uint32_t take_eq = tinfo[j * 2 + 0];
        uint32_t run_sel = wbase[(j * kSelWaves + wave) * 2 + 0];
        uint32_t run_eq = wbase[(j * kSelWaves + wave) * 2 + 1];
        int32_t* out_idx = t.idx + row * t.stride;
        float* out_sc = t.score ? t.score + row * t.stride : nullptr;
        for (int i0 = w0; i0 < w1; i0 += kWave) {
            const int i = i0 + lane;
            const uint32_t k = (i < w1) ? keys[i] : 0u;
            const bool is_eq = (i < w1) && k == T[j] && k != 0u;
            const uint64_t m_eq = __ballot(is_eq);
            const uint32_t r_eq = run_eq + (uint32_t)__popcll(m_eq & lt_mask);
            const bool sel = (i < w1) && (k > T[j] || (is_eq && r_eq < take_eq));
            const uint64_t m_sel = __ballot(sel);
            const uint32_t slot = run_sel + (uint32_t)__popcll(m_sel & lt_mask);
            if (sel && slot < M[j]) {                   // the bound holds whenever the counts agree
                out_idx[slot] = src.position(row, begin + i);
                if (out_sc) out_sc[slot] = key_score(k);
            }
            run_eq += (uint32_t)__popcll(m_eq);
            run_sel += (uint32_t)__popcll(m_sel);
        }
        if (split == g.S - 1) {
            for (uint32_t s = tinfo[j * 2 + 1] + tid; s < M[j]; s += kSelThreads) {
                out_idx[s] = -1;
                if (out_sc) out_sc[s] = __uint_as_float(0x7FC00000u);
            }
        }
    }

    // ---- the last workgroup of the row to leave resets the row's exchange area
    if (multi) {
        __syncthreads();
        if (tid == 0) {
            const uint32_t old = add_rlx(exitc, 1u);
            sm[0] = (old == (uint32_t)g.S - 1) ? 1u : 0u;
        }
        __syncthreads();
        if (sm[0]) {
            for (int i = tid; i < kB1 + 2 * kB2 + 2 * kB3; i += kSelThreads) st_rlx(&gh1[i], 0u);
            if (tid == 0) {
                st_rlx(ctrl, 0u);
                st_rlx(exitc, 0u);
            }
        }
    }
}

// ------------------------------------------------------------------- host

int plan_select(int64_t rows, int64_t n, int32_t min_chunk, SelPlan* out) {
    DeviceInfo di;
    if (int e = device_info(&di)) return e;
    if (rows < 0 || n < 1 || n >= (int64_t(1) << 31)) return fail(INVALID, "select: n must be in [1, 2^31)");
    int64_t cap = (int64_t)(di.max_lds / 4) - kLdsFixedWords;
    cap = cap / 1024 * 1024;
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
    p.rows_per_launch = (int32_t)(di.num_cus / S);
    if (rows > 0 && p.rows_per_launch > rows) p.rows_per_launch = (int32_t)rows;
    if (p.rows_per_launch < 1) p.rows_per_launch = 1;
    p.launches = rows > 0 ? (int32_t)((rows + p.rows_per_launch - 1) / p.rows_per_launch) : 0;
    p.row_words = kRowFixed + 4 * (int32_t)S;
    p.row_words = (p.row_words + 63) / 64 * 64;
    p.lds_bytes = (size_t)(chunk + kLdsFixedWords) * 4;
    p.ws_bytes = (size_t)(kWsHeaderWords + (size_t)p.rows_per_launch * p.row_words) * 4;
    *out = p;
    return OK;
}

namespace {

template <class Src>
int launch_rows(const SelPlan& p, const Src& src, const SelOutput* out, int nt, void* ws, hipStream_t stream) {
    auto fn = reinterpret_cast<const void*>(&k_select<Src>);
    static bool attr_set = false;
    if (!attr_set) {
        DeviceInfo di;
        if (int e = device_info(&di)) return e;
        hipError_t he = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)di.max_lds);
        if (he != hipSuccess) return hip_fail(he, "hipFuncSetAttribute(select)");
        attr_set = true;
    }
    SelTgt t[2];
    for (int j = 0; j < 2; ++j) {
        const SelOutput& o = out[j < nt ? j : 0];
        t[j] = SelTgt{o.idx, o.score, o.stride, o.M};
    }
    SelDev g;
    g.n = p.n;
    g.S = p.S;
    g.chunk = p.chunk;
    g.nt = nt;
    g.row_words = p.row_words;
    g.ws = reinterpret_cast<uint32_t*>(ws);
    // The workgroups of a row wait for each other, so every workgroup of a
    // launch must be resident at once. A launch holds at most rows_per_launch
    // * S <= #CUs workgroups; check that the kernel fits one workgroup per CU
    // with this LDS size (the occupancy query accounts for registers too).
    // Kernels on one stream run one after another, so the CUs are free when
    // the launch starts; a wait that still cannot finish gives up after a
    // bounded number of polls and flags the workspace status word.
    static size_t checked_lds = 0;
    if (checked_lds != p.lds_bytes) {
        int per_cu = 0;
        hipError_t he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kSelThreads, p.lds_bytes);
        if (he != hipSuccess) return hip_fail(he, "hipOccupancyMaxActiveBlocksPerMultiprocessor(select)");
        if (per_cu < 1) return fail(INVALID, "select: kernel does not fit on a CU with this LDS size");
        checked_lds = p.lds_bytes;
    }
    Src s = src;
    for (int64_t r0 = 0; r0 < p.rows; r0 += p.rows_per_launch) {
        const int64_t nr = (p.rows - r0) < p.rows_per_launch ? (p.rows - r0) : p.rows_per_launch;
        g.row0 = (int32_t)r0;
        void* args[] = {&s, &g, &t[0], &t[1]};
        hipError_t he = hipLaunchKernel(fn, dim3((unsigned)(nr * p.S)), dim3(kSelThreads), args,
                                        (unsigned)p.lds_bytes, stream);
        if (he != hipSuccess) return hip_fail(he, "hipLaunchKernel(select)");
    }
    return OK;
}

template <int KT, int QT, int D>
int run_scan_typed(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* ws,
                   hipStream_t stream) {
    if (source == SRC_SCAN) {
        SrcScan<KT, QT, D> s{a.q, a.k, a.N, a.rows_per_seq, a.q_pos};
        return launch_rows(p, s, out, nt, ws, stream);
    }
    SrcPool<KT, QT, D> s{a.q, a.k, a.N, a.pool, p.n};
    return launch_rows(p, s, out, nt, ws, stream);
}

template <int KT, int QT>
int run_scan_d(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* ws,
               hipStream_t stream) {
    if (a.d_idx == 64) return run_scan_typed<KT, QT, 64>(p, source, a, out, nt, ws, stream);
    if (a.d_idx == 128) return run_scan_typed<KT, QT, 128>(p, source, a, out, nt, ws, stream);
    return fail(INVALID, "d_idx must be 64 or 128");
}

template <int KT>
int run_scan_q(const SelPlan& p, int source, const ScanArgs& a, const SelOutput* out, int nt, void* ws,
               hipStream_t stream) {
    if (a.q_dtype == kF32) return run_scan_d<KT, kF32>(p, source, a, out, nt, ws, stream);
    if (a.q_dtype == kBF16) return run_scan_d<KT, kBF16>(p, source, a, out, nt, ws, stream);
    return fail(DTYPE, "indexer query dtype must be F32 or BF16");
}

}  // namespace

int run_select(const SelPlan& p, int source, const ScanArgs& scan, const ScoresArgs& sc, const SelOutput* out,
               int nt, void* ws, hipStream_t stream) {
    if (p.rows == 0) return OK;
    if (source == SRC_SCORES) {
        SrcScores s{sc.scores, sc.stride, sc.cand, p.n};
        return launch_rows(p, s, out, nt, ws, stream);
    }
    switch (scan.k_dtype) {
        case kF32: return run_scan_q<kF32>(p, source, scan, out, nt, ws, stream);
        case kBF16: return run_scan_q<kBF16>(p, source, scan, out, nt, ws, stream);
        case kE4M3: return run_scan_q<kE4M3>(p, source, scan, out, nt, ws, stream);
        default: return fail(DTYPE, "indexer key dtype must be F32, BF16 or E4M3");
    }
}

}  // namespace csa2
