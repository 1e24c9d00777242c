// Reindex-layer selection: score a row's candidate pool with the layer's own
// indexer query and take the exact top-K of the pool with one exchange.
//
// Each row's pool (at most 16,384 positions, ascending) is cut into S chunks
// of at most 1024 entries, one 1024-thread workgroup per chunk, all chunks of
// a row resident together. A workgroup
//   1. gathers the indexer keys of its chunk's pool positions (four lanes per
//      64-channel key row, 16-byte loads), computes the exact scores (fp64
//      products and sums, rounded once to fp32), turns them into
//      order-preserving u32 keys and publishes them to the row's key buffer
//      with device-coherent stores;
//   2. waits at the row barrier, then loads the whole row's keys (16-byte
//      coherent loads; thread t holds entries t*NK .. t*NK + NK - 1);
//   3. finds the exact threshold key T (the K-th largest key, or the smallest
//      valid one when the row has fewer than K) by radix passes of 11, 11 and
//      10 bits over LDS histograms - the third only when the bin found by the
//      second holds more than one key; every workgroup of the row computes
//      the same T from the same keys;
//   4. writes the positions of its own chunk's selected entries straight to
//      their output slots: an entry is selected if its key is above T, or
//      equal to T and among the first (K - #above T) such entries in pool
//      order; its slot is the number of selected entries before it, from one
//      block scan of per-thread counts. Pool order is position order, so the
//      output is ascending. Slots past the number selected hold -1.
//   5. (with the attention fused in) attends to its own selected positions,
//      which it keeps in LDS in output order, publishes its partial softmax
//      state, and after a second row barrier writes the output of heads
//      split, split + S, ... as the merge of the row's S states in slice
//      order - so the layer's attention needs no launch, position read-back
//      or merge of its own.
// NaN and -inf scores map to key 0 and are never selected; -0 ranks as +0.
// Ties at T go to the lowest pool entry, which is the lowest position.
#include <type_traits>

#include "attn_core.hpp"
#include "dot.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kPsThreads = 1024;
constexpr int kPsWaves = kPsThreads / kWave;
constexpr int kPsChunk = kPsThreads;            // pool entries per workgroup (4 per lane quad)
constexpr int kPsMaxN = (int)kPoolSelMaxN;      // pool entries per row (16 per thread)

struct PsDev {
    int32_t n, n4, S, K, row0;                  // n4: n rounded up to a multiple of 4 (key buffer row stride)
    uint32_t* ctrl;                             // workspace control region
    uint32_t* keys;                             // [rows of the launch][n4] published keys
};

struct PsLds {
    uint32_t hist[2048];
    uint32_t pos[kPsChunk];                     // positions of this chunk's entries
    uint32_t wsum[kPsWaves];
    uint32_t sh[4];
};

// Exclusive scan of v over the workgroup in thread order; `total` gets the sum.
__device__ __forceinline__ uint32_t ps_block_scan(uint32_t v, uint32_t* wsum, uint32_t& total) {
    const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(v);
    if (lane == kWave - 1) wsum[wave] = inc;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kPsWaves; ++w) {
        const uint32_t s = wsum[w];
        before += (w < wave) ? s : 0u;
        tot += s;
    }
    total = tot;
    __syncthreads();                            // wsum may be rewritten after this
    return before + inc - v;
}

// Bins h[NB-1] (highest) down to h[0]: the bin holding the M-th largest key,
// M = min(M_req, total). Every thread gets (bin, keys in higher bins, keys in
// the bin, M); M == 0 when the histogram is empty.
template <int NB>
__device__ __forceinline__ void ps_find(const uint32_t* h, uint32_t M_req, PsLds& L, uint32_t& bin, uint32_t& above,
                                        uint32_t& in_bin, uint32_t& M) {
    static_assert(NB == 2 * kPsThreads || NB == kPsThreads, "bins per thread");
    const int tid = threadIdx.x;
    const int hi = NB - 1 - (NB == 2 * kPsThreads ? 2 * tid : tid);
    const uint32_t a = h[hi];
    const uint32_t b = (NB == 2 * kPsThreads) ? h[hi - 1] : 0u;
    uint32_t tot;
    const uint32_t before = ps_block_scan(a + b, L.wsum, tot);
    const uint32_t m = M_req < tot ? M_req : tot;
    if (before < m && m <= before + a + b) {
        const bool in_hi = before + a >= m;
        L.sh[0] = in_hi ? (uint32_t)hi : (uint32_t)(hi - 1);
        L.sh[1] = in_hi ? before : before + a;
        L.sh[2] = in_hi ? a : b;
    }
    __syncthreads();
    bin = L.sh[0];
    above = L.sh[1];
    in_bin = L.sh[2];
    M = m;
}

// LDS of the fused attention: its positions (this chunk's selected entries in
// output order) and the waves' staging and merge areas.
struct alignas(16) PsAttnLds {
    AttnLds<kFuseWaves> a;
    int32_t apos[kPsChunk];
    uint32_t span[2];                           // this chunk's output slots [span[0], span[1])
};

template <int KT, int QT, int D, int NK, bool FA>
__global__ void __launch_bounds__(kPsThreads) k_pool_select(const void* __restrict__ q, const uint8_t* __restrict__ k,
                                                            int64_t N, const int32_t* __restrict__ pool, PsDev g,
                                                            int32_t* __restrict__ idx_out, int64_t idx_stride,
                                                            float* __restrict__ sc_out, AttnFuse af) {
    using KS = KeySlice<KT, D, QT>;
    constexpr int QB = (QT == kBF16) ? 2 : 4;
    __shared__ PsLds L;
    __shared__ typename std::conditional<FA, PsAttnLds, char>::type FL;
    const int tid = threadIdx.x;
    const int S = g.S, n = g.n;
    const int lrow = blockIdx.x / S;
    const int split = blockIdx.x - lrow * S;
    const int64_t row = (int64_t)g.row0 + lrow;
    const int begin = split * kPsChunk;
    const int cnt = min(kPsChunk, n - begin);
    uint32_t* status = g.ctrl;
    uint32_t* rc = g.ctrl + kSelCtrlOffsetWords + (size_t)lrow * kSelCtrlRowWords;   // zero between calls
    uint32_t* bar = rc;
    uint32_t* exitc = rc + 1;
    uint32_t* rkeys = g.keys + (size_t)lrow * g.n4;

    for (int i = tid; i < 2048; i += kPsThreads) L.hist[i] = 0u;

    // ---- 1. score this chunk: quad `quad` holds entries u*256 + quad (u = 0..3);
    // after the transposed reduction lane lq owns entry lq*256 + quad
    {
        const int quad = tid >> 2, lq = tid & 3;
        double qd[D / 4];
        load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
        const uint8_t* kb = k + row * N * (int64_t)KS::ROW_BYTES;
        const int32_t* pr = pool + row * (int64_t)n + begin;
        int32_t pv[4];
        bool ok[4];
        KS s[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int i = u * (kPsThreads / 4) + quad;
            pv[u] = (i < cnt) ? pr[i] : -1;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            ok[u] = pv[u] >= 0 && (int64_t)pv[u] < N;
            // padding entries read key row 0 and are discarded
            s[u].load(kb + (int64_t)(ok[u] ? pv[u] : 0) * KS::ROW_BYTES, lq);
        }
        typename KS::Part acc[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) acc[u] = s[u].dot(qd);
        const auto v = quad_transpose_sum(acc, lq);
        const int i = lq * (kPsThreads / 4) + quad;
        const bool okl = lq == 0 ? ok[0] : lq == 1 ? ok[1] : lq == 2 ? ok[2] : ok[3];
        const int32_t pvl = lq == 0 ? pv[0] : lq == 1 ? pv[1] : lq == 2 ? pv[2] : pv[3];
        if (i < cnt) {
            const __amdgpu_buffer_rsrc_t ws = __builtin_amdgcn_make_buffer_rsrc(rkeys, (short)0, g.n4 * 4, kRsrcWord3);
            __builtin_amdgcn_raw_buffer_store_b32(okl ? score_key(round_score(v)) : 0u, ws, (begin + i) * 4, 0, kCoherent);
            L.pos[i] = (uint32_t)pvl;
        }
    }

    // ---- 2. exchange: every chunk's keys, then the whole row in registers
    uint32_t gen = 0;
    if (S > 1) row_barrier(bar, (uint32_t)S, gen, status);
    else {
        wave_drain();
        __syncthreads();
    }
    uint32_t kv[NK];
    {
        // whole 16-byte words inside the row's n4 entries; past n4 the loads
        // return 0, and entries n .. n4-1 (never written) are cleared here
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(rkeys, (short)0, g.n4 * 4, kRsrcWord3);
#pragma unroll
        for (int j = 0; j < NK / 4; ++j) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid * NK + 4 * j) * 4, 0, kCoherent);
            kv[4 * j + 0] = w.x;
            kv[4 * j + 1] = w.y;
            kv[4 * j + 2] = w.z;
            kv[4 * j + 3] = w.w;
        }
#pragma unroll
        for (int j = 0; j < NK; ++j)
            if (tid * NK + j >= n) kv[j] = 0u;
    }
    if (S > 1 && !FA) {                         // the last workgroup past the barrier resets the row's words
        if (tid == 0 && add_rlx(exitc, 1u) == (uint32_t)S - 1) {
            st_rlx(exitc, 0u);
            st_rlx(bar, 0u);
        }
    }

    // ---- 3. threshold T by three radix passes (bits 31..21, 20..10, 9..0)
#pragma unroll
    for (int j = 0; j < NK; ++j)
        if (kv[j]) atomicAdd(&L.hist[kv[j] >> 21], 1u);
    __syncthreads();
    uint32_t b1, a1, c1, M;
    ps_find<2048>(L.hist, (uint32_t)g.K, L, b1, a1, c1, M);
    uint32_t T = 0u, gt = 0u, need = 0u;
    if (M > 0) {
        for (int i = tid; i < 2048; i += kPsThreads) L.hist[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int j = 0; j < NK; ++j)
            if (kv[j] && (kv[j] >> 21) == b1) atomicAdd(&L.hist[(kv[j] >> 10) & 2047u], 1u);
        __syncthreads();
        uint32_t b2, a2, c2, m2;
        ps_find<2048>(L.hist, M - a1, L, b2, a2, c2, m2);
        const uint32_t p21 = (b1 << 11) | b2;
        if (c2 == 1u) {
            // a single key with these 22 leading bits: it is T, and it is taken
#pragma unroll
            for (int j = 0; j < NK; ++j)
                if (kv[j] && (kv[j] >> 10) == p21) L.sh[3] = kv[j];
            __syncthreads();
            T = L.sh[3];
            gt = a1 + a2;
        } else {
            for (int i = tid; i < 1024; i += kPsThreads) L.hist[i] = 0u;
            __syncthreads();
#pragma unroll
            for (int j = 0; j < NK; ++j)
                if (kv[j] && (kv[j] >> 10) == p21) atomicAdd(&L.hist[kv[j] & 1023u], 1u);
            __syncthreads();
            uint32_t b3, a3, c3, m3;
            ps_find<1024>(L.hist, M - a1 - a2, L, b3, a3, c3, m3);
            T = (p21 << 10) | b3;
            gt = a1 + a2 + a3;
        }
        need = M - gt;                          // >= 1 keys equal to T are taken
    }

    // ---- 4. compaction of this chunk's entries in pool order
    int32_t* orow = idx_out + row * idx_stride;
    float* srow = sc_out ? sc_out + row * idx_stride : nullptr;
    if (M > 0) {
        uint32_t c_gt = 0, c_eq = 0;
#pragma unroll
        for (int j = 0; j < NK; ++j) {
            c_gt += kv[j] > T ? 1u : 0u;
            c_eq += kv[j] == T ? 1u : 0u;
        }
        uint32_t tot;
        const uint32_t before = ps_block_scan((c_gt << 16) | c_eq, L.wsum, tot);   // both < 2^15
        uint32_t bgt = before >> 16, beq = before & 0xFFFFu;
        if constexpr (FA) {
            // output slots of this chunk: the entries selected before its first entry and
            // before the next chunk's (chunk starts are multiples of NK: a thread's first entry)
            const uint32_t sel_before = bgt + (beq < need ? beq : need);
            if (tid * NK == begin) FL.span[0] = sel_before;
            if (split == S - 1) {
                if (tid == 0) FL.span[1] = M;
            } else if (tid * NK == begin + kPsChunk) {
                FL.span[1] = sel_before;
            }
            __syncthreads();
        }
        const int e0 = tid * NK;
        if (e0 < begin + cnt && e0 + NK > begin) {
#pragma unroll
            for (int j = 0; j < NK; ++j) {
                const int e = e0 + j;
                const bool take = kv[j] > T || (kv[j] == T && beq < need);
                if (take && e >= begin && e < begin + cnt) {
                    const uint32_t slot = bgt + (beq < need ? beq : need);
                    orow[slot] = (int32_t)L.pos[e - begin];
                    if (srow) srow[slot] = key_score(kv[j]);
                    if constexpr (FA) FL.apos[slot - FL.span[0]] = (int32_t)L.pos[e - begin];
                }
                bgt += kv[j] > T ? 1u : 0u;
                beq += kv[j] == T ? 1u : 0u;
            }
        }
    }
    if (split == S - 1) {
        for (int s = (int)M + tid; s < g.K; s += kPsThreads) {
            orow[s] = -1;
            if (srow) srow[s] = __uint_as_float(0x7FC00000u);
        }
    }
    if constexpr (FA) {
        // ---- 5. this chunk's share of the row's attention, then the merge
        __syncthreads();                        // the positions are in LDS
        const int nsel = M > 0 ? (int)(FL.span[1] - FL.span[0]) : 0;
        float* parts_row = af.parts + (size_t)lrow * S * kPartFloats;
        fused_attn_partial(af, row, FL.apos, nsel, FL.a, parts_row + (size_t)split * kPartFloats);
        if (S > 1) row_barrier(bar, (uint32_t)S, gen, status);
        else __syncthreads();
        fused_attn_merge<NK>(af, row, parts_row, S, split, S, FL.a.mg.f);   // S <= NK: n <= NK * kPsChunk
        if (S > 1 && tid == 0 && add_rlx(exitc, 1u) == (uint32_t)S - 1) {   // every chunk is past both barriers
            st_rlx(exitc, 0u);
            st_rlx(bar, 0u);
        }
    }
}

// ------------------------------------------------------------------- host

int plan_pool_select(int64_t rows, int64_t n, PoolSelPlan* out) {
    if (rows < 0 || n < 1 || n > kPsMaxN) return fail(INVALID, "pool select: n must be in [1, 16384]");
    DeviceInfo di;
    if (int e = device_info(&di)) return e;
    PoolSelPlan p;
    p.rows = rows;
    p.n = (int32_t)n;
    p.S = (int32_t)((n + kPsChunk - 1) / kPsChunk);
    // all chunks of a launch's rows are resident together: one workgroup per CU
    // is always possible, so rows_per_launch * S <= #CUs
    p.rows_per_launch = di.num_cus / p.S;
    if (p.rows_per_launch > kSelCtrlRows) p.rows_per_launch = kSelCtrlRows;
    if (rows > 0 && p.rows_per_launch > rows) p.rows_per_launch = (int32_t)rows;
    if (p.rows_per_launch < 1) return fail(INVALID, "pool select: a row needs more workgroups than the device holds");
    p.n4 = (int32_t)((n + 3) / 4 * 4);
    p.data_bytes = (size_t)p.rows_per_launch * (size_t)p.n4 * 4;
    *out = p;
    return OK;
}

namespace {

template <int KT, int QT, int D>
int launch_ps_typed(const PoolSelPlan& p, const PoolSelArgs& a, void* ws_ctrl, void* ws_data, hipStream_t stream) {
    const bool fa = a.attn != nullptr;
    auto fn = p.n <= 8 * kPsThreads ? (fa ? k_pool_select<KT, QT, D, 8, true> : k_pool_select<KT, QT, D, 8, false>)
                                    : (fa ? k_pool_select<KT, QT, D, 16, true> : k_pool_select<KT, QT, D, 16, false>);
    // the chunks of a row wait for each other: check once that a workgroup fits on a CU
    static bool fits[4] = {false, false, false, false};
    const int which = (p.n <= 8 * kPsThreads ? 0 : 1) + (fa ? 2 : 0);
    if (!fits[which]) {
        int per_cu = 0;
        const hipError_t he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kPsThreads, 0);
        if (he != hipSuccess) return hip_fail(he, "hipOccupancyMaxActiveBlocksPerMultiprocessor(pool select)");
        if (per_cu < 1) return fail(INVALID, "pool select: kernel does not fit on a CU");
        fits[which] = true;
    }
    PsDev g;
    g.n = p.n;
    g.n4 = p.n4;
    g.S = p.S;
    g.K = a.K;
    g.ctrl = reinterpret_cast<uint32_t*>(ws_ctrl);
    g.keys = reinterpret_cast<uint32_t*>(ws_data);
    AttnFuse af{};
    if (fa) {
        af = *a.attn;
        af.parts = reinterpret_cast<float*>(static_cast<uint8_t*>(ws_data) + p.data_bytes);
    }
    for (int64_t r0 = 0; r0 < p.rows; r0 += p.rows_per_launch) {
        const int64_t nr = (p.rows - r0) < p.rows_per_launch ? (p.rows - r0) : p.rows_per_launch;
        g.row0 = (int32_t)r0;
        hipLaunchKernelGGL(fn, dim3((unsigned)(nr * p.S)), dim3(kPsThreads), 0, stream, a.q, a.k, a.N, a.pool, g,
                           a.idx, a.idx_stride, a.score, af);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "launch k_pool_select");
    }
    return OK;
}

template <int KT, int QT>
int launch_ps_d(const PoolSelPlan& p, const PoolSelArgs& a, void* wc, void* wd, hipStream_t stream) {
    if (a.d_idx == 64) return launch_ps_typed<KT, QT, 64>(p, a, wc, wd, stream);
    if (a.d_idx == 128) return launch_ps_typed<KT, QT, 128>(p, a, wc, wd, stream);
    return fail(INVALID, "d_idx must be 64 or 128");
}

template <int KT>
int launch_ps_q(const PoolSelPlan& p, const PoolSelArgs& a, void* wc, void* wd, hipStream_t stream) {
    if (a.q_dtype == kF32) return launch_ps_d<KT, kF32>(p, a, wc, wd, stream);
    if (a.q_dtype == kBF16) return launch_ps_d<KT, kBF16>(p, a, wc, wd, stream);
    return fail(DTYPE, "indexer query dtype must be F32 or BF16");
}

}  // namespace

size_t pool_select_fused_bytes(const PoolSelPlan& p) {
    return p.data_bytes + (size_t)p.rows_per_launch * p.S * kPartFloats * 4;
}

int run_pool_select(const PoolSelPlan& p, const PoolSelArgs& a, void* ws_ctrl, void* ws_data, size_t data_bytes,
                    hipStream_t stream) {
    if (p.rows == 0) return OK;
    if (data_bytes < (a.attn ? pool_select_fused_bytes(p) : p.data_bytes))
        return fail(WORKSPACE, "pool select workspace too small");
    if (a.K < 1) return fail(INVALID, "pool select: K must be >= 1");
    switch (a.k_dtype) {
        case kF32: return launch_ps_q<kF32>(p, a, ws_ctrl, ws_data, stream);
        case kBF16: return launch_ps_q<kBF16>(p, a, ws_ctrl, ws_data, stream);
        case kE4M3: return launch_ps_q<kE4M3>(p, a, ws_ctrl, ws_data, stream);
        default: return fail(DTYPE, "indexer key dtype must be F32, BF16 or E4M3");
    }
}

}  // namespace csa2
