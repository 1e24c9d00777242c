// Dense indexer scores (the standalone Full and Reindex scoring calls).
//
// Same arithmetic as the fused scan inside the select kernel (dot.hpp): four
// lanes per key row, exact fp64 accumulation, one rounding to fp32. These
// kernels write the scores to HBM; the layer plan does not use them (its
// scores stay in LDS).
#include "dot.hpp"
#include "internal.hpp"

namespace csa2 {

constexpr int kIdxThreads = 256;
constexpr int kIdxKeysPerBlock = 1024;

template <int KT, int QT, int D>
__global__ void __launch_bounds__(kIdxThreads)
k_index_dense(const void* __restrict__ q, const uint8_t* __restrict__ k, int64_t N, int32_t Q,
              const int64_t* __restrict__ q_pos, float* __restrict__ scores) {
    using KS = KeySlice<KT, D, QT>;
    constexpr int QB = (QT == kBF16) ? 2 : 4;
    const int64_t row = blockIdx.y;                       // b*Q + i
    const int64_t seq = row / Q;
    const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
    double qd[D / 4];
    load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
    const int64_t qp = q_pos ? q_pos[row] : INT64_MAX;
    const uint8_t* kb = k + seq * N * (int64_t)KS::ROW_BYTES;
    float* out = scores + row * N;
    const int64_t t0 = (int64_t)blockIdx.x * kIdxKeysPerBlock;
    for (int j = 0; j < kIdxKeysPerBlock; j += kIdxThreads / 4) {
        const int64_t t = t0 + j + quad;
        KS s;
        if (t < N) s.load(kb + t * KS::ROW_BYTES, lq);
        else for (int w = 0; w < KS::RAW; ++w) s.raw[w] = make_uint4(0, 0, 0, 0);
        const auto v = quad_sum(s.dot(qd));
        if (lq == 0 && t < N) out[t] = (t > qp) ? -INFINITY : round_score(v);
    }
}

template <int KT, int QT, int D>
__global__ void __launch_bounds__(kIdxThreads)
k_index_pool(const void* __restrict__ q, const uint8_t* __restrict__ k, int64_t N, const int32_t* __restrict__ pool,
             int32_t P, float* __restrict__ scores) {
    using KS = KeySlice<KT, D, QT>;
    constexpr int QB = (QT == kBF16) ? 2 : 4;
    const int64_t row = blockIdx.y;
    const int quad = threadIdx.x >> 2, lq = threadIdx.x & 3;
    double qd[D / 4];
    load_query_slice<QT, D>(reinterpret_cast<const uint8_t*>(q) + row * (int64_t)(D * QB), lq, qd);
    const uint8_t* kb = k + row * N * (int64_t)KS::ROW_BYTES;
    const int64_t i0 = (int64_t)blockIdx.x * kIdxKeysPerBlock;
    for (int j = 0; j < kIdxKeysPerBlock; j += kIdxThreads / 4) {
        const int64_t i = i0 + j + quad;
        const int32_t pos = (i < P) ? pool[row * P + i] : -1;
        const bool ok = pos >= 0 && (int64_t)pos < N;
        KS s;
        if (ok) s.load(kb + (int64_t)pos * KS::ROW_BYTES, lq);
        else for (int w = 0; w < KS::RAW; ++w) s.raw[w] = make_uint4(0, 0, 0, 0);
        const auto v = quad_sum(s.dot(qd));
        if (lq == 0 && i < P) scores[row * P + i] = ok ? round_score(v) : -INFINITY;
    }
}

namespace {

template <int KT, int QT, int D>
int dense_typed(const ScanArgs& a, int32_t B, int32_t Q, float* scores, hipStream_t stream) {
    const dim3 grid((unsigned)((a.N + kIdxKeysPerBlock - 1) / kIdxKeysPerBlock), (unsigned)(B * Q));
    hipLaunchKernelGGL((k_index_dense<KT, QT, D>), grid, dim3(kIdxThreads), 0, stream, a.q, a.k, a.N, Q, a.q_pos,
                       scores);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_index_dense");
}

template <int KT, int QT, int D>
int pool_typed(const ScanArgs& a, int32_t B, int32_t P, float* scores, hipStream_t stream) {
    const dim3 grid((unsigned)((P + kIdxKeysPerBlock - 1) / kIdxKeysPerBlock), (unsigned)B);
    hipLaunchKernelGGL((k_index_pool<KT, QT, D>), grid, dim3(kIdxThreads), 0, stream, a.q, a.k, a.N, a.pool, P,
                       scores);
    const hipError_t e = hipGetLastError();
    return e == hipSuccess ? OK : hip_fail(e, "launch k_index_pool");
}

template <int KT, int QT>
int pick_d_dense(const ScanArgs& a, int32_t B, int32_t Q, float* s, hipStream_t st) {
    return a.d_idx == 64 ? dense_typed<KT, QT, 64>(a, B, Q, s, st) : dense_typed<KT, QT, 128>(a, B, Q, s, st);
}
template <int KT, int QT>
int pick_d_pool(const ScanArgs& a, int32_t B, int32_t P, float* s, hipStream_t st) {
    return a.d_idx == 64 ? pool_typed<KT, QT, 64>(a, B, P, s, st) : pool_typed<KT, QT, 128>(a, B, P, s, st);
}
template <int KT>
int pick_q_dense(const ScanArgs& a, int32_t B, int32_t Q, float* s, hipStream_t st) {
    return a.q_dtype == kF32 ? pick_d_dense<KT, kF32>(a, B, Q, s, st) : pick_d_dense<KT, kBF16>(a, B, Q, s, st);
}
template <int KT>
int pick_q_pool(const ScanArgs& a, int32_t B, int32_t P, float* s, hipStream_t st) {
    return a.q_dtype == kF32 ? pick_d_pool<KT, kF32>(a, B, P, s, st) : pick_d_pool<KT, kBF16>(a, B, P, s, st);
}

}  // namespace

int launch_index_dense(const ScanArgs& a, int32_t B, int32_t Q, float* scores, hipStream_t stream) {
    if (B == 0 || Q == 0 || a.N == 0) return OK;
    switch (a.k_dtype) {
        case kF32: return pick_q_dense<kF32>(a, B, Q, scores, stream);
        case kBF16: return pick_q_dense<kBF16>(a, B, Q, scores, stream);
        default: return pick_q_dense<kE4M3>(a, B, Q, scores, stream);
    }
}

int launch_index_pool(const ScanArgs& a, int32_t B, int32_t P, float* scores, hipStream_t stream) {
    if (B == 0 || P == 0) return OK;
    switch (a.k_dtype) {
        case kF32: return pick_q_pool<kF32>(a, B, P, scores, stream);
        case kBF16: return pick_q_pool<kBF16>(a, B, P, scores, stream);
        default: return pick_q_pool<kE4M3>(a, B, P, scores, stream);
    }
}

}  // namespace csa2
