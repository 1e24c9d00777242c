// csa2_sparse_attn_fp4_noalloc: the sparse FP4 attention call with its
// scratch memory in a fixed device array instead of a caller workspace, for
// callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid allocation).
//
// The attention kernel's scratch is the per-row merge counters (zero between
// calls; every completed call leaves them zero) and, for rows split over
// several workgroups, their partial (max, sum, accumulator) states. Split
// rows times splits stay below 512 for every shape, so one array of
// kNoAllocScratchBytes covers any call. Each device holds its own copy of the
// array for the life of the process; its address is looked up once per device
// (hipGetSymbolAddress) and only that address is passed to kernels. All calls
// on one device share the array: calls that may overlap on one device (two
// streams, or two host threads) race and must be ordered by the caller.
#include <hip/hip_runtime.h>
#include <math.h>

#include <cmath>
#include <mutex>
#include <string>

#include "csa2.h"
#include "internal.hpp"

namespace csa2 {
namespace {

constexpr int kMaxDevices = 64;
constexpr size_t kCounterBytes = (size_t)kAttnCtrlWords * 4;
constexpr size_t kPartsOffset = 1024;
static_assert(kCounterBytes <= kPartsOffset, "merge counters fit before the partial states");
// 4,260,864 bytes: 1 KiB of counters and 511 partial states of 8,320 bytes
constexpr size_t kNoAllocScratchBytes = kPartsOffset + (size_t)511 * (16 * 128 + 2 * 16) * 4;

static __device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void k_zero_words(uint32_t* p, int n) {
    const int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0u;
}

std::mutex g_mu;
uint8_t* g_ptr[kMaxDevices] = {};

// The device address of this device's array (looked up on the first call with
// that device current; its counters are cleared then by a fill kernel on
// `stream`, ordered before the call's own kernel).
int scratch_ptr(hipStream_t stream, uint8_t** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(INVALID, "csa2_sparse_attn_fp4_noalloc: device ordinal too large");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_ptr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
        const int n = (int)(kCounterBytes / 4);
        hipLaunchKernelGGL(k_zero_words, dim3((n + 255) / 256), dim3(256), 0, stream, reinterpret_cast<uint32_t*>(p), n);
        e = hipGetLastError();
        if (e != hipSuccess) return hip_fail(e, "launch k_zero_words");
        g_ptr[dev] = reinterpret_cast<uint8_t*>(p);
    }
    *out = g_ptr[dev];
    return OK;
}

}  // namespace
}  // namespace csa2

using namespace csa2;

extern "C" int csa2_sparse_attn_fp4_noalloc(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d,
                                            const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v_codes,
                                            const uint8_t* v_scales, int64_t N, int64_t code_stride_bytes,
                                            int64_t scale_stride_bytes, const int32_t* idx, int32_t K,
                                            float softmax_scale, float* out, hipStream_t stream) {
    const char* who = "csa2_sparse_attn_fp4_noalloc";
    if (B < 0 || Q < 0) return fail(INVALID, std::string(who) + ": negative size");
    if ((int64_t)B * Q == 0) return OK;
    if (int e = check_attn(q, H, d, k_codes, k_scales, v_codes, v_scales, N, code_stride_bytes, scale_stride_bytes, K,
                           who, false))
        return e;
    if (!idx || !out) return fail(INVALID, std::string(who) + ": null pointer");
    if (!(softmax_scale >= 0.f) || !std::isfinite(softmax_scale))
        return fail(INVALID, std::string(who) + ": softmax_scale must be >= 0 and finite");
    if (softmax_scale == 0.f) softmax_scale = 1.0f / std::sqrt((float)d);
    const int64_t rows = (int64_t)B * Q;
    const size_t need = attn_data_bytes(rows, K);
    if (need > kNoAllocScratchBytes - kPartsOffset)
        return fail(WORKSPACE, std::string(who) + ": this shape needs " + std::to_string(need) +
                                   " bytes of partial states, more than the fixed scratch holds (" +
                                   std::to_string(kNoAllocScratchBytes - kPartsOffset) + ")");
    uint8_t* base = nullptr;
    if (int e = scratch_ptr(stream, &base)) return e;
    AttnArgs a;
    a.q = q;
    a.rows = rows;
    a.rows_per_seq = Q;
    a.H = H;
    a.d = d;
    a.k_codes = k_codes;
    a.k_scales = k_scales;
    a.v_codes = v_codes;
    a.v_scales = v_scales;
    a.N = N;
    a.code_stride = code_stride_bytes;
    a.scale_stride = scale_stride_bytes;
    a.idx = idx;
    a.idx_stride = K;
    a.K = K;
    a.scale = softmax_scale;
    a.out = out;
    return launch_attn_scratch(a, reinterpret_cast<uint32_t*>(base), base + kPartsOffset,
                               kNoAllocScratchBytes - kPartsOffset, stream);
}
