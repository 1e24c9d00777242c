// C ABI of libcsa2: argument validation, the layer plan and kernel dispatch.
// Every check here runs on the host before any HIP call, so invalid calls are
// rejected on a machine without a GPU.
#include <math.h>
#include <stdint.h>
#include <string.h>

#include <mutex>
#include <string>
#include <vector>

#include "csa2.h"
#include "internal.hpp"

namespace csa2 {

static thread_local std::string g_err;

int fail(int code, const std::string& msg) {
    g_err = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    g_err = std::string(what) + ": " + hipGetErrorString(e);
    return HIP;
}

int device_info(DeviceInfo* out) {
    static std::mutex mu;
    static std::vector<DeviceInfo> cache;
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    std::lock_guard<std::mutex> lock(mu);
    for (const auto& d : cache)
        if (d.device == dev) {
            *out = d;
            return OK;
        }
    DeviceInfo d;
    d.device = dev;
    e = hipDeviceGetAttribute(&d.num_cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(CUs)");
    int lds = 0, lds_optin = 0;
    e = hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute(LDS)");
    if (hipDeviceGetAttribute(&lds_optin, hipDeviceAttributeSharedMemPerBlockOptin, dev) != hipSuccess) lds_optin = 0;
    (void)hipGetLastError();
    d.max_lds = (size_t)(lds_optin > lds ? lds_optin : lds);
    cache.push_back(d);
    *out = d;
    return OK;
}

}  // namespace csa2

using namespace csa2;

namespace {

constexpr size_t kAlign = 256;
size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool q_dtype_ok(int32_t t) { return t == CSA2_F32 || t == CSA2_BF16; }
bool k_dtype_ok(int32_t t) { return t == CSA2_F32 || t == CSA2_BF16 || t == CSA2_E4M3; }
int k_elem_bytes(int32_t t) { return t == CSA2_F32 ? 4 : (t == CSA2_BF16 ? 2 : 1); }

int check_ws(void* ws, size_t have, size_t need, const char* who) {
    if (need == 0) return OK;
    if (!ws) return fail(WORKSPACE, std::string(who) + ": workspace is null");
    if (!aligned(ws, kAlign)) return fail(WORKSPACE, std::string(who) + ": workspace must be 256-byte aligned");
    if (have < need)
        return fail(WORKSPACE, std::string(who) + ": workspace of " + std::to_string(have) + " bytes, need " +
                                   std::to_string(need));
    return OK;
}

int check_quant_layout(int64_t rows, int32_t C, int64_t x_stride, int64_t cs, int64_t ss, const void* x,
                       const void* codes, const void* scales, const char* who) {
    const std::string w(who);
    if (rows < 0) return fail(INVALID, w + ": rows < 0");
    if (C <= 0 || C % 16 != 0) return fail(INVALID, w + ": C must be a positive multiple of 16");
    if (x_stride < C) return fail(INVALID, w + ": bf16 row stride < C");
    if (cs < C / 2) return fail(INVALID, w + ": code row stride < C/2 bytes");
    if (ss < C / 16) return fail(INVALID, w + ": scale row stride < C/16 bytes");
    if (rows == 0) return OK;
    if (!x || !codes || !scales) return fail(INVALID, w + ": null pointer");
    if (!aligned(x, 16) || (x_stride * 2) % 16 != 0) return fail(INVALID, w + ": bf16 rows must be 16-byte aligned");
    if (!aligned(codes, 8) || cs % 8 != 0) return fail(INVALID, w + ": code rows must be 8-byte aligned");
    return OK;
}

int check_mx_layout(int64_t rows, int32_t C, int64_t x_stride, int64_t cs, int64_t ss, const void* x,
                    const void* codes, const void* scales, int code_align, const char* who) {
    const std::string w(who);
    if (rows < 0) return fail(INVALID, w + ": rows < 0");
    if (C <= 0 || C % 32 != 0) return fail(INVALID, w + ": C must be a positive multiple of 32");
    if (x_stride < C) return fail(INVALID, w + ": bf16 row stride < C");
    if (cs < C / 2) return fail(INVALID, w + ": code row stride < C/2 bytes");
    if (ss < C / 32) return fail(INVALID, w + ": scale row stride < C/32 bytes");
    if (rows == 0) return OK;
    if (!x || !codes || !scales) return fail(INVALID, w + ": null pointer");
    if (!aligned(x, 16) || (x_stride * 2) % 16 != 0) return fail(INVALID, w + ": bf16 rows must be 16-byte aligned");
    if (!aligned(codes, code_align) || cs % code_align != 0)
        return fail(INVALID, w + ": code rows must be " + std::to_string(code_align) + "-byte aligned");
    return OK;
}

int check_scan(const void* q_idx, int32_t q_dtype, const void* k_idx, int32_t k_dtype, int32_t d_idx, const char* who) {
    const std::string w(who);
    if (!q_dtype_ok(q_dtype)) return fail(DTYPE, w + ": indexer query dtype must be CSA2_F32 or CSA2_BF16");
    if (!k_dtype_ok(k_dtype)) return fail(DTYPE, w + ": indexer key dtype must be CSA2_F32, CSA2_BF16 or CSA2_E4M3");
    if (d_idx != 64 && d_idx != 128) return fail(INVALID, w + ": d_idx must be 64 or 128");
    if (!q_idx || !k_idx) return fail(INVALID, w + ": null indexer pointer");
    if (!aligned(k_idx, 16)) return fail(INVALID, w + ": indexer keys must be 16-byte aligned");
    if (!aligned(q_idx, q_dtype == CSA2_F32 ? 4 : 2)) return fail(INVALID, w + ": indexer query misaligned");
    return OK;
}

}  // namespace

namespace csa2 {

int check_attn(const uint16_t* q, int32_t H, int32_t d, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
               const uint8_t* vs, int64_t N, int64_t cs, int64_t ss, int32_t K, const char* who, bool mx) {
    const std::string w(who);
    if (H < 1 || H > 16) return fail(INVALID, w + ": H must be in 1..16");
    if (d != 128) return fail(INVALID, w + ": head dim d must be 128");
    if (K < 1) return fail(INVALID, w + ": K must be >= 1");
    if (N < 1) return fail(INVALID, w + ": N must be >= 1");
    if (cs < d / 2 || ss < (mx ? d / 32 : d / 16)) return fail(INVALID, w + ": KV code/scale stride smaller than one row");
    if (!q || !kc || !ks || !vc || !vs) return fail(INVALID, w + ": null pointer");
    if (!aligned(kc, 16) || !aligned(vc, 16) || cs % 16 != 0)
        return fail(INVALID, w + ": KV code rows must be 16-byte aligned");
    if (!aligned(q, 16)) return fail(INVALID, w + ": query must be 16-byte aligned");
    const int sa = mx ? 4 : 8;                  // each position's K (V) scales are read as one word
    if (!aligned(ks, sa) || !aligned(vs, sa) || ss % sa != 0)
        return fail(INVALID, w + (mx ? ": KV scale rows must be 4-byte aligned" : ": KV scale rows must be 8-byte aligned"));
    return OK;
}

}  // namespace csa2

extern "C" {

const char* csa2_last_error(void) { return g_err.c_str(); }

int csa2_version(void) { return 100; }

int kv_quant_fp4(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride, uint8_t* codes,
                 int64_t code_stride_bytes, uint8_t* scales, int64_t scale_stride_bytes, hipStream_t stream) {
    g_err.clear();
    if (int e = check_quant_layout(rows, C, x_stride, code_stride_bytes, scale_stride_bytes, x, codes, scales,
                                   "kv_quant_fp4"))
        return e;
    return launch_quant(x, rows, C, x_stride, codes, code_stride_bytes, scales, scale_stride_bytes, stream);
}

int kv_dequant_fp4(const uint8_t* codes, int64_t code_stride_bytes, const uint8_t* scales, int64_t scale_stride_bytes,
                   int64_t rows, int32_t C, uint16_t* y, int64_t y_stride, hipStream_t stream) {
    g_err.clear();
    if (int e = check_quant_layout(rows, C, y_stride, code_stride_bytes, scale_stride_bytes, y, codes, scales,
                                   "kv_dequant_fp4"))
        return e;
    return launch_dequant(codes, code_stride_bytes, scales, scale_stride_bytes, rows, C, y, y_stride, stream);
}

int kv_quant_mxfp4(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride, uint8_t* codes,
                   int64_t code_stride_bytes, uint8_t* scales, int64_t scale_stride_bytes, hipStream_t stream) {
    g_err.clear();
    if (int e = check_mx_layout(rows, C, x_stride, code_stride_bytes, scale_stride_bytes, x, codes, scales, 16,
                                "kv_quant_mxfp4"))
        return e;
    return launch_quant_mx(x, rows, C, x_stride, codes, code_stride_bytes, scales, scale_stride_bytes, stream);
}

int kv_dequant_mxfp4(const uint8_t* codes, int64_t code_stride_bytes, const uint8_t* scales, int64_t scale_stride_bytes,
                     int64_t rows, int32_t C, uint16_t* y, int64_t y_stride, hipStream_t stream) {
    g_err.clear();
    if (int e = check_mx_layout(rows, C, y_stride, code_stride_bytes, scale_stride_bytes, y, codes, scales, 4,
                                "kv_dequant_mxfp4"))
        return e;
    return launch_dequant_mx(codes, code_stride_bytes, scales, scale_stride_bytes, rows, C, y, y_stride, stream);
}

int csa2_kv_project(const uint16_t* h, int64_t T, int32_t D, int64_t h_stride, const uint16_t* w_t, int64_t w_stride,
                    int32_t kv_format, uint8_t* codes, int64_t code_stride_bytes, uint8_t* scales,
                    int64_t scale_stride_bytes, uint16_t* c_out, int64_t c_stride, hipStream_t stream) {
    g_err.clear();
    const char* w = "csa2_kv_project";
    if (T < 0) return fail(INVALID, std::string(w) + ": T < 0");
    if (D <= 0 || D % 64 != 0) return fail(INVALID, std::string(w) + ": D must be a positive multiple of 64");
    if (kv_format != CSA2_KV_FP4_E4M3 && kv_format != CSA2_KV_MXFP4)
        return fail(INVALID, std::string(w) + ": kv_format must be CSA2_KV_FP4_E4M3 or CSA2_KV_MXFP4");
    const bool mx = kv_format == CSA2_KV_MXFP4;
    if (h_stride < D || w_stride < D) return fail(INVALID, std::string(w) + ": row stride < D");
    if (code_stride_bytes < 128) return fail(INVALID, std::string(w) + ": code row stride < 128 bytes");
    if (scale_stride_bytes < (mx ? 8 : 16)) return fail(INVALID, std::string(w) + ": scale row stride too small");
    if (c_out && c_stride < 256) return fail(INVALID, std::string(w) + ": c_out row stride < 256");
    if (T == 0) return OK;
    if (!h || !w_t || !codes || !scales) return fail(INVALID, std::string(w) + ": null pointer");
    if (!aligned(h, 16) || (h_stride * 2) % 16 || !aligned(w_t, 16) || (w_stride * 2) % 16)
        return fail(INVALID, std::string(w) + ": h and w_t rows must be 16-byte aligned");
    const int ca = mx ? 16 : 8;
    if (!aligned(codes, ca) || code_stride_bytes % ca)
        return fail(INVALID, std::string(w) + ": code rows must be " + std::to_string(ca) + "-byte aligned");
    if (c_out && (!aligned(c_out, 16) || (c_stride * 2) % 16))
        return fail(INVALID, std::string(w) + ": c_out rows must be 16-byte aligned");
    return launch_kv_project(h, T, D, h_stride, w_t, w_stride, mx, codes, code_stride_bytes, scales,
                             scale_stride_bytes, c_out, c_stride, stream);
}

int csa2_index_full(const void* q_idx, int32_t q_dtype, const void* k_idx, int32_t k_dtype, int32_t B, int32_t Q,
                    int64_t N, int32_t d_idx, const int64_t* q_pos, float* scores, hipStream_t stream) {
    g_err.clear();
    if (B < 0 || Q < 0 || N < 0) return fail(INVALID, "csa2_index_full: negative size");
    if ((int64_t)B * Q > 65535) return fail(INVALID, "csa2_index_full: B*Q must be <= 65535");
    if ((int64_t)B * Q == 0 || N == 0) return OK;
    if (int e = check_scan(q_idx, q_dtype, k_idx, k_dtype, d_idx, "csa2_index_full")) return e;
    if (!scores) return fail(INVALID, "csa2_index_full: scores is null");
    ScanArgs a;
    a.q = q_idx;
    a.k = reinterpret_cast<const uint8_t*>(k_idx);
    a.N = N;
    a.q_pos = q_pos;
    a.q_dtype = q_dtype;
    a.k_dtype = k_dtype;
    a.d_idx = d_idx;
    return launch_index_dense(a, B, Q, scores, stream);
}

int csa2_index_reindex(const void* q_idx, int32_t q_dtype, const void* k_idx, int32_t k_dtype, int32_t B, int64_t N,
                       int32_t d_idx, const int32_t* pool, int32_t P, float* scores, hipStream_t stream) {
    g_err.clear();
    if (B < 0 || N < 0 || P < 0) return fail(INVALID, "csa2_index_reindex: negative size");
    if (B > 65535) return fail(INVALID, "csa2_index_reindex: B must be <= 65535");
    if (B == 0 || P == 0) return OK;
    if (int e = check_scan(q_idx, q_dtype, k_idx, k_dtype, d_idx, "csa2_index_reindex")) return e;
    if (!pool || !scores) return fail(INVALID, "csa2_index_reindex: null pointer");
    ScanArgs a;
    a.q = q_idx;
    a.k = reinterpret_cast<const uint8_t*>(k_idx);
    a.N = N;
    a.pool = pool;
    a.q_dtype = q_dtype;
    a.k_dtype = k_dtype;
    a.d_idx = d_idx;
    return launch_index_pool(a, B, P, scores, stream);
}

int csa2_topk_workspace_bytes(int64_t rows, int64_t n, int32_t K, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(INVALID, "csa2_topk_workspace_bytes: bytes is null");
    if (rows < 0 || n < 1 || n >= (int64_t(1) << 31) || K < 1)
        return fail(INVALID, "csa2_topk_workspace_bytes: need rows >= 0, 1 <= n < 2^31, K >= 1");
    SelPlan p;
    if (int e = plan_select(rows, n, 1024, &p)) return e;
    *bytes = align_up(p.ws_bytes);
    return OK;
}

int csa2_topk(const float* scores, int64_t rows, int64_t n, int64_t score_stride, const int32_t* cand, int32_t K,
              int32_t* idx, float* sel_scores, void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    if (rows < 0 || n < 1 || n >= (int64_t(1) << 31) || K < 1)
        return fail(INVALID, "csa2_topk: need rows >= 0, 1 <= n < 2^31, K >= 1");
    if (score_stride < n) return fail(INVALID, "csa2_topk: score_stride < n");
    if (rows == 0) return OK;
    if (!scores || !idx) return fail(INVALID, "csa2_topk: null pointer");
    SelPlan p;
    if (int e = plan_select(rows, n, 1024, &p)) return e;
    if (int e = check_ws(ws, ws_bytes, p.ws_bytes, "csa2_topk")) return e;
    ScanArgs scan;
    ScoresArgs sc;
    sc.scores = scores;
    sc.stride = score_stride;
    sc.cand = cand;
    SelOutput o;
    o.idx = idx;
    o.score = sel_scores;
    o.stride = K;
    o.M = K;
    return run_select(p, SRC_SCORES, scan, sc, &o, 1, ws, static_cast<uint8_t*>(ws) + kCtrlBytes, stream);
}

int csa2_sparse_attn_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t d, int32_t K, size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(INVALID, "csa2_sparse_attn_workspace_bytes: bytes is null");
    if (B < 0 || Q < 0 || H < 1 || H > 16 || d != 128 || K < 1)
        return fail(INVALID, "csa2_sparse_attn_workspace_bytes: bad sizes");
    *bytes = align_up(kCtrlBytes + attn_data_bytes((int64_t)B * Q, K));
    return OK;
}

int csa2_sparse_attn_fp4(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d, const uint8_t* k_codes,
                         const uint8_t* k_scales, const uint8_t* v_codes, const uint8_t* v_scales, int64_t N,
                         int64_t code_stride_bytes, int64_t scale_stride_bytes, const int32_t* idx, int32_t K,
                         float softmax_scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    if (B < 0 || Q < 0) return fail(INVALID, "csa2_sparse_attn_fp4: negative size");
    if ((int64_t)B * Q == 0) return OK;
    if (int e = check_attn(q, H, d, k_codes, k_scales, v_codes, v_scales, N, code_stride_bytes, scale_stride_bytes, K,
                           "csa2_sparse_attn_fp4", false))
        return e;
    if (!idx || !out) return fail(INVALID, "csa2_sparse_attn_fp4: null pointer");
    if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
        return fail(INVALID, "csa2_sparse_attn_fp4: softmax_scale must be >= 0 and finite");
    if (softmax_scale == 0.f) softmax_scale = 1.0f / sqrtf((float)d);
    const size_t need = kCtrlBytes + attn_data_bytes((int64_t)B * Q, K);
    if (int e = check_ws(ws, ws_bytes, need, "csa2_sparse_attn_fp4")) return e;
    AttnArgs a;
    a.q = q;
    a.rows = (int64_t)B * Q;
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
    return launch_attn(a, ws, static_cast<uint8_t*>(ws) + kCtrlBytes, ws_bytes - kCtrlBytes, stream);
}

int csa2_sparse_attn_mxfp4(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d, const uint8_t* k_codes,
                         const uint8_t* k_scales, const uint8_t* v_codes, const uint8_t* v_scales, int64_t N,
                         int64_t code_stride_bytes, int64_t scale_stride_bytes, const int32_t* idx, int32_t K,
                         float softmax_scale, float* out, void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    if (B < 0 || Q < 0) return fail(INVALID, "csa2_sparse_attn_mxfp4: negative size");
    if ((int64_t)B * Q == 0) return OK;
    if (int e = check_attn(q, H, d, k_codes, k_scales, v_codes, v_scales, N, code_stride_bytes, scale_stride_bytes, K,
                           "csa2_sparse_attn_mxfp4", true))
        return e;
    if (!idx || !out) return fail(INVALID, "csa2_sparse_attn_mxfp4: null pointer");
    if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
        return fail(INVALID, "csa2_sparse_attn_mxfp4: softmax_scale must be >= 0 and finite");
    if (softmax_scale == 0.f) softmax_scale = 1.0f / sqrtf((float)d);
    const size_t need = kCtrlBytes + attn_data_bytes((int64_t)B * Q, K);
    if (int e = check_ws(ws, ws_bytes, need, "csa2_sparse_attn_mxfp4")) return e;
    AttnArgs a;
    a.q = q;
    a.rows = (int64_t)B * Q;
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
    a.mx = true;
    return launch_attn(a, ws, static_cast<uint8_t*>(ws) + kCtrlBytes, ws_bytes - kCtrlBytes, stream);
}

int csa2_sparse_attn_swa_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t d, int32_t K, int32_t W,
                                         size_t* bytes) {
    g_err.clear();
    if (!bytes) return fail(INVALID, "csa2_sparse_attn_swa_workspace_bytes: bytes is null");
    if (B < 0 || Q < 0 || H < 1 || H > 16 || d != 128 || K < 1 || W < 0)
        return fail(INVALID, "csa2_sparse_attn_swa_workspace_bytes: bad sizes");
    *bytes = align_up(kCtrlBytes + attn_data_bytes((int64_t)B * Q, K, W));
    return OK;
}

int csa2_sparse_attn_swa(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d, int32_t kv_format,
                         const uint8_t* k_codes, const uint8_t* k_scales, const uint8_t* v_codes,
                         const uint8_t* v_scales, int64_t N, int64_t code_stride_bytes, int64_t scale_stride_bytes,
                         const int32_t* idx, int32_t K, const uint16_t* win_k, const uint16_t* win_v,
                         int64_t win_row_stride, int32_t W, const int32_t* win_len, float softmax_scale, float* out,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    const char* who = "csa2_sparse_attn_swa";
    if (B < 0 || Q < 0 || W < 0) return fail(INVALID, std::string(who) + ": negative size");
    if ((int64_t)B * Q == 0) return OK;
    if (kv_format != CSA2_KV_FP4_E4M3 && kv_format != CSA2_KV_MXFP4)
        return fail(INVALID, std::string(who) + ": kv_format must be CSA2_KV_FP4_E4M3 or CSA2_KV_MXFP4");
    const bool mx = kv_format == CSA2_KV_MXFP4;
    if (int e = check_attn(q, H, d, k_codes, k_scales, v_codes, v_scales, N, code_stride_bytes, scale_stride_bytes, K,
                           who, mx))
        return e;
    if (!idx || !out) return fail(INVALID, std::string(who) + ": null pointer");
    if (W > 0) {
        if (!win_k || !win_v) return fail(INVALID, std::string(who) + ": window pointers are null");
        if (!aligned(win_k, 16) || !aligned(win_v, 16)) return fail(INVALID, std::string(who) + ": window rows must be 16-byte aligned");
        if (win_row_stride < (int64_t)W * d) return fail(INVALID, std::string(who) + ": window row stride < W*d");
        if (win_row_stride % 8) return fail(INVALID, std::string(who) + ": window row stride must keep 16-byte alignment");
    }
    if (!(softmax_scale >= 0.f) || !isfinite(softmax_scale))
        return fail(INVALID, std::string(who) + ": softmax_scale must be >= 0 and finite");
    if (softmax_scale == 0.f) softmax_scale = 1.0f / sqrtf((float)d);
    const size_t need = kCtrlBytes + attn_data_bytes((int64_t)B * Q, K, W);
    if (int e = check_ws(ws, ws_bytes, need, who)) return e;
    AttnArgs a;
    a.q = q;
    a.rows = (int64_t)B * Q;
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
    a.mx = mx;
    a.win_k = win_k;
    a.win_v = win_v;
    a.win_rs = win_row_stride;
    a.Wn = W;
    a.win_len = win_len;
    return launch_attn(a, ws, static_cast<uint8_t*>(ws) + kCtrlBytes, ws_bytes - kCtrlBytes, stream);
}

// ------------------------------------------------------------------- plan

struct csa2_plan {
    std::vector<int32_t> modes;
    std::vector<int32_t> group;         // per layer: index of its Full layer's group (its cache)
    std::vector<uint8_t> group_pool;    // per group: a Reindex layer follows its Full layer
    int32_t groups = 0;
    csa2_plan_params p;
    bool has_reindex = false;
    // timing aid: events[(run * 2L + slot) * 2 + {0 start, 1 stop}]
    mutable std::vector<hipEvent_t> events;
    mutable std::vector<uint8_t> used;        // [run][slot] recorded?
    mutable int32_t max_runs = 0, runs = 0;

    void drop_events() const {
        for (hipEvent_t e : events)
            if (e) (void)hipEventDestroy(e);
        events.clear();
        used.clear();
        max_runs = runs = 0;
    }
    ~csa2_plan() { drop_events(); }
};

namespace {

// Records the start/stop events of one kernel slot when profiling is on.
struct SlotTimer {
    const csa2_plan* plan;
    int slot;
    hipStream_t stream;
    bool on;
    SlotTimer(const csa2_plan* pl, int s, hipStream_t st) : plan(pl), slot(s), stream(st) {
        on = pl->runs < pl->max_runs;
        if (on) {
            const size_t L2 = 2 * pl->modes.size();
            (void)hipEventRecord(pl->events[((size_t)pl->runs * L2 + slot) * 2 + 0], stream);
            pl->used[(size_t)pl->runs * L2 + slot] = 1;
        }
    }
    ~SlotTimer() {
        if (on) {
            const size_t L2 = 2 * plan->modes.size();
            (void)hipEventRecord(plan->events[((size_t)plan->runs * L2 + slot) * 2 + 1], stream);
        }
    }
};

}  // namespace

int csa2_plan_profile_begin(csa2_plan* plan, int32_t max_runs) {
    g_err.clear();
    if (!plan || max_runs < 0) return fail(INVALID, "csa2_plan_profile_begin: bad arguments");
    plan->drop_events();
    if (max_runs == 0) return OK;
    const size_t n = (size_t)max_runs * 2 * plan->modes.size() * 2;
    plan->events.assign(n, nullptr);
    for (size_t i = 0; i < n; ++i) {
        hipError_t e = hipEventCreate(&plan->events[i]);
        if (e != hipSuccess) {
            plan->drop_events();
            return hip_fail(e, "hipEventCreate");
        }
    }
    plan->used.assign((size_t)max_runs * 2 * plan->modes.size(), 0);
    plan->max_runs = max_runs;
    plan->runs = 0;
    return OK;
}

int csa2_plan_profile_read(csa2_plan* plan, float* avg_ms, int32_t* runs) {
    g_err.clear();
    if (!plan || !avg_ms || !runs) return fail(INVALID, "csa2_plan_profile_read: null pointer");
    const size_t L2 = 2 * plan->modes.size();
    for (size_t s = 0; s < L2; ++s) {
        double sum = 0.0;
        int n = 0;
        for (int32_t r = 0; r < plan->runs; ++r) {
            if (!plan->used[(size_t)r * L2 + s]) continue;
            hipEvent_t a = plan->events[((size_t)r * L2 + s) * 2 + 0], b = plan->events[((size_t)r * L2 + s) * 2 + 1];
            hipError_t e = hipEventSynchronize(b);
            if (e != hipSuccess) return hip_fail(e, "hipEventSynchronize");
            float ms = 0.f;
            e = hipEventElapsedTime(&ms, a, b);
            if (e != hipSuccess) return hip_fail(e, "hipEventElapsedTime");
            sum += ms;
            ++n;
        }
        avg_ms[s] = n ? (float)(sum / n) : 0.f;
    }
    *runs = plan->runs;
    return OK;
}

int csa2_plan_create(const int32_t* modes, int32_t L, const csa2_plan_params* params, csa2_plan** out) {
    g_err.clear();
    if (!out) return fail(INVALID, "csa2_plan_create: out is null");
    *out = nullptr;
    if (!modes || !params || L < 1) return fail(INVALID, "csa2_plan_create: need modes, params and L >= 1");
    const csa2_plan_params& p = *params;
    for (int32_t l = 0; l < L; ++l)
        if (modes[l] != CSA2_FULL && modes[l] != CSA2_REINDEX && modes[l] != CSA2_REUSE)
            return fail(BAD_PLAN, "csa2_plan_create: unknown mode at layer " + std::to_string(l));
    if (modes[0] != CSA2_FULL) return fail(BAD_PLAN, "csa2_plan_create: the first layer must be Full");
    bool has_reindex = false;
    for (int32_t l = 0; l < L; ++l) has_reindex |= modes[l] == CSA2_REINDEX;
    if (p.K < 1) return fail(INVALID, "csa2_plan_create: K must be >= 1");
    if (has_reindex && p.P < p.K) return fail(BAD_PLAN, "csa2_plan_create: a Reindex layer needs P >= K");
    if (p.H < 1 || p.H > 16) return fail(INVALID, "csa2_plan_create: H must be in 1..16");
    if (p.d != 128) return fail(INVALID, "csa2_plan_create: d must be 128");
    if (p.d_idx != 64 && p.d_idx != 128) return fail(INVALID, "csa2_plan_create: d_idx must be 64 or 128");
    if (!q_dtype_ok(p.q_idx_dtype)) return fail(DTYPE, "csa2_plan_create: indexer query dtype");
    if (!k_dtype_ok(p.k_idx_dtype)) return fail(DTYPE, "csa2_plan_create: indexer key dtype");
    if (!(p.softmax_scale >= 0.f) || !isfinite(p.softmax_scale))
        return fail(INVALID, "csa2_plan_create: softmax_scale must be >= 0 and finite");
    if (p.kv_format != CSA2_KV_FP4_E4M3 && p.kv_format != CSA2_KV_MXFP4)
        return fail(INVALID, "csa2_plan_create: kv_format must be CSA2_KV_FP4_E4M3 or CSA2_KV_MXFP4");
    if (p.swa_window < 0 || p.swa_window > 65536)
        return fail(INVALID, "csa2_plan_create: swa_window must be in 0..65536");
    csa2_plan* plan = new csa2_plan;
    plan->modes.assign(modes, modes + L);
    plan->p = p;
    if (plan->p.softmax_scale == 0.f) plan->p.softmax_scale = 1.0f / sqrtf((float)p.d);
    plan->has_reindex = has_reindex;
    for (int32_t l = 0; l < L; ++l) {
        if (modes[l] == CSA2_FULL) {
            plan->groups += 1;
            plan->group_pool.push_back(0);
        }
        plan->group.push_back(plan->groups - 1);
        if (modes[l] == CSA2_REINDEX) plan->group_pool.back() = 1;
    }
    *out = plan;
    return OK;
}

void csa2_plan_destroy(csa2_plan* plan) { delete plan; }

namespace {

// Plan workspace: the shared control region, then the data regions of the
// Full select, the Reindex select, the pool, the attention and the positions.
struct PlanLayout {
    SelPlan full, pool;
    PoolSelPlan psel;               // Reindex select when the pool has at most kPoolSelMaxN entries
    bool use_psel = false;
    bool fuse_reindex = false;      // the Reindex layers' attention runs inside the pool select
    bool fuse_full = false;         // the Full layers' attention runs inside their select
    size_t off_full = 0, off_pool = 0, off_attn = 0, off_idx = 0, off_poolbuf = 0, total = 0;
};

int plan_layout(const csa2_plan* plan, int32_t B, int64_t N, PlanLayout* lay) {
    if (int e = plan_select(B, N, 1024, &lay->full)) return e;
    size_t off = align_up(kCtrlBytes);
    lay->off_full = off;
    off += align_up(lay->full.data_bytes);
    if (plan->has_reindex) {
        lay->use_psel = plan->p.P <= kPoolSelMaxN;
        size_t pool_data = 0;
        if (lay->use_psel) {
            if (int e = plan_pool_select(B, plan->p.P, &lay->psel)) return e;
            // the fused attention covers the E4M3-scaled cache without a sliding window
            lay->fuse_reindex = plan->p.kv_format == CSA2_KV_FP4_E4M3 && plan->p.swa_window == 0;
            pool_data = lay->fuse_reindex ? pool_select_fused_bytes(lay->psel) : lay->psel.data_bytes;
        } else {
            if (int e = plan_select(B, plan->p.P, 512, &lay->pool)) return e;
            pool_data = lay->pool.data_bytes;
        }
        lay->off_pool = off;
        off += align_up(pool_data);
        lay->off_poolbuf = off;
        off += align_up((size_t)B * plan->p.P * 4);
    }
    // the fused attention covers the E4M3-scaled cache without a sliding window, up to 4096 positions,
    // in rows of at most 8 chunks (their states merge in one batch of loads; longer rows keep the
    // attention kernel, which spreads a row over at most 8 workgroups)
    lay->fuse_full = plan->p.kv_format == CSA2_KV_FP4_E4M3 && plan->p.swa_window == 0 && plan->p.K <= 4096 &&
                     lay->full.S <= 8;
    lay->off_attn = off;
    size_t attn_bytes = attn_data_bytes(B, plan->p.K, plan->p.swa_window);
    if (lay->fuse_full && select_fused_part_bytes(lay->full) > attn_bytes) attn_bytes = select_fused_part_bytes(lay->full);
    off += align_up(attn_bytes);
    lay->off_idx = off;
    off += align_up((size_t)B * plan->p.K * 4);
    lay->total = off;
    return OK;
}

}  // namespace

int csa2_plan_workspace_bytes(const csa2_plan* plan, int32_t B, int64_t N, size_t* bytes) {
    g_err.clear();
    if (!plan || !bytes) return fail(INVALID, "csa2_plan_workspace_bytes: null pointer");
    if (B < 1 || N < 1) return fail(INVALID, "csa2_plan_workspace_bytes: B and N must be >= 1");
    PlanLayout lay;
    if (int e = plan_layout(plan, B, N, &lay)) return e;
    *bytes = lay.total;
    return OK;
}

int csa2_plan_run_decode(const csa2_plan* plan, const csa2_cache* cache, const csa2_layer_io* io, int32_t B, int64_t N,
                         void* ws, size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    if (!plan || !cache || !io) return fail(INVALID, "csa2_plan_run_decode: null pointer");
    if (B < 1 || N < 1) return fail(INVALID, "csa2_plan_run_decode: B and N must be >= 1");
    if (B > 65535) return fail(INVALID, "csa2_plan_run_decode: B must be <= 65535");
    const csa2_plan_params& p = plan->p;
    const int L = (int)plan->modes.size();
    if (plan->has_reindex && p.P > N) return fail(INVALID, "csa2_plan_run_decode: pool size P exceeds N");
    for (int32_t gi = 0; gi < plan->groups; ++gi) {      // one cache per Full layer
        const csa2_cache* c = &cache[gi];
        if (int e = check_attn(io[0].q, p.H, p.d, c->k_codes, c->k_scales, c->v_codes, c->v_scales, N,
                               c->code_stride_bytes, c->scale_stride_bytes, p.K, "csa2_plan_run_decode",
                               p.kv_format == CSA2_KV_MXFP4))
            return e;
        if (!c->k_idx || !aligned(c->k_idx, 16))
            return fail(INVALID, "csa2_plan_run_decode: indexer keys null or not 16-byte aligned");
    }
    for (int l = 0; l < L; ++l) {
        if (!io[l].q || !io[l].out) return fail(INVALID, "csa2_plan_run_decode: layer " + std::to_string(l) + " needs q and out");
        if (plan->modes[l] != CSA2_REUSE && !io[l].q_idx)
            return fail(INVALID, "csa2_plan_run_decode: layer " + std::to_string(l) + " needs q_idx");
        if (p.swa_window > 0 && (!io[l].win_k || !io[l].win_v || !aligned(io[l].win_k, 16) || !aligned(io[l].win_v, 16)))
            return fail(INVALID, "csa2_plan_run_decode: layer " + std::to_string(l) +
                                     " needs 16-byte aligned window rows win_k and win_v (the plan has swa_window > 0)");
    }
    PlanLayout lay;
    if (int e = plan_layout(plan, B, N, &lay)) return e;
    if (int e = check_ws(ws, ws_bytes, lay.total, "csa2_plan_run_decode")) return e;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);

    const int32_t* cur_idx = nullptr;
    const int32_t* pool = nullptr;
    for (int l = 0; l < L; ++l) {
        const int32_t mode = plan->modes[l];
        const csa2_cache* gc = &cache[plan->group[l]];
        if (mode == CSA2_FULL || mode == CSA2_REINDEX) {
            int32_t* idx_dst = io[l].idx_out ? io[l].idx_out : reinterpret_cast<int32_t*>(wsb + lay.off_idx);
            ScanArgs a;
            a.q = io[l].q_idx;
            a.k = reinterpret_cast<const uint8_t*>(gc->k_idx);
            a.N = N;
            a.q_dtype = p.q_idx_dtype;
            a.k_dtype = p.k_idx_dtype;
            a.d_idx = p.d_idx;
            ScoresArgs none;
            SelOutput o[2];
            int nt = 1;
            int e;
            SlotTimer timer(plan, 2 * l, stream);
            AttnFuse fa{};                      // the layer's attention, when it runs inside the select
            fa.q = io[l].q;
            fa.k_codes = gc->k_codes;
            fa.k_scales = gc->k_scales;
            fa.v_codes = gc->v_codes;
            fa.v_scales = gc->v_scales;
            fa.N = N;
            fa.cs = gc->code_stride_bytes;
            fa.ss = gc->scale_stride_bytes;
            fa.H = p.H;
            fa.rows_per_seq = 1;
            fa.scale = p.softmax_scale;
            fa.out = io[l].out;
            if (mode == CSA2_FULL) {
                pool = nullptr;                 // a Full layer opens a group: its own pool, if any
                if (plan->group_pool[plan->group[l]]) {
                    int32_t* pool_dst = io[l].pool_out ? io[l].pool_out : reinterpret_cast<int32_t*>(wsb + lay.off_poolbuf);
                    o[0] = SelOutput{pool_dst, nullptr, p.P, p.P};
                    o[1] = SelOutput{idx_dst, nullptr, p.K, p.K};
                    nt = 2;
                    pool = pool_dst;
                } else {
                    o[0] = SelOutput{idx_dst, nullptr, p.K, p.K};
                }
                if (lay.fuse_full) {
                    fa.parts = reinterpret_cast<float*>(wsb + lay.off_attn);
                    a.attn = &fa;
                }
                e = run_select(lay.full, SRC_SCAN, a, none, o, nt, wsb, wsb + lay.off_full, stream);
            } else if (lay.use_psel) {
                PoolSelArgs ps;
                ps.q = io[l].q_idx;
                ps.k = a.k;
                ps.N = N;
                ps.pool = pool;
                ps.q_dtype = p.q_idx_dtype;
                ps.k_dtype = p.k_idx_dtype;
                ps.d_idx = p.d_idx;
                ps.K = p.K;
                ps.idx = idx_dst;
                ps.idx_stride = p.K;
                if (lay.fuse_reindex) ps.attn = &fa;
                e = run_pool_select(lay.psel, ps, wsb, wsb + lay.off_pool,
                                    lay.fuse_reindex ? pool_select_fused_bytes(lay.psel) : lay.psel.data_bytes, stream);
            } else {
                a.pool = pool;
                o[0] = SelOutput{idx_dst, nullptr, p.K, p.K};
                e = run_select(lay.pool, SRC_POOL, a, none, o, 1, wsb, wsb + lay.off_pool, stream);
            }
            if (e) return e;
            cur_idx = idx_dst;
            if ((mode == CSA2_REINDEX && lay.use_psel && lay.fuse_reindex) || (mode == CSA2_FULL && lay.fuse_full))
                continue;                       // attended in the select
        }
        AttnArgs at;
        at.q = io[l].q;
        at.rows = B;
        at.rows_per_seq = 1;
        at.H = p.H;
        at.d = p.d;
        at.k_codes = gc->k_codes;
        at.k_scales = gc->k_scales;
        at.v_codes = gc->v_codes;
        at.v_scales = gc->v_scales;
        at.N = N;
        at.code_stride = gc->code_stride_bytes;
        at.scale_stride = gc->scale_stride_bytes;
        at.idx = cur_idx;
        at.idx_stride = p.K;
        at.K = p.K;
        at.scale = p.softmax_scale;
        at.out = io[l].out;
        at.mx = p.kv_format == CSA2_KV_MXFP4;
        if (p.swa_window > 0) {
            at.win_k = io[l].win_k;
            at.win_v = io[l].win_v;
            at.win_rs = (int64_t)p.swa_window * p.d;
            at.Wn = p.swa_window;
            at.win_len = io[l].win_len;
        }
        SlotTimer timer(plan, 2 * l + 1, stream);
        if (int e = launch_attn(at, wsb, wsb + lay.off_attn, lay.off_idx - lay.off_attn, stream)) return e;
    }
    if (plan->runs < plan->max_runs) plan->runs += 1;
    return OK;
}

}  // extern "C"

namespace {

// Prefill selection workspace (one region, at the start of the data area):
// (matrix-core indexer path) the key maxima, the sample scores (later reused
// for the candidate lists), the sample top-R, the thresholds and counters,
// the repair queue and map, one data region shared by the three select calls
// (they run one after another); or (exact path) one select region.
constexpr int32_t kSampleStride = 64;           // every 64th position is sampled
constexpr int32_t kRepairRows = 64;             // queued rows the multi-workgroup exact repair pass takes
constexpr int64_t kRthMaxSamples = 16384;       // sample rows the threshold kernel holds in registers

struct PrefillLayout {
    bool mfma = false;
    int32_t M = 0;                              // the (larger) number of positions selected per query
    int64_t rows = 0, ns = 0;
    int32_t R = 0, nr = 0, nrd = 0, cap = 0;
    int64_t cand_dense = 0;                     // most candidates per query the exact select holds
    SelPlan sel_sample, sel_cand, sel_exact;
    size_t off_kmax = 0, off_dense = 0, off_sidx = 0, off_ssc = 0, off_thr = 0, off_csc = 0, off_cnt = 0,
           off_rep = 0, off_sel = 0, end = 0;   // end: first byte after the selection region
};

bool prefill_uses_mfma(const csa2_plan_params& p, int64_t N, int32_t M) {
    return p.q_idx_dtype == CSA2_BF16 && (p.k_idx_dtype == CSA2_E4M3 || p.k_idx_dtype == CSA2_BF16) && p.d_idx == 64 &&
           N >= 65536 && (int64_t)M * 16 <= N;
}

// Selection region for the top-M positions of B*Q queries, starting at `base`.
int prefill_layout(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, int32_t M, size_t base, PrefillLayout* lay) {
    const csa2_plan_params& p = plan->p;
    lay->M = M;
    lay->rows = (int64_t)B * Q;
    lay->mfma = prefill_uses_mfma(p, N, M);
    size_t off = base;
    if (!lay->mfma) {
        if (int e = plan_select(lay->rows, N, 1024, &lay->sel_exact)) return e;
        lay->off_sel = off;
        off += align_up(lay->sel_exact.data_bytes);
    } else {
        const int64_t rows = lay->rows;
        lay->ns = (N - kSampleStride / 2 + kSampleStride - 1) / kSampleStride;
        // R: f times the expected share of the top-M in the sample, f = 2 or (for M >= 7776) 1.5. The
        // R-th largest sample score t ranks about 64R = f*M among all positions, with a standard
        // deviation of about sqrt(64 f M) positions; a query needs a second, exact pass when t ranks
        // below M, which lies (f - 1) * sqrt(M / (64 f)) deviations away: 4 at f = 2 and M = 2048,
        // 4.6 at f = 1.5 and M = 8192. A smaller f leaves fewer candidates to list and score exactly.
        const int64_t f2 = M >= 7776 ? 3 : 4;  // 2f
        lay->R = (int32_t)((f2 * (int64_t)M * lay->ns + 2 * N - 1) / (2 * N));
        if (lay->R < 1) lay->R = 1;
        lay->nr = (int32_t)(N / 65536 < 1 ? 1 : (N / 65536 > 16 ? 16 : N / 65536));
        lay->nrd = (int32_t)(lay->ns / 2048 < 1 ? 1 : (lay->ns / 2048 > 8 ? 8 : lay->ns / 2048));
        // slots per (query, range): four times the expected share of the ~2M candidates, or - when
        // that still leaves twice the share - as many as keep a query's lists within one select
        // chunk (32,768 slots: one workgroup per query, no row exchanges). A range that overflows
        // sends its query to the exact repair.
        int64_t cap = 4 * 2 * (int64_t)M / lay->nr;
        const int64_t one_chunk = 32768 / lay->nr;
        if (cap > one_chunk && one_chunk >= 2 * 2 * (int64_t)M / lay->nr) cap = one_chunk;
        if (cap < 512) cap = 512;
        lay->cap = (int32_t)((cap + 63) / 64 * 64);
        if (int e = plan_select(rows, lay->ns, 1024, &lay->sel_sample)) return e;
        if (int e = plan_select(rows, (int64_t)lay->nr * lay->cap, 1024, &lay->sel_cand)) return e;
        // the candidates' keys and positions in LDS for at most cand_dense candidates per query (a
        // query with more goes to the exact repair; the lists' slots exceed the candidates ~4 times)
        lay->cand_dense = plan_select_dense(&lay->sel_cand);
        if (int e = plan_select(kRepairRows, N, 1024, &lay->sel_exact)) return e;
        lay->off_kmax = off;
        off += align_up(pf_kmax_floats(B) * 4);
        lay->off_dense = off;                   // sample scores, then candidate lists
        const size_t dense = (size_t)rows * lay->ns * 4, cand = (size_t)rows * lay->nr * lay->cap * 4;
        off += align_up(dense > cand ? dense : cand);
        lay->off_sidx = off;
        off += align_up((size_t)rows * lay->R * 4);
        lay->off_ssc = off;
        off += align_up((size_t)rows * lay->R * 4);
        lay->off_thr = off;
        off += align_up((size_t)rows * 2 * 4);
        lay->off_csc = off;                     // exact scores of the selected candidates
        off += align_up((size_t)rows * M * 4);
        lay->off_cnt = off;
        off += align_up((size_t)rows * lay->nr * 4);
        lay->off_rep = off;                     // [count][pad][rows queue slots][kRepairRows map]
        off += align_up((size_t)(64 + rows + kRepairRows) * 4);
        lay->off_sel = off;
        size_t sel = lay->sel_sample.data_bytes;
        if (lay->sel_cand.data_bytes > sel) sel = lay->sel_cand.data_bytes;
        if (lay->sel_exact.data_bytes > sel) sel = lay->sel_exact.data_bytes;
        off += align_up(sel);
    }
    lay->end = off;
    return OK;
}

// The exact top-M positions (out[0], M = out[0].M) of B*Q prefill queries
// under the causal rule, and with nt = 2 also their top-out[1].M (a prefix of
// the same order, out[1].M <= M). Matrix-core candidates + exact re-scoring +
// verification + repair, or the exact scan select.
int prefill_select(const csa2_plan* plan, const PrefillLayout& lay, const csa2_cache* cache, const void* q_idx,
                   const int64_t* q_pos, int32_t B, int32_t Q, int64_t N, SelOutput* o, int nt, uint8_t* wsb,
                   hipStream_t stream) {
    const csa2_plan_params& p = plan->p;
    const int64_t rows = lay.rows;
    ScanArgs a;
    a.q = q_idx;
    a.k = reinterpret_cast<const uint8_t*>(cache->k_idx);
    a.N = N;
    a.rows_per_seq = Q;
    a.q_pos = q_pos;
    a.q_dtype = p.q_idx_dtype;
    a.k_dtype = p.k_idx_dtype;
    a.d_idx = p.d_idx;
    ScoresArgs none;
    if (!lay.mfma) return run_select(lay.sel_exact, SRC_SCAN, a, none, o, nt, wsb, wsb + lay.off_sel, stream);
    const uint16_t* qb = reinterpret_cast<const uint16_t*>(q_idx);
    float* kmax = reinterpret_cast<float*>(wsb + lay.off_kmax);
    float* dense = reinterpret_cast<float*>(wsb + lay.off_dense);
    int32_t* sidx = reinterpret_cast<int32_t*>(wsb + lay.off_sidx);
    float* ssc = reinterpret_cast<float*>(wsb + lay.off_ssc);
    float* thr = reinterpret_cast<float*>(wsb + lay.off_thr);
    float* csc = reinterpret_cast<float*>(wsb + lay.off_csc);
    uint32_t* cnt = reinterpret_cast<uint32_t*>(wsb + lay.off_cnt);
    uint32_t* rep_count = reinterpret_cast<uint32_t*>(wsb + lay.off_rep);
    int32_t* rep_rows = reinterpret_cast<int32_t*>(wsb + lay.off_rep) + 64;
    int32_t* rep_map = rep_rows + rows;
    int32_t* cand = reinterpret_cast<int32_t*>(wsb + lay.off_dense);   // reuses the sample scores
    uint32_t* status = reinterpret_cast<uint32_t*>(wsb);
    if (int e = launch_pf_kmax(a.k, p.k_idx_dtype, B, N, kmax, stream)) return e;
    PfTiles t;
    t.q = qb;
    t.k = a.k;
    t.N = N;
    t.B = B;
    t.Q = Q;
    t.q_pos = q_pos;
    t.key_off = kSampleStride / 2;
    t.key_stride = kSampleStride;
    t.nkeys = lay.ns;
    t.nranges = lay.nrd;
    t.dense = dense;
    if (int e = launch_pf_tiles(t, p.k_idx_dtype, true, stream)) return e;
    if (lay.ns <= kRthMaxSamples) {
        // the R-th largest sample score of each row (exact) straight from the dense scores
        if (int e = launch_pf_rth(dense, rows, (int32_t)lay.ns, lay.R, ssc, stream)) return e;
        if (int e = launch_pf_thresholds(qb, rows, Q, ssc, 1, kmax, thr, rep_count, stream)) return e;
    } else {
        ScoresArgs sa;
        sa.scores = dense;
        sa.stride = lay.ns;
        SelOutput so{sidx, ssc, lay.R, lay.R};
        if (int e = run_select(lay.sel_sample, SRC_SCORES, a, sa, &so, 1, wsb, wsb + lay.off_sel, stream)) return e;
        if (int e = launch_pf_thresholds(qb, rows, Q, ssc, lay.R, kmax, thr, rep_count, stream)) return e;
    }
    t.key_off = 0;
    t.key_stride = 1;
    t.nkeys = N;
    t.nranges = lay.nr;
    t.dense = nullptr;
    t.thr = thr;
    t.cand = cand;
    t.cap = lay.cap;
    t.cnt = cnt;
    if (int e = launch_pf_tiles(t, p.k_idx_dtype, false, stream)) return e;
    ScanArgs ca = a;
    ca.cand = cand;
    ca.cnt = cnt;
    ca.nranges = lay.nr;
    ca.cap = lay.cap;
    SelOutput oc[2] = {o[0], nt > 1 ? o[1] : o[0]};
    oc[0].score = csc;                          // the M-th exact score decides the verification
    if (int e = run_select(lay.sel_cand, SRC_CAND, ca, none, oc, nt, wsb, wsb + lay.off_sel, stream)) return e;
    if (int e = launch_pf_verify(rows, lay.nr, lay.cap, lay.cand_dense, cnt, csc, thr, q_pos, N, lay.M, rep_rows, rep_count,
                                 (int32_t)rows, status, stream))
        return e;
    // queued rows: the first kRepairRows by the multi-workgroup exact select, any others by one
    // workgroup each per target (that kernel returns at once when the queue is no longer)
    if (int e = launch_pf_repair_map(rep_rows, rep_count, 0, kRepairRows, rep_map, stream)) return e;
    ScanArgs ra = a;
    ra.rowmap = rep_map;
    if (int e = run_select(lay.sel_exact, SRC_SCAN, ra, none, o, nt, wsb, wsb + lay.off_sel, stream)) return e;
    for (int j = 0; j < nt; ++j)
        if (int e = launch_pf_repair_rest(qb, a.k, p.k_idx_dtype, N, Q, q_pos, rep_rows, rep_count, kRepairRows,
                                          o[j].M, o[j].idx, stream))
            return e;
    return OK;
}

AttnArgs prefill_attn_args(const csa2_plan_params& p, const csa2_cache* c, const uint16_t* q, int64_t rows, int32_t Q,
                           int64_t N, const int32_t* idx, float* out) {
    AttnArgs at;
    at.q = q;
    at.rows = rows;
    at.rows_per_seq = Q;
    at.H = p.H;
    at.d = p.d;
    at.k_codes = c->k_codes;
    at.k_scales = c->k_scales;
    at.v_codes = c->v_codes;
    at.v_scales = c->v_scales;
    at.N = N;
    at.code_stride = c->code_stride_bytes;
    at.scale_stride = c->scale_stride_bytes;
    at.idx = idx;
    at.idx_stride = p.K;
    at.K = p.K;
    at.scale = p.softmax_scale;
    at.out = out;
    at.mx = p.kv_format == CSA2_KV_MXFP4;
    return at;
}

// Full-layer prefill workspace: selection region (top-K), then the attention data.
int full_prefill_layout(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, PrefillLayout* lay, size_t* off_attn,
                        size_t* total) {
    if (int e = prefill_layout(plan, B, Q, N, plan->p.K, align_up(kCtrlBytes), lay)) return e;
    *off_attn = lay->end;
    *total = lay->end + align_up(attn_data_bytes(lay->rows, plan->p.K));
    return OK;
}

// Prefill through the whole plan: the Full layers' selection region (sized
// for top-P when a group needs a pool, else top-K), the per-query pools, the
// per-query positions, the Reindex select's data region and the attention's.
struct PlanPrefillLayout {
    PrefillLayout full;                         // selection of a Full layer that picks a pool (M = P), or top-K
    PrefillLayout full_k;                       // selection of a Full layer without a pool (M = K)
    SelPlan reidx;                              // Reindex selection: top-K of each query's pool
    size_t off_pool = 0, off_idx = 0, off_reidx = 0, off_attn = 0, total = 0;
};

int plan_prefill_layout(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, PlanPrefillLayout* lay) {
    const csa2_plan_params& p = plan->p;
    const size_t base = align_up(kCtrlBytes);
    bool any_pool = false;
    for (uint8_t g : plan->group_pool) any_pool |= g != 0;
    size_t end = base;
    if (any_pool) {
        if (int e = prefill_layout(plan, B, Q, N, p.P, base, &lay->full)) return e;
        end = lay->full.end;
    }
    if (int e = prefill_layout(plan, B, Q, N, p.K, base, &lay->full_k)) return e;
    if (lay->full_k.end > end) end = lay->full_k.end;
    const int64_t rows = (int64_t)B * Q;
    size_t off = end;
    if (any_pool) {
        lay->off_pool = off;
        off += align_up((size_t)rows * p.P * 4);
        if (int e = plan_select(rows, p.P, 1024, &lay->reidx)) return e;
        lay->off_reidx = off;
        off += align_up(lay->reidx.data_bytes);
    }
    lay->off_idx = off;
    off += align_up((size_t)rows * p.K * 4);
    lay->off_attn = off;
    off += align_up(attn_data_bytes(rows, p.K));
    lay->total = off;
    return OK;
}

}  // namespace

extern "C" {

int csa2_prefill_workspace_bytes(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, size_t* bytes) {
    g_err.clear();
    if (!plan || !bytes) return fail(INVALID, "csa2_prefill_workspace_bytes: null pointer");
    if (B < 1 || Q < 1 || N < 1) return fail(INVALID, "csa2_prefill_workspace_bytes: sizes must be >= 1");
    PrefillLayout lay;
    size_t off_attn = 0, total = 0;
    if (int e = full_prefill_layout(plan, B, Q, N, &lay, &off_attn, &total)) return e;
    *bytes = total;
    return OK;
}

int csa2_prefill_full(const csa2_plan* plan, const csa2_cache* cache, const void* q_idx, const uint16_t* q,
                      const int64_t* q_pos, int32_t B, int32_t Q, int64_t N, int32_t* idx_out, float* out, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
    g_err.clear();
    if (!plan || !cache) return fail(INVALID, "csa2_prefill_full: null pointer");
    if (B < 1 || Q < 1 || N < 1) return fail(INVALID, "csa2_prefill_full: sizes must be >= 1");
    const csa2_plan_params& p = plan->p;
    if (int e = check_attn(q, p.H, p.d, cache->k_codes, cache->k_scales, cache->v_codes, cache->v_scales, N,
                           cache->code_stride_bytes, cache->scale_stride_bytes, p.K, "csa2_prefill_full",
                           p.kv_format == CSA2_KV_MXFP4))
        return e;
    if (int e = check_scan(q_idx, p.q_idx_dtype, cache->k_idx, p.k_idx_dtype, p.d_idx, "csa2_prefill_full")) return e;
    if (!q_pos || !idx_out || !out) return fail(INVALID, "csa2_prefill_full: null pointer");
    PrefillLayout lay;
    size_t off_attn = 0, total = 0;
    if (int e = full_prefill_layout(plan, B, Q, N, &lay, &off_attn, &total)) return e;
    if (int e = check_ws(ws, ws_bytes, total, "csa2_prefill_full")) return e;
    if (lay.mfma && !aligned(q_idx, 16)) return fail(INVALID, "csa2_prefill_full: indexer query must be 16-byte aligned");
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    SelOutput o{idx_out, nullptr, p.K, p.K};
    if (int e = prefill_select(plan, lay, cache, q_idx, q_pos, B, Q, N, &o, 1, wsb, stream)) return e;
    const AttnArgs at = prefill_attn_args(p, cache, q, lay.rows, Q, N, idx_out, out);
    return launch_attn(at, wsb, wsb + off_attn, total - off_attn, stream);
}

int csa2_plan_prefill_workspace_bytes(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, size_t* bytes) {
    g_err.clear();
    if (!plan || !bytes) return fail(INVALID, "csa2_plan_prefill_workspace_bytes: null pointer");
    if (B < 1 || Q < 1 || N < 1) return fail(INVALID, "csa2_plan_prefill_workspace_bytes: sizes must be >= 1");
    PlanPrefillLayout lay;
    if (int e = plan_prefill_layout(plan, B, Q, N, &lay)) return e;
    *bytes = lay.total;
    return OK;
}

int csa2_plan_run_prefill(const csa2_plan* plan, const csa2_cache* cache, const csa2_prefill_io* io,
                          const int64_t* q_pos, int32_t B, int32_t Q, int64_t N, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
    g_err.clear();
    const char* who = "csa2_plan_run_prefill";
    if (!plan || !cache || !io || !q_pos) return fail(INVALID, std::string(who) + ": null pointer");
    if (B < 1 || Q < 1 || N < 1) return fail(INVALID, std::string(who) + ": sizes must be >= 1");
    const csa2_plan_params& p = plan->p;
    if (plan->has_reindex && p.P > N) return fail(INVALID, std::string(who) + ": pool size P exceeds N");
    if (p.swa_window > 0) return fail(INVALID, std::string(who) + ": the sliding window is a decode-time branch here");
    const int L = (int)plan->modes.size();
    for (int32_t gi = 0; gi < plan->groups; ++gi) {
        const csa2_cache* c = &cache[gi];
        if (int e = check_attn(io[0].q, p.H, p.d, c->k_codes, c->k_scales, c->v_codes, c->v_scales, N,
                               c->code_stride_bytes, c->scale_stride_bytes, p.K, who, p.kv_format == CSA2_KV_MXFP4))
            return e;
    }
    for (int l = 0; l < L; ++l) {
        if (!io[l].q || !io[l].out) return fail(INVALID, std::string(who) + ": layer " + std::to_string(l) + " needs q and out");
        if (plan->modes[l] != CSA2_REUSE) {
            const csa2_cache* c = &cache[plan->group[l]];
            if (int e = check_scan(io[l].q_idx, p.q_idx_dtype, c->k_idx, p.k_idx_dtype, p.d_idx, who)) return e;
            if (!aligned(io[l].q_idx, 16)) return fail(INVALID, std::string(who) + ": indexer queries must be 16-byte aligned");
        }
    }
    PlanPrefillLayout lay;
    if (int e = plan_prefill_layout(plan, B, Q, N, &lay)) return e;
    if (int e = check_ws(ws, ws_bytes, lay.total, who)) return e;
    uint8_t* wsb = reinterpret_cast<uint8_t*>(ws);
    const int64_t rows = (int64_t)B * Q;
    int32_t* pool = reinterpret_cast<int32_t*>(wsb + lay.off_pool);
    const int32_t* cur_idx = nullptr;
    for (int l = 0; l < L; ++l) {
        const int32_t mode = plan->modes[l];
        const int32_t gi = plan->group[l];
        const csa2_cache* gc = &cache[gi];
        int32_t* idx_dst = io[l].idx_out ? io[l].idx_out : reinterpret_cast<int32_t*>(wsb + lay.off_idx);
        if (mode == CSA2_FULL) {
            if (plan->group_pool[gi]) {         // the group's per-query pools and top-K in one selection
                SelOutput o[2] = {SelOutput{pool, nullptr, p.P, p.P}, SelOutput{idx_dst, nullptr, p.K, p.K}};
                if (int e = prefill_select(plan, lay.full, gc, io[l].q_idx, q_pos, B, Q, N, o, 2, wsb, stream)) return e;
            } else {
                SelOutput o{idx_dst, nullptr, p.K, p.K};
                if (int e = prefill_select(plan, lay.full_k, gc, io[l].q_idx, q_pos, B, Q, N, &o, 1, wsb, stream))
                    return e;
            }
            cur_idx = idx_dst;
        } else if (mode == CSA2_REINDEX) {      // each query's top-K of its own pool, with this layer's query
            ScanArgs a;
            a.q = io[l].q_idx;
            a.k = reinterpret_cast<const uint8_t*>(gc->k_idx);
            a.N = N;
            a.rows_per_seq = Q;
            a.pool = pool;
            a.q_dtype = p.q_idx_dtype;
            a.k_dtype = p.k_idx_dtype;
            a.d_idx = p.d_idx;
            ScoresArgs none;
            SelOutput o{idx_dst, nullptr, p.K, p.K};
            if (int e = run_select(lay.reidx, SRC_POOL, a, none, &o, 1, wsb, wsb + lay.off_reidx, stream)) return e;
            cur_idx = idx_dst;
        }
        const AttnArgs at = prefill_attn_args(p, gc, io[l].q, rows, Q, N, cur_idx, io[l].out);
        if (int e = launch_attn(at, wsb, wsb + lay.off_attn, lay.total - lay.off_attn, stream)) return e;
    }
    return OK;
}

}  // extern "C"
