// Host-side interfaces between the C ABI (api.cpp) and the kernel launchers.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include <string>

namespace csa2 {

// Status codes mirror csa2.h.
enum Status : int { OK = 0, INVALID = 1, DTYPE = 2, BAD_PLAN = 3, WORKSPACE = 4, HIP = 5, DEVICE = 6 };

// Set the thread-local error message; returns `code` for convenience.
int fail(int code, const std::string& msg);
int hip_fail(hipError_t e, const char* what);

// Device facts cached per device ordinal.
struct DeviceInfo {
    int device = -1;
    int num_cus = 0;
    size_t max_lds = 0;     // bytes of LDS one workgroup may allocate
};
int device_info(DeviceInfo* out);

// ------------------------------------------------------------ workspaces
// Every workspace starts with one control region whose layout is the same for
// every call and every problem shape: a header, the select kernels' per-row
// barrier and exit counters and histogram accumulators, and the attention
// kernel's per-row merge counters. Each call leaves the words it used zero,
// so one zero-filled buffer can serve calls of any kind and shape in turn.
// The region of data that a call writes (lists, partial results, outputs
// kept in the workspace) follows it; data never lands on a control word.
constexpr int kCtrlHeaderWords = 64;        // [0] device status word
constexpr int kSelCtrlRowWords = 8256;      // barrier, exit, 2048 + 2*2048 + 2*1024 histogram bins, padded
constexpr int kSelCtrlRows = 256;           // rows per select launch (at most one workgroup per CU)
constexpr int kAttnCtrlWords = 256;         // rows whose attention is split over workgroups (< 256)
constexpr size_t kCtrlWords = kCtrlHeaderWords + (size_t)kSelCtrlRows * kSelCtrlRowWords + kAttnCtrlWords;
constexpr size_t kCtrlBytes = kCtrlWords * 4;
constexpr size_t kSelCtrlOffsetWords = kCtrlHeaderWords;
constexpr size_t kAttnCtrlOffsetWords = kCtrlHeaderWords + (size_t)kSelCtrlRows * kSelCtrlRowWords;

// ------------------------------------------------------------- selection
// Geometry of one selection problem: `rows` rows of `n` entries split into S
// chunks of `chunk` entries, one workgroup per chunk, all chunks of a row
// co-resident; `rows_per_launch` rows per cooperative launch.
struct SelPlan {
    int64_t rows = 0, n = 0;
    int32_t S = 1, chunk = 0, chunk_pad = 0, rows_per_launch = 0, launches = 0;
    int32_t row_words = 0;          // data words per row in the workspace
    size_t lds_bytes = 0;
    size_t data_bytes = 0;          // data region bytes (rows_per_launch rows)
    size_t ws_bytes = 0;            // control region + data region
    int32_t skew = 0;               // even chunks take chunk + skew entries, odd ones chunk - skew
    int32_t dense_cap = 0;          // > 0: a source that stores only its valid entries densely holds at
                                    // most this many per row (LDS sized for them, not for the chunk)
};

enum SelSource : int { SRC_SCORES = 0, SRC_SCAN = 1, SRC_POOL = 2, SRC_CAND = 3 };

// Plan a selection. `min_chunk` bounds how finely a row may be split.
int plan_select(int64_t rows, int64_t n, int32_t min_chunk, SelPlan* out);
// For a one-chunk candidate selection whose keys and positions would not both
// fit in LDS at the chunk's size: size LDS for the most valid entries that do
// (p->dense_cap); rows with more valid entries are left to the caller (the
// select writes nothing for them). Returns the number of valid entries a row
// may hold: all n of them unless a dense capacity is set.
int64_t plan_select_dense(SelPlan* p);

struct SelOutput {
    int32_t* idx = nullptr;         // [rows][stride] positions
    float* score = nullptr;         // optional selected scores
    int64_t stride = 0;
    int32_t M = 0;
};

// An attention fused into a selection kernel, for an FP4 cache with E4M3
// scales (128 channels, at most 16 heads, no sliding window).
struct AttnFuse {
    const uint16_t* q;                          // [rows][H][128] bf16 attention queries
    const uint8_t *k_codes, *k_scales, *v_codes, *v_scales;   // sequence s starts at + s * N * stride
    int64_t N, cs, ss;                          // positions per sequence, code and scale row strides
    int32_t H, rows_per_seq;
    float scale;                                // softmax scale
    float* out;                                 // [rows][H][128] fp32
    float* parts;                               // [launch rows][S][kAttnPartFloats] partial states
};
constexpr int kAttnPartFloats = 16 * 128 + 2 * 16;   // one partial state: acc [16][128], (max, sum) [16][2]

struct ScanArgs {                   // indexer keys scored inside the select kernel
    const void* q = nullptr;        // [rows][d_idx] indexer queries (q_dtype)
    const uint8_t* k = nullptr;     // [seqs][N][d_idx] keys (k_dtype)
    int64_t N = 0;                  // positions per sequence
    int32_t rows_per_seq = 1;       // row r reads sequence r / rows_per_seq
    const int64_t* q_pos = nullptr; // causal limit per row, or null
    const int32_t* pool = nullptr;  // SRC_POOL: [rows][n] positions to score
    const int32_t* cand = nullptr;  // SRC_CAND: [rows][nranges][cap] positions, valid below cnt
    const uint32_t* cnt = nullptr;  //           [rows][nranges]
    int32_t nranges = 0, cap = 0;
    const int32_t* rowmap = nullptr;// scan sources: launch row -> query row (-1: none), or null
    int32_t q_dtype = 0, k_dtype = 0, d_idx = 64;
    const AttnFuse* attn = nullptr; // SRC_SCAN: attend to the last target's positions in the same launch
};
// Workspace bytes of the partial states of a select launch with the attention fused in.
size_t select_fused_part_bytes(const SelPlan& p);

struct ScoresArgs {                 // precomputed scores
    const float* scores = nullptr;
    int64_t stride = 0;
    const int32_t* cand = nullptr;  // [rows][n] positions or null
};

// Run a planned selection for all rows (several launches if needed).
// nt = number of targets (1 or 2, out[0].M >= out[1].M).
// ws_ctrl: start of the workspace (its control region); ws_data: this call's
// data region of p.data_bytes bytes.
int run_select(const SelPlan& p, int source, const ScanArgs& scan, const ScoresArgs& sc,
               const SelOutput* out, int nt, void* ws_ctrl, void* ws_data, hipStream_t stream);

// Reindex selection (pool of at most 16,384 entries per row): score the pool
// and select top-K with one all-keys exchange per row (poolsel.hip).
struct PoolSelPlan {
    int64_t rows = 0;
    int32_t n = 0, n4 = 0, S = 1, rows_per_launch = 0;
    size_t data_bytes = 0;          // published keys, rows_per_launch rows of n4 words
};
struct PoolSelArgs {
    const void* q = nullptr;        // [rows][d_idx] indexer queries (q_dtype)
    const uint8_t* k = nullptr;     // [rows][N][d_idx] keys (k_dtype); row r reads sequence r
    int64_t N = 0;
    const int32_t* pool = nullptr;  // [rows][n] ascending positions
    int32_t q_dtype = 0, k_dtype = 0, d_idx = 64, K = 0;
    int32_t* idx = nullptr;         // [rows][idx_stride] ascending positions, -1 padding
    int64_t idx_stride = 0;
    float* score = nullptr;         // optional selected scores
    const AttnFuse* attn = nullptr; // attend to the selected positions in the same launch
};
constexpr int64_t kPoolSelMaxN = 16384;
int plan_pool_select(int64_t rows, int64_t n, PoolSelPlan* out);
// Data bytes of a pool select with the attention fused in (the key buffer, then the partial states).
size_t pool_select_fused_bytes(const PoolSelPlan& p);
int run_pool_select(const PoolSelPlan& p, const PoolSelArgs& a, void* ws_ctrl, void* ws_data, size_t data_bytes,
                    hipStream_t stream);

// --------------------------------------------------------- prefill indexer
struct PfTiles {
    const uint16_t* q = nullptr;    // [B*Q][64] bf16 indexer queries
    const uint8_t* k = nullptr;     // [B][N][64] indexer keys
    int64_t N = 0;
    int32_t B = 0, Q = 0;
    const int64_t* q_pos = nullptr;
    int64_t key_off = 0, key_stride = 1, nkeys = 0;
    int32_t nranges = 1;
    float* dense = nullptr;         // dense mode output [B*Q][nkeys]
    const float* thr = nullptr;     // candidate mode: [B*Q][2] (lo, check bound)
    int32_t* cand = nullptr;
    int32_t cap = 0;
    uint32_t* cnt = nullptr;
};
size_t pf_kmax_floats(int32_t B);
int launch_pf_kmax(const uint8_t* k, int k_dtype, int32_t B, int64_t N, float* partial, hipStream_t stream);
int launch_pf_tiles(const PfTiles& t, int k_dtype, bool dense, hipStream_t stream);
// R-th largest of each of `rows` rows of n sample scores (n <= 16384) -> tval[rows].
int launch_pf_rth(const float* dense, int64_t rows, int32_t n, int32_t R, float* tval, hipStream_t stream);
int launch_pf_thresholds(const uint16_t* q, int64_t rows, int32_t Q, const float* sel, int32_t R,
                         const float* kmax_partial, float* thr, uint32_t* repair_count, hipStream_t stream);
int launch_pf_verify(int64_t rows, int32_t nranges, int32_t cap, int64_t dense_cap, const uint32_t* cnt, const float* sel,
                     const float* thr, const int64_t* q_pos, int64_t N, int32_t K, int32_t* repair_rows,
                     uint32_t* repair_count, int32_t repair_cap, uint32_t* status, hipStream_t stream);
// Exact top-K of the queued queries in queue slots [first, count): one workgroup per query.
int launch_pf_repair_rest(const uint16_t* q, const uint8_t* k, int k_dtype, int64_t N, int32_t Q,
                          const int64_t* q_pos, const int32_t* repair_rows, const uint32_t* repair_count, int32_t first,
                          int32_t K, int32_t* idx_out, hipStream_t stream);
int launch_pf_repair_map(const int32_t* repair_rows, const uint32_t* repair_count, int32_t first, int32_t n,
                         int32_t* map, hipStream_t stream);

// ---------------------------------------------------------- other kernels
int launch_quant(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride, uint8_t* codes,
                 int64_t cs, uint8_t* scales, int64_t ss, hipStream_t stream);
int launch_dequant(const uint8_t* codes, int64_t cs, const uint8_t* scales, int64_t ss, int64_t rows,
                   int32_t C, uint16_t* y, int64_t y_stride, hipStream_t stream);
int launch_quant_mx(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride, uint8_t* codes, int64_t cs,
                    uint8_t* scales, int64_t ss, hipStream_t stream);
int launch_dequant_mx(const uint8_t* codes, int64_t cs, const uint8_t* scales, int64_t ss, int64_t rows, int32_t C,
                      uint16_t* y, int64_t y_stride, hipStream_t stream);
int launch_kv_project(const uint16_t* h, int64_t T, int32_t D, int64_t hs, const uint16_t* wt, int64_t wsd, bool mx,
                      uint8_t* codes, int64_t cs, uint8_t* scales, int64_t ss, uint16_t* cout, int64_t cos,
                      hipStream_t stream);
int launch_index_dense(const ScanArgs& a, int32_t B, int32_t Q, float* scores, hipStream_t stream);
int launch_index_pool(const ScanArgs& a, int32_t B, int32_t P, float* scores, hipStream_t stream);

struct AttnArgs {
    const uint16_t* q = nullptr;    // [rows][H][d]
    int64_t rows = 0;               // B*Q query rows
    int32_t rows_per_seq = 1;       // row r reads sequence r / rows_per_seq
    int32_t H = 0, d = 128;
    const uint8_t *k_codes = nullptr, *k_scales = nullptr, *v_codes = nullptr, *v_scales = nullptr;
    int64_t N = 0, code_stride = 0, scale_stride = 0;
    const int32_t* idx = nullptr;   // [rows][idx_stride]
    int64_t idx_stride = 0;
    int32_t K = 0;
    float scale = 0.f;
    float* out = nullptr;           // [rows][H][d]
    bool mx = false;                // cache format: E4M3 scale per 16 channels, or MXFP4 (E8M0 per 32)
    const uint16_t* win_k = nullptr;// sliding window: row r's Wn bf16 K rows at win_k + r*win_rs (d each)
    const uint16_t* win_v = nullptr;
    int64_t win_rs = 0;
    int32_t Wn = 0;                 // window rows per query row (0: no window)
    const int32_t* win_len = nullptr;   // [rows] valid window rows, or null (all Wn)
};
size_t attn_data_bytes(int64_t rows, int32_t K, int32_t W = 0);  // data region of one attention call
int launch_attn(const AttnArgs& a, void* ws_ctrl, void* ws_data, size_t data_bytes, hipStream_t stream);
// The same with the merge counters (kAttnCtrlWords words, zero between calls) and the partial
// states given directly.
int launch_attn_scratch(const AttnArgs& a, uint32_t* counters, void* parts, size_t parts_bytes, hipStream_t stream);

// Host-side argument checks of the attention call (api.cpp).
int check_attn(const uint16_t* q, int32_t H, int32_t d, const uint8_t* kc, const uint8_t* ks, const uint8_t* vc,
               const uint8_t* vs, int64_t N, int64_t cs, int64_t ss, int32_t K, const char* who, bool mx);

}  // namespace csa2
