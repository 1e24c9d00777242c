/*
 * csa2.h - C ABI of libcsa2: the decode-time CSA2 step (Compressed Sparse
 * Attention 2) over an FP4 E2M1 main KV cache with one E4M3 scale per 16
 * channels, for AMD Instinct MI355X (gfx950).
 *
 * Pages this interface follows (titles and sections):
 *   [ezic]     "DeepSeek-V4.1-Flash: KVキャッシュ1トークン890バイト" (ai2.x.ezic.info),
 *              "先に要点だけ" and "KVを捨てる、共有する、作り直す".
 *   [zaikei]   "DeepSeek-V4.1-Flash、KVキャッシュを約4分の1に圧縮" (zaikei.co.jp),
 *              "■CSA2とFP4でキャッシュを圧縮".
 *   [jiwasawa] "DeepSeek-V4.1-Flash" report digest (jiwasawa.github.io),
 *              "Compressed Sparse Attention 2 (CSA2) による極限のKV cache圧縮" and
 *              "FP4 メイン KV Cache と SWA Bounded Replay".
 *
 * Conventions for every call:
 *   - Buffers named as device buffers are device pointers owned by the caller;
 *     the library never allocates, frees or retains device memory. Scratch
 *     comes from a caller-provided workspace sized by the matching
 *     *_workspace_bytes call.
 *   - Workspaces must be zero-filled before their first use. Every workspace
 *     starts with a control region of fixed layout (about 8 MiB: counters and
 *     histogram accumulators), and every call that completes normally leaves
 *     it zero again, so one zero-fill at allocation is enough and one buffer
 *     may serve calls of any kind and shape in turn, as long as it is large
 *     enough for each. One workspace must not be used by two calls that can
 *     run at the same time.
 *   - All work is enqueued on `stream` (a hipStream_t; NULL = default stream).
 *     No call synchronizes the host with the device.
 *   - Arguments are validated on the host before any HIP call. Device data
 *     (positions, code bytes) is not validated except where stated; positions
 *     outside [0, N) are treated as padding by every kernel that reads them.
 *   - Return value: CSA2_OK or one of the error codes below; on error nothing
 *     was enqueued (except CSA2_ERR_HIP, reported by the launch itself) and
 *     csa2_last_error() describes the failure (thread-local string).
 *   - Element counts and strides are in elements of the named dtype unless
 *     the argument name ends in _bytes or the comment says bytes.
 *   - Selection kernels (csa2_topk, csa2_plan_run_decode, csa2_prefill_full)
 *     split a row over several workgroups that wait for each other, at most
 *     one workgroup per compute unit, so they expect the compute units to be
 *     free when they start (kernels of other streams that hold compute units
 *     can delay them). Every such wait is bounded: after 2^20 polls it gives
 *     up, sets bit 0 of the workspace's first 32-bit word (the status word)
 *     and lets the kernel finish; the outputs of that call are then
 *     unspecified. The status word is never cleared by the library.
 *
 * Storage formats (readings where the pages are silent are marked R):
 *   FP4 codes: one byte holds two E2M1 codes; channel 2j in the low nibble,
 *     channel 2j+1 in the high nibble of byte j (R). Code bit 3 is the sign;
 *     magnitudes {0, .5, 1, 1.5, 2, 3, 4, 6} ([jiwasawa] FP4: OCP E2M1).
 *   Scales: one E4M3FN byte (bias 7, max 448, 0x7F/0xFF = NaN) per 16
 *     channels ([ezic] key points), byte g covers channels 16g..16g+15.
 *   Main KV cache of a sequence with N positions: for position t, the K codes
 *     start at k_codes + t*code_stride_bytes, the K scales at
 *     k_scales + t*scale_stride_bytes, likewise for V. Sequence b starts at
 *     position b*N. The recommended record layout is code_stride = 128 with
 *     v_codes = k_codes + 64 and scale_stride = 16 with v_scales = k_scales + 8:
 *     144 bytes per token for K and V of 128 channels.
 */
#ifndef CSA2_H_
#define CSA2_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define CSA2_OK 0
#define CSA2_ERR_INVALID_ARG 1      /* null pointer, bad size, stride or alignment */
#define CSA2_ERR_UNSUPPORTED_DTYPE 2
#define CSA2_ERR_BAD_PLAN 3         /* layer modes violate the plan rules */
#define CSA2_ERR_WORKSPACE 4        /* workspace null, misaligned or too small */
#define CSA2_ERR_HIP 5              /* a HIP call failed; see csa2_last_error() */
#define CSA2_ERR_DEVICE 6           /* the device reported a failed in-kernel wait */

/* Element types of indexer queries and keys. */
#define CSA2_F32 0                  /* IEEE fp32 */
#define CSA2_BF16 1                 /* bfloat16, stored as uint16 bit patterns */
#define CSA2_E4M3 2                 /* OCP E4M3FN byte, no scale */

/* Main KV cache formats: FP4 E2M1 with one E4M3 scale per 16 channels
 * ([ezic] key points), or MXFP4: FP4 E2M1 with one E8M0 (power-of-two) scale
 * per 32 channels, the OCP MX format ([jiwasawa] FP4 main KV cache). */
#define CSA2_KV_FP4_E4M3 0
#define CSA2_KV_MXFP4 1

/* Layer modes ([zaikei] CSA2とFP4; [jiwasawa] CSA2). */
#define CSA2_FULL 0
#define CSA2_REINDEX 1
#define CSA2_REUSE 2

/* Message for the last failing call on this thread ("" if none). */
const char* csa2_last_error(void);

/* Library version as major*10000 + minor*100 + patch. */
int csa2_version(void);

/*
 * kv_quant_fp4 - S1: quantize bf16 rows to FP4 E2M1 codes with one E4M3 scale
 * per 16 channels ([ezic] key points and "KVを捨てる、共有する、作り直す";
 * [zaikei] CSA2とFP4: the main KV cache is stored in FP4 E2M1).
 *
 * Per row r and 16-channel group g (R: the pages do not say how the scale is
 * chosen): amax = max |x|; S = RNE_E4M3(amax / 6) saturating at 448; if S is
 * 0 every code of the group is 0x0, else code_i = RNE_E2M1(x_i / S) with the
 * sign of x_i kept (a negative value rounding to zero gives 0x8).
 *
 *   x             device, bf16 bit patterns; row r starts at x + r*x_stride
 *   rows          number of rows (>= 0; 0 is a no-op)
 *   C             channels per row, a positive multiple of 16
 *   x_stride      elements between row starts (>= C)
 *   codes         device; row r's C/2 code bytes start at codes + r*code_stride_bytes
 *   scales        device; row r's C/16 scale bytes start at scales + r*scale_stride_bytes
 * Alignment: x and x_stride*2 bytes to 16 bytes; codes and code_stride_bytes
 * to 8 bytes. Inputs must be finite (NaN/Inf give unspecified codes).
 */
int kv_quant_fp4(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride,
                 uint8_t* codes, int64_t code_stride_bytes,
                 uint8_t* scales, int64_t scale_stride_bytes, hipStream_t stream);

/*
 * kv_dequant_fp4 - inverse image of kv_quant_fp4 ([zaikei] CSA2とFP4: the cache
 * is dequantized before attention): y = E2M1(code) * E4M3(scale), which is
 * exact in bf16. Same layouts and alignment rules as kv_quant_fp4 (y like x).
 */
int kv_dequant_fp4(const uint8_t* codes, int64_t code_stride_bytes,
                   const uint8_t* scales, int64_t scale_stride_bytes,
                   int64_t rows, int32_t C, uint16_t* y, int64_t y_stride, hipStream_t stream);

/*
 * kv_quant_mxfp4 - S1 in the MXFP4 reading of the format ([jiwasawa] "FP4
 * メイン KV Cache と SWA Bounded Replay": OCP-standard MXFP4, E2M1 elements):
 * per row r and 32-channel block b, the shared scale is X = 2^(floor(log2(
 * amax)) - 2) stored as the E8M0 byte floor(log2(amax)) - 2 + 127 clamped to
 * [0, 254] (byte 0 for an all-zero block); code_i = RNE_E2M1(x_i / X) with
 * saturation at 6 and the sign of x_i kept (R).
 *
 *   x             device, bf16; row r starts at x + r*x_stride (16-byte aligned rows)
 *   C             channels per row, a positive multiple of 32
 *   codes         device; row r's C/2 code bytes (nibble order as kv_quant_fp4) at
 *                 codes + r*code_stride_bytes (16-byte aligned rows)
 *   scales        device; row r's C/32 E8M0 bytes at scales + r*scale_stride_bytes
 * Inputs must be finite.
 */
int kv_quant_mxfp4(const uint16_t* x, int64_t rows, int32_t C, int64_t x_stride,
                   uint8_t* codes, int64_t code_stride_bytes,
                   uint8_t* scales, int64_t scale_stride_bytes, hipStream_t stream);

/*
 * kv_dequant_mxfp4 - inverse image of kv_quant_mxfp4: y = E2M1(code) *
 * 2^(scale - 127), exact in bf16 (scale byte 0xFF gives NaN). Code rows
 * 4-byte aligned, y rows 16-byte aligned.
 */
int kv_dequant_mxfp4(const uint8_t* codes, int64_t code_stride_bytes,
                     const uint8_t* scales, int64_t scale_stride_bytes,
                     int64_t rows, int32_t C, uint16_t* y, int64_t y_stride, hipStream_t stream);

/*
 * csa2_kv_project - the KV write path ([jiwasawa] "Causal Encoder-Decoder
 * (CED) アーキテクチャ", its projection equation; [zaikei] "■CEDで入力処理の
 * 計算量を削減"): a decoder layer's global KV rows are projected from the
 * encoder's last hidden state, C = H W, and stored in FP4 in the same kernel.
 *
 * R: C has 256 channels, one shared KV head with K in channels 0..127 and V in
 * 128..255; each element is the product-sum (bf16 inputs, fp32 accumulation)
 * rounded once to bf16 (nearest even), then quantized per group exactly as
 * kv_quant_fp4 (kv_format CSA2_KV_FP4_E4M3) or kv_quant_mxfp4 (CSA2_KV_MXFP4)
 * would quantize that bf16 row.
 *
 *   h       device [T][D] bf16 (row r at h + r*h_stride), D a positive multiple of 64
 *   w_t     device [256][D] bf16: W transposed, row c holds the D weights of output
 *           channel c (row c at w_t + c*w_stride)
 *   codes   device; token r's 128 code bytes [K 64 | V 64] at codes + r*code_stride_bytes
 *           (8-byte aligned rows; 16-byte for MXFP4) - the main KV cache record layout
 *   scales  device; token r's scale bytes [K | V] (8 + 8 E4M3, or 4 + 4 E8M0) at
 *           scales + r*scale_stride_bytes
 *   c_out   device [T][256] bf16 (row r at c_out + r*c_stride), the rounded C itself, or NULL
 * h, w_t and c_out rows must be 16-byte aligned.
 */
int csa2_kv_project(const uint16_t* h, int64_t T, int32_t D, int64_t h_stride,
                    const uint16_t* w_t, int64_t w_stride, int32_t kv_format,
                    uint8_t* codes, int64_t code_stride_bytes, uint8_t* scales, int64_t scale_stride_bytes,
                    uint16_t* c_out, int64_t c_stride, hipStream_t stream);

/*
 * csa2_index_full - S2a, dense form: indexer scores of Q queries per sequence
 * against all N indexer keys of that sequence ([jiwasawa] CSA2: a Full layer
 * computes its own indexer Q and scores the whole context; [zaikei] CSA2とFP4:
 * the retrieval keys are shared across layers).
 *
 * Score (R: the pages give no formula) = the exact dot product q . k rounded
 * once to fp32 (nearest-even). A bf16 query against E4M3 keys accumulates its
 * exact products with fp64 FMAs (exact while the query's nonzero elements span
 * at most 2^21 in magnitude); every other dtype pair accumulates a double-double
 * sum, exact while the query's and key's exponents together span less than
 * about 46 binades, rounded once to fp32. A key with an E4M3 NaN byte scores
 * NaN; infinite fp32 / bf16 operands give NaN or an infinity (not specified:
 * the error-free sums turn inf - inf into NaN). With q_pos
 * given, positions t > q_pos[b*Q + i] score -inf (causal prefill).
 *
 *   q_idx    device [B][Q][d_idx] of q_dtype (CSA2_F32 or CSA2_BF16)
 *   k_idx    device [B][N][d_idx] of k_dtype (CSA2_F32, CSA2_BF16 or CSA2_E4M3)
 *   d_idx    64 or 128
 *   q_pos    device [B][Q] int64 or NULL (no mask)
 *   scores   device [B][Q][N] fp32 (output)
 * k_idx must be 16-byte aligned.
 */
int csa2_index_full(const void* q_idx, int32_t q_dtype, const void* k_idx, int32_t k_dtype,
                    int32_t B, int32_t Q, int64_t N, int32_t d_idx, const int64_t* q_pos,
                    float* scores, hipStream_t stream);

/*
 * csa2_index_reindex - S2b: a Reindex layer's scores over the candidate pool
 * only ([jiwasawa] CSA2, Hierarchical Sparse Indexer: the first Full layer
 * picks a pool from the whole context and Reindex layers search only inside
 * it; a Reindex layer re-scores with its own Q against the shared indexer K).
 *
 *   q_idx    device [B][d_idx]; k_idx device [B][N][d_idx] (shared keys)
 *   pool     device [B][P] int32 positions; entries outside [0, N) score -inf
 *   scores   device [B][P] fp32 (output), same score definition as csa2_index_full
 */
int csa2_index_reindex(const void* q_idx, int32_t q_dtype, const void* k_idx, int32_t k_dtype,
                       int32_t B, int64_t N, int32_t d_idx, const int32_t* pool, int32_t P,
                       float* scores, hipStream_t stream);

/*
 * csa2_topk - S3: top-K positions per row ([jiwasawa] CSA2: Full and Reindex
 * layers produce fresh Top-K indices; [zaikei] CSA2とFP4: the selected token
 * positions are shared across layers).
 *
 * Order (R): higher score first, equal scores by lower position; -0 == +0;
 * NaN and -inf are never selected. The first min(K, #selectable) entries are
 * written sorted by ascending position, then -1 up to K.
 *
 *   scores       device; row r's n scores start at scores + r*score_stride
 *   cand         device [rows][n] int32 positions of the entries, or NULL
 *                (position = entry index)
 *   idx          device [rows][K] int32 (output)
 *   sel_scores   device [rows][K] fp32 (output, NaN in padding slots) or NULL
 *   ws           workspace of csa2_topk_workspace_bytes(rows, n, K) bytes, 256-byte aligned
 * Limits: 1 <= K <= n, n < 2^31.
 */
int csa2_topk_workspace_bytes(int64_t rows, int64_t n, int32_t K, size_t* bytes);
int csa2_topk(const float* scores, int64_t rows, int64_t n, int64_t score_stride,
              const int32_t* cand, int32_t K, int32_t* idx, float* sel_scores,
              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_fp4 - S4 + S5: gather the FP4 K and V rows at the selected
 * positions, dequantize them in registers and run softmax attention
 * ([jiwasawa] CSA2: sparse attention over the Top-K positions; [zaikei]
 * CSA2とFP4: dequantize before attention).
 *
 * R: all H query heads share the one KV head and one position list; logits
 * are (q_h . K_j) * softmax_scale (0 selects 1/sqrt(d)); no mask beyond the
 * position list; a query whose list has no valid position gets zeros.
 *
 *   q          device [B][Q][H][d] bf16 bit patterns
 *   H          1..16 query heads;  d = 128
 *   k_codes, k_scales, v_codes, v_scales, code_stride_bytes, scale_stride_bytes:
 *              the main KV cache of B sequences of N positions (see the top)
 *   idx        device [B][Q][K] int32 positions; -1 or >= N = padding
 *   out        device [B][Q][H][d] fp32 (output)
 *   ws         workspace of csa2_sparse_attn_workspace_bytes(...) bytes
 * Alignment: code pointers and code_stride_bytes to 16 bytes; scale
 * pointers and scale_stride_bytes to 8 bytes (each position's 8 K and 8 V
 * scale bytes are read as one 8-byte word each).
 * Numerics: each head's query is scaled by a power of two into f16 range
 * (exact for every element within 2^28 of the head's largest |q|; any finite
 * bf16 query is accepted), the dequantized K and V are exact in f16, each
 * softmax weight is carried as two f16 terms (about 22 significant bits),
 * products accumulate in fp32.
 */
int csa2_sparse_attn_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t d, int32_t K, size_t* bytes);
int csa2_sparse_attn_fp4(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d,
                         const uint8_t* k_codes, const uint8_t* k_scales,
                         const uint8_t* v_codes, const uint8_t* v_scales,
                         int64_t N, int64_t code_stride_bytes, int64_t scale_stride_bytes,
                         const int32_t* idx, int32_t K, float softmax_scale,
                         float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_mxfp4 - csa2_sparse_attn_fp4 over an MXFP4 cache (codes as
 * kv_quant_fp4; 4 E8M0 scale bytes per position for K and 4 for V, one per 32
 * channels). Same arguments and semantics; scale pointers and
 * scale_stride_bytes must be 4-byte aligned (the recommended record is 8
 * bytes: [K scales 4 | V scales 4], 136 bytes per token with the codes).
 * Numerics: the dequantized K and V and the bf16 query are exact bf16 matrix
 * core operands; each softmax weight is carried as two bf16 terms (16
 * significant bits); products accumulate in fp32. Shares the workspace rules
 * (and csa2_sparse_attn_workspace_bytes) of csa2_sparse_attn_fp4.
 */
int csa2_sparse_attn_mxfp4(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d,
                           const uint8_t* k_codes, const uint8_t* k_scales,
                           const uint8_t* v_codes, const uint8_t* v_scales,
                           int64_t N, int64_t code_stride_bytes, int64_t scale_stride_bytes,
                           const int32_t* idx, int32_t K, float softmax_scale,
                           float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_swa - the sparse attention of a decoder layer together
 * with its sliding-window branch, in one softmax ([zaikei] "■CEDで入力処理の
 * 計算量を削減": each decoder layer attends to a window of recent tokens;
 * [jiwasawa] "FP4 メイン KV Cache と SWA Bounded Replay": the window's KV
 * is kept apart from the FP4 main cache).
 *
 * R: the window KV is bf16; query row r (of B*Q) has W window rows of d = 128
 * channels, K at win_k + r*win_row_stride + j*128 and V likewise at win_v,
 * j < W, of which the first win_len[r] (all W when win_len is NULL) are valid.
 * They are keys of the same softmax as the selected main-cache positions (a
 * window row is never merged with a main-cache position). Everything else -
 * main cache in kv_format (CSA2_KV_FP4_E4M3 or CSA2_KV_MXFP4), idx, scale,
 * out, numerics - as csa2_sparse_attn_fp4 / csa2_sparse_attn_mxfp4; window
 * rows are bf16 matrix-core operands (exact), the query scaled per head by a
 * power of two as for the sparse part.
 *   win_k, win_v     device bf16, 16-byte aligned; win_row_stride >= W*128, a multiple of 8
 *   win_len          device [B*Q] int32 or NULL
 *   ws               workspace of csa2_sparse_attn_swa_workspace_bytes(B, Q, H, d, K, W) bytes
 */
int csa2_sparse_attn_swa_workspace_bytes(int32_t B, int32_t Q, int32_t H, int32_t d, int32_t K, int32_t W,
                                         size_t* bytes);
int csa2_sparse_attn_swa(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d, int32_t kv_format,
                         const uint8_t* k_codes, const uint8_t* k_scales,
                         const uint8_t* v_codes, const uint8_t* v_scales,
                         int64_t N, int64_t code_stride_bytes, int64_t scale_stride_bytes,
                         const int32_t* idx, int32_t K,
                         const uint16_t* win_k, const uint16_t* win_v, int64_t win_row_stride, int32_t W,
                         const int32_t* win_len, float softmax_scale,
                         float* out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * csa2_sparse_attn_fp4_noalloc - csa2_sparse_attn_fp4 for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation. Same arguments,
 * semantics and results (bit-identical outputs) without ws / ws_bytes.
 *
 * Scratch: a fixed device array inside the library (4,260,864 bytes per
 * device, held until the process ends): 256 merge counters and up to 511
 * partial softmax states, which covers every shape this call accepts (rows
 * split over several workgroups times their splits stay below 512); a shape
 * that would need more is rejected with CSA2_ERR_WORKSPACE. The array's
 * device address is looked up on the first call on each device (that call
 * also enqueues a small kernel clearing the counters); the call itself never
 * allocates or frees memory.
 * Concurrency: every call on one device shares that device's array and the
 * counters must be zero when a call starts (each completed call leaves them
 * zero), so calls that may overlap on one device - on two streams or from two
 * host threads - race; the caller must order them.
 */
int csa2_sparse_attn_fp4_noalloc(const uint16_t* q, int32_t B, int32_t Q, int32_t H, int32_t d,
                                 const uint8_t* k_codes, const uint8_t* k_scales,
                                 const uint8_t* v_codes, const uint8_t* v_scales,
                                 int64_t N, int64_t code_stride_bytes, int64_t scale_stride_bytes,
                                 const int32_t* idx, int32_t K, float softmax_scale,
                                 float* out, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Layer plan - S6: a static per-layer mode table ([zaikei] CSA2とFP4: each
 * CSA2 layer is fixed to Full, Reindex or Reuse; [jiwasawa] CSA2: modes are
 * assigned statically; Full computes its indexer Q and fresh Top-K; Reindex
 * shares main KV and indexer K and re-scores with its own Q; Reuse shares main
 * KV and Top-K indices and skips the indexer; Hierarchical Sparse Indexer:
 * the first Full layer picks the candidate pool that Reindex layers search).
 *
 * Plan rules (checked at creation): the first layer is Full; a Reindex layer
 * needs an earlier Full layer and P >= K; a Reuse layer takes the positions of
 * the immediately preceding layer (R). The pool is the top-P of the first
 * Full layer's scores, in the top-K order (R), so it holds that layer's top-K.
 * ------------------------------------------------------------------------- */
typedef struct csa2_plan csa2_plan;

typedef struct {
    int32_t K;              /* positions attended per query */
    int32_t P;              /* pool size (used when the plan has a Reindex layer) */
    int32_t H;              /* query heads (1..16) */
    int32_t d;              /* head dim (128) */
    int32_t d_idx;          /* indexer dim (64 or 128) */
    int32_t q_idx_dtype;    /* CSA2_F32 or CSA2_BF16 */
    int32_t k_idx_dtype;    /* CSA2_F32, CSA2_BF16 or CSA2_E4M3 */
    float softmax_scale;    /* 0 selects 1/sqrt(d) */
    int32_t kv_format;      /* CSA2_KV_FP4_E4M3 or CSA2_KV_MXFP4: the main KV cache's format */
    int32_t swa_window;     /* W > 0: every layer also attends to its W-row sliding window (see
                               csa2_sparse_attn_swa) in the same softmax; 0: no window */
} csa2_plan_params;

typedef struct {
    const uint8_t* k_codes; /* main KV cache of B sequences x N positions, in the plan's kv_format */
    const uint8_t* k_scales;
    const uint8_t* v_codes;
    const uint8_t* v_scales;
    int64_t code_stride_bytes;
    int64_t scale_stride_bytes;
    const void* k_idx;      /* device [B][N][d_idx] indexer keys, k_idx_dtype */
} csa2_cache;

typedef struct {
    const uint16_t* q;      /* device [B][H][d] bf16 attention query of this layer */
    const void* q_idx;      /* device [B][d_idx] indexer query (Full, Reindex); ignored for Reuse */
    float* out;             /* device [B][H][d] fp32 attention output */
    int32_t* idx_out;       /* device [B][K] positions selected by this layer (Full, Reindex)
                               or NULL to keep them in the workspace; ignored for Reuse */
    int32_t* pool_out;      /* device [B][P] pool of the first Full layer, or NULL */
    const uint16_t* win_k;  /* swa_window > 0: device [B][W][d] bf16 window K rows of this layer */
    const uint16_t* win_v;  /*                 device [B][W][d] bf16 window V rows */
    const int32_t* win_len; /*                 device [B] valid window rows, or NULL (all W) */
} csa2_layer_io;

/* One layer's inputs and outputs for csa2_plan_run_prefill (a chunk of Q queries per sequence). */
typedef struct {
    const uint16_t* q;      /* device [B][Q][H][d] bf16 attention queries of this layer */
    const void* q_idx;      /* device [B][Q][d_idx] indexer queries (Full, Reindex; 16-byte aligned);
                               ignored for Reuse */
    float* out;             /* device [B][Q][H][d] fp32 attention output */
    int32_t* idx_out;       /* device [B][Q][K] positions this layer attends, or NULL */
} csa2_prefill_io;

int csa2_plan_create(const int32_t* modes, int32_t L, const csa2_plan_params* params, csa2_plan** out);
void csa2_plan_destroy(csa2_plan* plan);
int csa2_plan_workspace_bytes(const csa2_plan* plan, int32_t B, int64_t N, size_t* bytes);
/* One decode step of the whole stack for B sequences, one query each; layers
 * run in order on `stream`. io has one entry per layer. `cache` points to one
 * csa2_cache per Full layer, in layer order (R: a Full layer computes KV
 * afresh, so each Full layer opens a group - its own main KV cache, indexer
 * keys and pool - that the Reindex and Reuse layers after it share, up to the
 * next Full layer; a one-Full plan reads one cache). */
int csa2_plan_run_decode(const csa2_plan* plan, const csa2_cache* cache, const csa2_layer_io* io,
                         int32_t B, int64_t N, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Per-kernel timing of csa2_plan_run_decode (a measurement aid). After
 * csa2_plan_profile_begin(plan, max_runs), each of the next max_runs calls of
 * csa2_plan_run_decode records a HIP event on `stream` before and after each
 * kernel it launches. Kernel slot 2*l is layer l's indexer/selection kernel
 * (none for Reuse), slot 2*l+1 its attention kernel. csa2_plan_profile_read
 * waits for the recorded events and writes the average milliseconds per
 * launch of every slot (0 for a slot that never ran) into avg_ms[2*L] and the
 * number of profiled runs into *runs. max_runs = 0 stops profiling. Events are
 * host-side HIP objects owned by the plan; no device memory is allocated.
 */
int csa2_plan_profile_begin(csa2_plan* plan, int32_t max_runs);
int csa2_plan_profile_read(csa2_plan* plan, float* avg_ms, int32_t* runs);

/*
 * csa2_prefill_full - a chunk of Q queries per sequence through the plan's
 * first (Full) layer: indexer scores over the whole context with the causal
 * rule that query i selects only positions <= q_pos[b][i] (R), top-K, and
 * sparse FP4 attention per query.
 *
 *   q_idx   device [B][Q][d_idx];  q device [B][Q][H][d] bf16
 *   q_pos   device [B][Q] int64 positions of the queries
 *   idx_out device [B][Q][K] int32 (output);  out device [B][Q][H][d] fp32 (output)
 *
 * With bf16 indexer queries, E4M3 or bf16 keys, d_idx = 64 and long contexts
 * the indexer runs on the matrix cores and only nominates candidates; their
 * exact scores decide the top-K. A query whose result the candidates cannot
 * certify (ties or near-ties at its threshold, an overflowing candidate list,
 * more candidates than the exact select holds: 16,640 per query when its
 * lists have more slots than LDS holds keys and positions for)
 * is re-selected by an exact scan of its whole causal range: every such
 * query, however many (beyond 64 per call this fallback is slow: one
 * workgroup per query). The result is always the exact top-K.
 */
int csa2_prefill_workspace_bytes(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, size_t* bytes);
/*
 * csa2_plan_run_prefill - a prefill chunk of Q queries per sequence through
 * every layer of the plan ([jiwasawa] CSA2, Hierarchical Sparse Indexer:
 * the pool of a Full layer is what later Reindex layers search; each query
 * of a chunk is one step of the stack at its own position): per query, each
 * Full layer selects under the causal rule (positions <= q_pos) its top-K and,
 * when a Reindex layer follows in its group, its own pool (top-P); a Reindex
 * layer takes the top-K of that query's pool with its own indexer query; a
 * Reuse layer takes the preceding layer's positions; every layer runs sparse
 * FP4 attention for all B*Q queries. Every selection is the exact top-K (or
 * top-P), as csa2_prefill_full. `cache`: one per Full layer, as
 * csa2_plan_run_decode; io: one csa2_prefill_io per layer; q_pos: device
 * [B][Q] int64. The plan's sliding window (swa_window) is not applied here
 * (the call rejects a plan that has one).
 */
int csa2_plan_prefill_workspace_bytes(const csa2_plan* plan, int32_t B, int32_t Q, int64_t N, size_t* bytes);
int csa2_plan_run_prefill(const csa2_plan* plan, const csa2_cache* cache, const csa2_prefill_io* io,
                          const int64_t* q_pos, int32_t B, int32_t Q, int64_t N, void* ws, size_t ws_bytes,
                          hipStream_t stream);
int csa2_prefill_full(const csa2_plan* plan, const csa2_cache* cache, const void* q_idx,
                      const uint16_t* q, const int64_t* q_pos, int32_t B, int32_t Q, int64_t N,
                      int32_t* idx_out, float* out, void* ws, size_t ws_bytes, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* CSA2_H_ */
