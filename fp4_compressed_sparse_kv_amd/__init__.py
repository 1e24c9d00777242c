"""Python binding of libcsa2: the decode-time CSA2 step over an FP4 E2M1 main KV cache on MI355X.

A thin ctypes layer over the C ABI in include/csa2.h: it turns torch tensors
into device pointers, picks strides and the current HIP stream, allocates
workspaces with torch (zero-filled once, then reused) and raises Csa2Error on
any non-zero status. Every step of the computation runs in the library's HIP
kernels; there is no fallback path. If libcsa2.so is missing the first call
raises.

Build first:  python -m fp4_compressed_sparse_kv_amd.build
"""

import ctypes
import os
import threading

import torch

__all__ = [
    "Csa2Error", "lib", "F32", "BF16", "E4M3", "FULL", "REINDEX", "REUSE",
    "kv_quant_fp4", "kv_dequant_fp4", "kv_quant_mxfp4", "kv_dequant_mxfp4", "kv_project", "index_full", "index_reindex", "topk",
    "sparse_attn_fp4", "sparse_attn_swa", "sparse_attn_fp4_noalloc", "KVCache", "Plan", "status_word",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcsa2.so")

F32, BF16, E4M3 = 0, 1, 2
FULL, REINDEX, REUSE = 0, 1, 2
MODE_CODES = {"full": FULL, "reindex": REINDEX, "reuse": REUSE}
DTYPE_CODES = {"f32": F32, "bf16": BF16, "e4m3": E4M3}

_c_i32, _c_i64, _c_sz, _c_f32, _vp = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t, ctypes.c_float, ctypes.c_void_p


class Csa2Error(RuntimeError):
    pass


KV_FP4_E4M3, KV_MXFP4 = 0, 1
KV_FORMATS = {"fp4_e4m3": KV_FP4_E4M3, "mxfp4": KV_MXFP4}


class PlanParams(ctypes.Structure):
    _fields_ = [("K", _c_i32), ("P", _c_i32), ("H", _c_i32), ("d", _c_i32), ("d_idx", _c_i32),
                ("q_idx_dtype", _c_i32), ("k_idx_dtype", _c_i32), ("softmax_scale", _c_f32), ("kv_format", _c_i32),
                ("swa_window", _c_i32)]


class CacheDesc(ctypes.Structure):
    _fields_ = [("k_codes", _vp), ("k_scales", _vp), ("v_codes", _vp), ("v_scales", _vp),
                ("code_stride_bytes", _c_i64), ("scale_stride_bytes", _c_i64), ("k_idx", _vp)]


class PrefillIO(ctypes.Structure):
    _fields_ = [("q", _vp), ("q_idx", _vp), ("out", _vp), ("idx_out", _vp)]


class LayerIO(ctypes.Structure):
    _fields_ = [("q", _vp), ("q_idx", _vp), ("out", _vp), ("idx_out", _vp), ("pool_out", _vp),
                ("win_k", _vp), ("win_v", _vp), ("win_len", _vp)]


_SIGS = {
    "csa2_last_error": (ctypes.c_char_p, []),
    "csa2_version": (ctypes.c_int, []),
    "kv_quant_fp4": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp]),
    "kv_dequant_fp4": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _c_i64, _c_i32, _vp, _c_i64, _vp]),
    "kv_quant_mxfp4": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i64, _vp, _c_i64, _vp, _c_i64, _vp]),
    "kv_dequant_mxfp4": (ctypes.c_int, [_vp, _c_i64, _vp, _c_i64, _c_i64, _c_i32, _vp, _c_i64, _vp]),
    "csa2_kv_project": (ctypes.c_int, [_vp, _c_i64, _c_i32, _c_i64, _vp, _c_i64, _c_i32, _vp, _c_i64, _vp, _c_i64,
                                       _vp, _c_i64, _vp]),
    "csa2_index_full": (ctypes.c_int, [_vp, _c_i32, _vp, _c_i32, _c_i32, _c_i32, _c_i64, _c_i32, _vp, _vp, _vp]),
    "csa2_index_reindex": (ctypes.c_int, [_vp, _c_i32, _vp, _c_i32, _c_i32, _c_i64, _c_i32, _vp, _c_i32, _vp, _vp]),
    "csa2_topk_workspace_bytes": (ctypes.c_int, [_c_i64, _c_i64, _c_i32, ctypes.POINTER(_c_sz)]),
    "csa2_topk": (ctypes.c_int, [_vp, _c_i64, _c_i64, _c_i64, _vp, _c_i32, _vp, _vp, _vp, _c_sz, _vp]),
    "csa2_sparse_attn_workspace_bytes": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, ctypes.POINTER(_c_sz)]),
    "csa2_sparse_attn_fp4": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_i64, _c_i64,
                                            _c_i64, _vp, _c_i32, _c_f32, _vp, _vp, _c_sz, _vp]),
    "csa2_sparse_attn_mxfp4": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_i64, _c_i64,
                                              _c_i64, _vp, _c_i32, _c_f32, _vp, _vp, _c_sz, _vp]),
    "csa2_sparse_attn_swa_workspace_bytes": (ctypes.c_int, [_c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32,
                                                            ctypes.POINTER(_c_sz)]),
    "csa2_sparse_attn_swa": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_i64,
                                            _c_i64, _c_i64, _vp, _c_i32, _vp, _vp, _c_i64, _c_i32, _vp, _c_f32, _vp,
                                            _vp, _c_sz, _vp]),
    "csa2_sparse_attn_fp4_noalloc": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i32, _c_i32, _vp, _vp, _vp, _vp, _c_i64,
                                                    _c_i64, _c_i64, _vp, _c_i32, _c_f32, _vp, _vp]),
    "csa2_plan_create": (ctypes.c_int, [ctypes.POINTER(_c_i32), _c_i32, ctypes.POINTER(PlanParams),
                                        ctypes.POINTER(_vp)]),
    "csa2_plan_destroy": (None, [_vp]),
    "csa2_plan_workspace_bytes": (ctypes.c_int, [_vp, _c_i32, _c_i64, ctypes.POINTER(_c_sz)]),
    "csa2_plan_run_decode": (ctypes.c_int, [_vp, ctypes.POINTER(CacheDesc), ctypes.POINTER(LayerIO), _c_i32, _c_i64,
                                            _vp, _c_sz, _vp]),
    "csa2_plan_profile_begin": (ctypes.c_int, [_vp, _c_i32]),
    "csa2_plan_profile_read": (ctypes.c_int, [_vp, ctypes.POINTER(_c_f32), ctypes.POINTER(_c_i32)]),
    "csa2_prefill_workspace_bytes": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i64, ctypes.POINTER(_c_sz)]),
    "csa2_plan_prefill_workspace_bytes": (ctypes.c_int, [_vp, _c_i32, _c_i32, _c_i64, ctypes.POINTER(_c_sz)]),
    "csa2_plan_run_prefill": (ctypes.c_int, [_vp, ctypes.POINTER(CacheDesc), ctypes.POINTER(PrefillIO), _vp, _c_i32,
                                             _c_i32, _c_i64, _vp, _c_sz, _vp]),
    "csa2_prefill_full": (ctypes.c_int, [_vp, ctypes.POINTER(CacheDesc), _vp, _vp, _vp, _c_i32, _c_i32, _c_i64, _vp,
                                         _vp, _vp, _c_sz, _vp]),
}

_lib = None
_lock = threading.Lock()


def lib():
    """Load libcsa2.so (once) and declare its signatures. Raises if it is not built."""
    global _lib
    if _lib is None:
        with _lock:
            if _lib is None:
                if not os.path.exists(LIB_PATH):
                    raise Csa2Error(f"{LIB_PATH} is not built; run python -m fp4_compressed_sparse_kv_amd.build")
                h = ctypes.CDLL(LIB_PATH)
                for name, (res, args) in _SIGS.items():
                    f = getattr(h, name)
                    f.restype = res
                    f.argtypes = args
                _lib = h
    return _lib


def _check(rc, what):
    if rc != 0:
        msg = lib().csa2_last_error().decode(errors="replace")
        raise Csa2Error(f"{what} failed with status {rc}: {msg}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dtype_code(t):
    if t.dtype == torch.float32:
        return F32
    if t.dtype in (torch.bfloat16, torch.int16, torch.uint16):
        return BF16
    if t.dtype in (torch.float8_e4m3fn, torch.uint8):
        return E4M3
    raise Csa2Error(f"unsupported dtype {t.dtype}")


def _need_cuda(*ts):
    for t in ts:
        if t is not None and not t.is_cuda:
            raise Csa2Error("all tensors must be on the GPU")


_ws_cache = {}


def workspace(nbytes, device, key="default"):
    """A zero-filled device workspace of at least nbytes, reused across calls with the same key."""
    k = (key, str(device))
    ws = _ws_cache.get(k)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(int(nbytes), 256), dtype=torch.uint8, device=device)
        _ws_cache[k] = ws
    return ws


STATUS_BARRIER_TIMEOUT = 1      # a selection kernel's in-kernel wait gave up: that call's outputs are unspecified


def status_word(ws):
    """The device status word of a workspace (its first 32-bit word; synchronizes with the device).
    0 = every call that used this workspace completed normally; the library never clears it."""
    torch.cuda.synchronize(ws.device)
    return int(ws[:4].view(torch.int32).item())


def _check_status(ws, what):
    st = status_word(ws)
    if st:
        raise Csa2Error(f"{what}: device status word {st:#x} (bit 0: a selection kernel's in-kernel wait "
                        f"timed out) - the outputs are not valid")


# ------------------------------------------------------------------- calls

def kv_quant_fp4(x, codes=None, scales=None, stream=None):
    """Quantize bf16 rows x [T][C] into (codes [T][C/2] u8, scales [T][C/16] u8)."""
    _need_cuda(x)
    T, C = x.shape
    if codes is None:
        codes = torch.empty(T, C // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(T, C // 16, dtype=torch.uint8, device=x.device)
    _check(lib().kv_quant_fp4(_ptr(x), T, C, x.stride(0), _ptr(codes), codes.stride(0), _ptr(scales),
                              scales.stride(0), _stream(stream)), "kv_quant_fp4")
    return codes, scales


def kv_dequant_fp4(codes, scales, C, y=None, stream=None):
    """Dequantize (codes, scales) of rows with C channels into bf16 y [T][C]."""
    _need_cuda(codes, scales)
    T = codes.shape[0]
    if y is None:
        y = torch.empty(T, C, dtype=torch.bfloat16, device=codes.device)
    _check(lib().kv_dequant_fp4(_ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0), T, C, _ptr(y),
                                y.stride(0), _stream(stream)), "kv_dequant_fp4")
    return y


def kv_quant_mxfp4(x, codes=None, scales=None, stream=None):
    """MXFP4: quantize bf16 rows x [T][C] (C % 32 == 0) into (codes [T][C/2] u8, E8M0 scales [T][C/32] u8)."""
    _need_cuda(x)
    T, C = x.shape
    if codes is None:
        codes = torch.empty(T, C // 2, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(T, C // 32, dtype=torch.uint8, device=x.device)
    _check(lib().kv_quant_mxfp4(_ptr(x), T, C, x.stride(0), _ptr(codes), codes.stride(0), _ptr(scales),
                                scales.stride(0), _stream(stream)), "kv_quant_mxfp4")
    return codes, scales


def kv_dequant_mxfp4(codes, scales, C, y=None, stream=None):
    """Dequantize MXFP4 (codes, E8M0 scales) of rows with C channels into bf16 y [T][C]."""
    _need_cuda(codes, scales)
    T = codes.shape[0]
    if y is None:
        y = torch.empty(T, C, dtype=torch.bfloat16, device=codes.device)
    _check(lib().kv_dequant_mxfp4(_ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0), T, C, _ptr(y),
                                  y.stride(0), _stream(stream)), "kv_dequant_mxfp4")
    return y


def kv_project(h, w_t, kv_format="fp4_e4m3", codes=None, scales=None, c_out=None, stream=None):
    """KV write path: C = h [T][D] @ w_t[256][D]^T (bf16), rounded to bf16 and quantized in one kernel into
    codes [T][128] u8 and scales [T][16 or 8] u8 (the cache record layout; views of a KVCache's planes
    work); c_out [T][256] bf16 receives the rounded C when given."""
    _need_cuda(h, w_t)
    T, D = h.shape
    blk = 32 if kv_format == "mxfp4" else 16
    if codes is None:
        codes = torch.empty(T, 128, dtype=torch.uint8, device=h.device)
    if scales is None:
        scales = torch.empty(T, 256 // blk, dtype=torch.uint8, device=h.device)
    _check(lib().csa2_kv_project(_ptr(h), T, D, h.stride(0), _ptr(w_t), w_t.stride(0), KV_FORMATS[kv_format],
                                 _ptr(codes), codes.stride(0), _ptr(scales), scales.stride(0), _ptr(c_out),
                                 c_out.stride(0) if c_out is not None else 0, _stream(stream)), "csa2_kv_project")
    return codes, scales


def index_full(q_idx, k_idx, q_pos=None, scores=None, stream=None):
    """Dense indexer scores. q_idx [B][Q][d_idx], k_idx [B][N][d_idx] -> scores [B][Q][N] fp32."""
    _need_cuda(q_idx, k_idx, q_pos)
    B, Q, d_idx = q_idx.shape
    N = k_idx.shape[1]
    if scores is None:
        scores = torch.empty(B, Q, N, dtype=torch.float32, device=q_idx.device)
    _check(lib().csa2_index_full(_ptr(q_idx), _dtype_code(q_idx), _ptr(k_idx), _dtype_code(k_idx), B, Q, N, d_idx,
                                 _ptr(q_pos), _ptr(scores), _stream(stream)), "csa2_index_full")
    return scores


def index_reindex(q_idx, k_idx, pool, scores=None, stream=None):
    """Reindex scores over the pool. q_idx [B][d_idx], k_idx [B][N][d_idx], pool [B][P] -> [B][P] fp32."""
    _need_cuda(q_idx, k_idx, pool)
    B, d_idx = q_idx.shape
    N = k_idx.shape[1]
    P = pool.shape[1]
    if scores is None:
        scores = torch.empty(B, P, dtype=torch.float32, device=q_idx.device)
    _check(lib().csa2_index_reindex(_ptr(q_idx), _dtype_code(q_idx), _ptr(k_idx), _dtype_code(k_idx), B, N, d_idx,
                                    _ptr(pool), P, _ptr(scores), _stream(stream)), "csa2_index_reindex")
    return scores


def topk(scores, K, cand=None, idx=None, sel_scores=None, want_scores=False, stream=None, ws=None):
    """Top-K positions per row of scores [rows][n] (stride allowed): idx [rows][K] ascending, -1 padded.
    ws: optional zero-filled uint8 workspace (default: a cached one)."""
    _need_cuda(scores, cand)
    rows, n = scores.shape
    dev = scores.device
    if idx is None:
        idx = torch.empty(rows, K, dtype=torch.int32, device=dev)
    if want_scores and sel_scores is None:
        sel_scores = torch.empty(rows, K, dtype=torch.float32, device=dev)
    nb = ctypes.c_size_t(0)
    _check(lib().csa2_topk_workspace_bytes(rows, n, K, ctypes.byref(nb)), "csa2_topk_workspace_bytes")
    if ws is None:
        ws = workspace(nb.value, dev, "topk")
    _check(lib().csa2_topk(_ptr(scores), rows, n, scores.stride(0), _ptr(cand), K, _ptr(idx), _ptr(sel_scores),
                           _ptr(ws), ws.numel(), _stream(stream)), "csa2_topk")
    return (idx, sel_scores) if want_scores else idx


class KVCache:
    """Main KV cache of B sequences x N positions in the 144-byte record layout.

    codes [B*N][128] u8 = [K codes 64 | V codes 64], scales [B*N][16] u8 =
    [K scales 8 | V scales 8] (E4M3 per 16 channels) or [B*N][8] u8 = [K 4 | V 4]
    (MXFP4: E8M0 per 32 channels); k_idx [B][N][d_idx] indexer keys.
    """

    def __init__(self, B, N, d=128, device="cuda", k_idx=None, kv_format="fp4_e4m3"):
        self.B, self.N, self.d = B, N, d
        self.kv_format = kv_format
        self.block = 32 if kv_format == "mxfp4" else 16     # channels per scale
        self.codes = torch.empty(B * N, d, dtype=torch.uint8, device=device)
        self.scales = torch.empty(B * N, 2 * d // self.block, dtype=torch.uint8, device=device)
        self.k_idx = k_idx

    @property
    def k_codes(self):
        return self.codes[:, : self.d // 2]

    @property
    def v_codes(self):
        return self.codes[:, self.d // 2:]

    @property
    def k_scales(self):
        return self.scales[:, : self.d // self.block]

    @property
    def v_scales(self):
        return self.scales[:, self.d // self.block:]

    def fill(self, k_bf16, v_bf16, row0=0, stream=None):
        """Quantize bf16 K and V rows [n][d] into positions [row0, row0+n) (flat over B*N)."""
        n = k_bf16.shape[0]
        quant = kv_quant_mxfp4 if self.kv_format == "mxfp4" else kv_quant_fp4
        quant(k_bf16, self.k_codes[row0:row0 + n], self.k_scales[row0:row0 + n], stream)
        quant(v_bf16, self.v_codes[row0:row0 + n], self.v_scales[row0:row0 + n], stream)

    def desc(self):
        return CacheDesc(self.codes.data_ptr(), self.scales.data_ptr(), self.codes.data_ptr() + self.d // 2,
                         self.scales.data_ptr() + self.d // self.block, self.codes.stride(0), self.scales.stride(0),
                         None if self.k_idx is None else self.k_idx.data_ptr())


def sparse_attn_fp4(q, cache, idx, softmax_scale=None, out=None, stream=None, ws=None):
    """Sparse FP4 attention. q [B][Q][H][d] bf16, idx [B][Q][K] int32 -> out [B][Q][H][d] fp32.
    ws: optional zero-filled uint8 workspace (default: a cached one)."""
    _need_cuda(q, idx)
    B, Q, H, d = q.shape
    K = idx.shape[-1]
    if out is None:
        out = torch.empty(B, Q, H, d, dtype=torch.float32, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale     # 0: the library's default 1/sqrt(d)
    nb = ctypes.c_size_t(0)
    _check(lib().csa2_sparse_attn_workspace_bytes(B, Q, H, d, K, ctypes.byref(nb)), "csa2_sparse_attn_workspace_bytes")
    if ws is None:
        ws = workspace(nb.value, q.device, "attn")
    c = cache.desc()
    name = "csa2_sparse_attn_mxfp4" if cache.kv_format == "mxfp4" else "csa2_sparse_attn_fp4"
    _check(getattr(lib(), name)(_ptr(q), B, Q, H, d, c.k_codes, c.k_scales, c.v_codes, c.v_scales, cache.N,
                                c.code_stride_bytes, c.scale_stride_bytes, _ptr(idx), K, scale, _ptr(out),
                                _ptr(ws), ws.numel(), _stream(stream)), name)
    return out


def sparse_attn_swa(q, cache, idx, win_k, win_v, win_len=None, softmax_scale=None, out=None, stream=None, ws=None):
    """Sparse attention plus a sliding-window branch in one softmax. q [B][Q][H][d] bf16, idx [B][Q][K];
    win_k, win_v [B][Q][W][d] bf16 (each query row's window rows); win_len [B*Q] int32 or None (all W)."""
    _need_cuda(q, idx, win_k, win_v, win_len)
    B, Q, H, d = q.shape
    K = idx.shape[-1]
    W = win_k.shape[-2]
    if out is None:
        out = torch.empty(B, Q, H, d, dtype=torch.float32, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale
    nb = ctypes.c_size_t(0)
    _check(lib().csa2_sparse_attn_swa_workspace_bytes(B, Q, H, d, K, W, ctypes.byref(nb)),
           "csa2_sparse_attn_swa_workspace_bytes")
    if ws is None:
        ws = workspace(nb.value, q.device, "attn")
    c = cache.desc()
    rs = win_k.stride(-3) if win_k.dim() >= 3 else W * d
    _check(lib().csa2_sparse_attn_swa(_ptr(q), B, Q, H, d, KV_FORMATS[cache.kv_format], c.k_codes, c.k_scales,
                                      c.v_codes, c.v_scales, cache.N, c.code_stride_bytes, c.scale_stride_bytes,
                                      _ptr(idx), K, _ptr(win_k), _ptr(win_v), rs, W, _ptr(win_len), scale,
                                      _ptr(out), _ptr(ws), ws.numel(), _stream(stream)), "csa2_sparse_attn_swa")
    return out


def sparse_attn_fp4_noalloc(q, cache, idx, softmax_scale=None, out=None, stream=None):
    """sparse_attn_fp4 through the library's allocation-free entry point (scratch in a fixed device
    array; calls that may overlap on one device race)."""
    _need_cuda(q, idx)
    B, Q, H, d = q.shape
    K = idx.shape[-1]
    if out is None:
        out = torch.empty(B, Q, H, d, dtype=torch.float32, device=q.device)
    scale = 0.0 if softmax_scale is None else softmax_scale
    c = cache.desc()
    _check(lib().csa2_sparse_attn_fp4_noalloc(_ptr(q), B, Q, H, d, c.k_codes, c.k_scales, c.v_codes, c.v_scales,
                                              cache.N, c.code_stride_bytes, c.scale_stride_bytes, _ptr(idx), K, scale,
                                              _ptr(out), _stream(stream)), "csa2_sparse_attn_fp4_noalloc")
    return out


class Plan:
    """A static Full / Reindex / Reuse layer plan (csa2_plan_*)."""

    def __init__(self, modes, K, P=0, H=16, d=128, d_idx=64, q_idx_dtype="bf16", k_idx_dtype="e4m3",
                 softmax_scale=0.0, kv_format="fp4_e4m3", swa_window=0):
        codes = [MODE_CODES[m] if isinstance(m, str) else int(m) for m in modes]
        arr = (_c_i32 * len(codes))(*codes)
        self.modes = list(codes)
        self.params = PlanParams(K, P or 0, H, d, d_idx, DTYPE_CODES[q_idx_dtype], DTYPE_CODES[k_idx_dtype],
                                 softmax_scale, KV_FORMATS[kv_format], swa_window)
        h = ctypes.c_void_p(None)
        _check(lib().csa2_plan_create(arr, len(codes), ctypes.byref(self.params), ctypes.byref(h)), "csa2_plan_create")
        self._h = h

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.csa2_plan_destroy(h)
            self._h = None

    def workspace_bytes(self, B, N):
        nb = ctypes.c_size_t(0)
        _check(lib().csa2_plan_workspace_bytes(self._h, B, N, ctypes.byref(nb)), "csa2_plan_workspace_bytes")
        return nb.value

    @staticmethod
    def _caches(cache):
        """One KVCache or a list of them (one per Full layer) -> (first cache, ctypes array of descriptors)."""
        cs = list(cache) if isinstance(cache, (list, tuple)) else [cache]
        arr = (CacheDesc * len(cs))(*[c.desc() for c in cs])
        return cs[0], arr

    def decode_workspace(self, cache):
        """The cached workspace run_decode uses for this cache's shape (zero-filled once)."""
        c0 = cache[0] if isinstance(cache, (list, tuple)) else cache
        return workspace(self.workspace_bytes(c0.B, c0.N), c0.codes.device, ("plan", id(self)))

    def run_decode(self, cache, layers, ws=None, stream=None, check=True):
        """layers: list of dicts with 'q' [B][H][d] bf16, 'q_idx' [B][d_idx], 'out' [B][H][d] fp32 and
        optional 'idx_out' [B][K] int32, 'pool_out' [B][P] int32; with swa_window W > 0 also 'win_k',
        'win_v' [B][W][d] bf16 and optional 'win_len' [B] int32.
        check: synchronize and raise Csa2Error if the workspace status word is nonzero (pass False in
        timing loops and read status_word(plan.decode_workspace(cache)) afterwards)."""
        c0, descs = self._caches(cache)
        B, N = c0.B, c0.N
        if ws is None:
            ws = self.decode_workspace(cache)
        io = (LayerIO * len(layers))()
        for i, L in enumerate(layers):
            def p(key):
                t = L.get(key)
                return t.data_ptr() if t is not None else None
            io[i] = LayerIO(L["q"].data_ptr(), p("q_idx"), L["out"].data_ptr(), p("idx_out"), p("pool_out"),
                            p("win_k"), p("win_v"), p("win_len"))
        _check(lib().csa2_plan_run_decode(self._h, descs, io, B, N, _ptr(ws), ws.numel(),
                                          _stream(stream)), "csa2_plan_run_decode")
        if check:
            _check_status(ws, "csa2_plan_run_decode")

    def profile_begin(self, max_runs):
        """Record HIP events around every kernel of the next max_runs run_decode calls."""
        _check(lib().csa2_plan_profile_begin(self._h, max_runs), "csa2_plan_profile_begin")

    def profile_read(self):
        """Average ms per launch for each kernel slot (2*l: selection of layer l, 2*l+1: attention)."""
        n = 2 * len(self.modes)
        arr = (_c_f32 * n)()
        runs = _c_i32(0)
        _check(lib().csa2_plan_profile_read(self._h, arr, ctypes.byref(runs)), "csa2_plan_profile_read")
        return list(arr), runs.value

    def prefill_workspace_bytes(self, B, Q, N):
        nb = ctypes.c_size_t(0)
        _check(lib().csa2_prefill_workspace_bytes(self._h, B, Q, N, ctypes.byref(nb)), "csa2_prefill_workspace_bytes")
        return nb.value

    def run_prefill(self, cache, layers, q_pos, ws=None, stream=None, check=True):
        """A prefill chunk through every layer (csa2_plan_run_prefill). cache: a KVCache or one per Full
        layer; layers: dicts with 'q' [B][Q][H][d] bf16, 'q_idx' [B][Q][d_idx] (Full, Reindex), 'out'
        [B][Q][H][d] fp32 and optional 'idx_out' [B][Q][K] int32; q_pos [B][Q] int64."""
        c0, descs = self._caches(cache)
        B, Q = q_pos.shape
        nb = ctypes.c_size_t(0)
        _check(lib().csa2_plan_prefill_workspace_bytes(self._h, B, Q, c0.N, ctypes.byref(nb)),
               "csa2_plan_prefill_workspace_bytes")
        if ws is None:
            ws = workspace(nb.value, c0.codes.device, ("plan_prefill", id(self)))
        io = (PrefillIO * len(layers))()
        for i, L in enumerate(layers):
            io[i] = PrefillIO(L["q"].data_ptr(), L["q_idx"].data_ptr() if L.get("q_idx") is not None else None,
                              L["out"].data_ptr(), L["idx_out"].data_ptr() if L.get("idx_out") is not None else None)
        _check(lib().csa2_plan_run_prefill(self._h, descs, io, _ptr(q_pos), B, Q, c0.N, _ptr(ws), ws.numel(),
                                           _stream(stream)), "csa2_plan_run_prefill")
        if check:
            _check_status(ws, "csa2_plan_run_prefill")

    def prefill_workspace(self, cache, Q):
        """The cached workspace prefill_full uses for this shape (zero-filled once)."""
        nb = self.prefill_workspace_bytes(cache.B, Q, cache.N)
        return workspace(nb, cache.codes.device, ("prefill", id(self)))

    def prefill_status(self, cache, Q):
        """Device status word of the cached prefill workspace (synchronizes); 0 = clean."""
        return status_word(self.prefill_workspace(cache, Q))

    def prefill_full(self, cache, q_idx, q, q_pos, idx_out=None, out=None, ws=None, stream=None, check=True):
        """Full-layer prefill: q_idx [B][Q][d_idx], q [B][Q][H][d] bf16, q_pos [B][Q] int64.
        check: synchronize and raise Csa2Error if the workspace status word is nonzero."""
        B, Q = q_pos.shape
        dev = q.device
        K = self.params.K
        if idx_out is None:
            idx_out = torch.empty(B, Q, K, dtype=torch.int32, device=dev)
        if out is None:
            out = torch.empty(B, Q, q.shape[2], q.shape[3], dtype=torch.float32, device=dev)
        if ws is None:
            ws = self.prefill_workspace(cache, Q)
        desc = cache.desc()
        _check(lib().csa2_prefill_full(self._h, ctypes.byref(desc), _ptr(q_idx), _ptr(q), _ptr(q_pos), B, Q, cache.N,
                                       _ptr(idx_out), _ptr(out), _ptr(ws), ws.numel(), _stream(stream)),
               "csa2_prefill_full")
        if check:
            _check_status(ws, "csa2_prefill_full")
        return idx_out, out
