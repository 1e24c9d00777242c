"""Sparse softmax attention over the selected positions of the FP4 main KV cache.

[jiwasawa] CSA2: sparse attention runs over the Top-K positions (a Reuse layer
runs it directly on inherited positions). [zaikei] "■CSA2とFP4でキャッシュを
圧縮": the FP4 cache is dequantized before the attention computation.

Readings: one shared KV head for all H query heads; logits scaled by
1/sqrt(d) unless a scale is given; no mask at decode, no sink, no RoPE;
positions of -1 are padding; a query with no valid position gets zeros.
Everything in fp64.
"""

import numpy as np

from .formats import bf16_decode
from .mxfp4 import dequant_mxfp4, quant_mxfp4
from .quant import dequant_fp4, quant_fp4

# KV storage formats: FP4 E2M1 with an E4M3 scale per 16 channels ([ezic] key
# points), or MXFP4 with an E8M0 scale per 32 channels ([jiwasawa] FP4 main KV).
FORMATS = {"fp4_e4m3": (quant_fp4, dequant_fp4, 16), "mxfp4": (quant_mxfp4, dequant_mxfp4, 32)}


def dequant_rows(codes, scales, rows, C, fmt="fp4_e4m3"):
    """Dequantize only the listed rows of a (codes [N][>=C/2], scales [N][>=C/block]) plane."""
    _, deq, blk = FORMATS[fmt]
    rows = np.asarray(rows, dtype=np.int64)
    return deq(np.asarray(codes)[rows][:, : C // 2], np.asarray(scales)[rows][:, : C // blk], C)


def kv_rows(kv, which, rows, C):
    """Dequantized rows of the K or V plane of `kv`.

    The cache is given either as stored planes ('k_codes', 'k_scales', ...) or
    as the bf16 rows before quantization ('k_bf16', 'v_bf16'); in the second
    case only the listed rows are quantized here. Quantization works row by
    row, so this equals quantizing the whole plane first. kv['format'] names
    the storage format ('fp4_e4m3' when absent, or 'mxfp4').
    """
    fmt = kv.get("format", "fp4_e4m3")
    if f"{which}_codes" in kv:
        return dequant_rows(kv[f"{which}_codes"], kv[f"{which}_scales"], rows, C, fmt)
    quant, deq, _ = FORMATS[fmt]
    codes, scales = quant(np.asarray(kv[f"{which}_bf16"])[np.asarray(rows, dtype=np.int64)])
    return deq(codes, scales, C)


def sparse_attn(q_bits, kv, idx, softmax_scale=None):
    """One query.

    q_bits: (H, d) bf16 bit patterns. kv: dict with 'k_codes', 'k_scales',
    'v_codes', 'v_scales' (planes over all N positions, [N][d/2] and [N][d/16],
    or [N][d/32] for 'format': 'mxfp4'), or 'k_bf16', 'v_bf16' (the rows before
    quantization; see kv_rows).
    idx: (K,) positions, -1 = padding. Returns (H, d) fp64.
    """
    q = bf16_decode(q_bits)
    H, d = q.shape
    scale = 1.0 / np.sqrt(d) if softmax_scale is None else float(softmax_scale)
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[idx >= 0]
    if sel.size == 0:
        return np.zeros((H, d))
    K_hat = kv_rows(kv, "k", sel, d)                                 # (k, d)
    V_hat = kv_rows(kv, "v", sel, d)
    logits = (q @ K_hat.T) * scale                                   # (H, k)
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (w @ V_hat) / w.sum(axis=1, keepdims=True)


def sparse_attn_swa(q_bits, kv, idx, win_k_bits, win_v_bits, softmax_scale=None):
    """One query of a decoder layer with a sliding-window branch beside CSA2: one softmax over the
    selected positions of the FP4 main KV cache and the window's own KV rows.

    [zaikei] "■CEDで入力処理の計算量を削減": each decoder layer keeps a sliding-window attention over the
    most recent tokens; [jiwasawa] "FP4 メイン KV Cache と SWA Bounded Replay": the window's KV is kept
    apart from the FP4 main cache. Readings: the window KV is bf16 (win_k_bits, win_v_bits: (W, d) bit
    patterns, the valid rows of the window), attended by every head with the same scale as the sparse
    part; its rows are separate keys of the same softmax (no position is merged with a main-cache one).
    Returns (H, d) fp64; zeros when there is neither a valid position nor a window row.
    """
    q = bf16_decode(q_bits)
    H, d = q.shape
    scale = 1.0 / np.sqrt(d) if softmax_scale is None else float(softmax_scale)
    idx = np.asarray(idx, dtype=np.int64)
    sel = idx[idx >= 0]
    Ks, Vs = [], []
    if sel.size:
        Ks.append(kv_rows(kv, "k", sel, d))
        Vs.append(kv_rows(kv, "v", sel, d))
    wk = bf16_decode(np.asarray(win_k_bits, dtype=np.uint16).reshape(-1, d))
    wv = bf16_decode(np.asarray(win_v_bits, dtype=np.uint16).reshape(-1, d))
    if wk.shape[0]:
        Ks.append(wk)
        Vs.append(wv)
    if not Ks:
        return np.zeros((H, d))
    K_all, V_all = np.concatenate(Ks), np.concatenate(Vs)
    logits = (q @ K_all.T) * scale
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (w @ V_all) / w.sum(axis=1, keepdims=True)
