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
from .quant import dequant_fp4, quant_fp4


def dequant_rows(codes, scales, rows, C):
    """Dequantize only the listed rows of a (codes [N][>=C/2], scales [N][>=C/16]) plane."""
    rows = np.asarray(rows, dtype=np.int64)
    return dequant_fp4(np.asarray(codes)[rows][:, : C // 2], np.asarray(scales)[rows][:, : C // 16], C)


def kv_rows(kv, which, rows, C):
    """Dequantized rows of the K or V plane of `kv`.

    The cache is given either as stored planes ('k_codes', 'k_scales', ...) or
    as the bf16 rows before quantization ('k_bf16', 'v_bf16'); in the second
    case only the listed rows are quantized here. Quantization works row by
    row, so this equals quantizing the whole plane first.
    """
    if f"{which}_codes" in kv:
        return dequant_rows(kv[f"{which}_codes"], kv[f"{which}_scales"], rows, C)
    codes, scales = quant_fp4(np.asarray(kv[f"{which}_bf16"])[np.asarray(rows, dtype=np.int64)])
    return dequant_fp4(codes, scales, C)


def sparse_attn(q_bits, kv, idx, softmax_scale=None):
    """One query.

    q_bits: (H, d) bf16 bit patterns. kv: dict with 'k_codes', 'k_scales',
    'v_codes', 'v_scales' (planes over all N positions, [N][d/2] and [N][d/16]),
    or 'k_bf16', 'v_bf16' (the rows before quantization; see kv_rows).
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
