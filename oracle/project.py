"""The KV write path: the decoder's KV rows projected from the encoder's last hidden state, quantized to FP4.

[jiwasawa] "Causal Encoder-Decoder (CED) アーキテクチャ" (its projection
equation) and [zaikei] "■CEDで入力処理の計算量を削減": a decoder layer l above
the middle of the stack computes its global KV from the encoder's final
hidden state, C_l = H_{L/2} W_l^{KV}, so a prefill runs only the lower half.
That projection is the step before kv_quant_fp4 on the write path.

Readings (the pages give the equation only):
  * H [T][D] and W [D][C] are bf16 (the model's activation and weight type);
    C = 256 holds one shared KV head, K in channels 0..127 and V in 128..255;
  * C_l is an activation, so each element is the exact product-sum rounded
    once to bf16 (nearest even) before it is quantized; the quantizer is
    quant.py's (E4M3 per 16 channels) or mxfp4.py's (E8M0 per 32);
  * D (the hidden size) is not given; the workload takes 4096.

The exact product-sum is computed with fp64 matmul (a library routine): each
bf16 x bf16 product is exact in fp64 and the fp64 sum's error, at most about
D * 2^-53 of the sum of |products|, is far below a bf16 unit.
"""

import numpy as np

from .formats import bf16_decode


def project_exact(h_bits, w_bits):
    """fp64 product H @ W of bf16 inputs (bit patterns): h [T][D], w [D][C] -> [T][C]."""
    return bf16_decode(h_bits) @ bf16_decode(w_bits)


def round_to_bf16(x):
    """fp64 values -> bf16 bit patterns, round to nearest even (finite inputs within bf16's range).

    bf16 keeps 8 significant bits: a value m * 2^e (m in [0.5, 1)) sits on a grid of spacing 2^(e-8),
    and below the smallest normal 2^-126 on the subnormal grid 2^-133. x is scaled exactly onto its
    grid, rounded half-to-even (numpy.rint) and scaled back.
    """
    x = np.asarray(x, dtype=np.float64)
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    v = np.ldexp(np.rint(np.ldexp(x, 8 - e)), e - 8)
    return (v.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
