"""FP4 E2M1 quantization of KV rows with one E4M3 scale per 16 channels, and its inverse.

[ezic] key points / "KVを捨てる、共有する、作り直す": E2M1 elements, one E4M3
scale per 16 channels. [zaikei] "■CSA2とFP4でキャッシュを圧縮": the main KV
cache is stored in FP4 E2M1 and dequantized before attention.

Readings (the pages do not say how the scale is picked):
  * scale S = RNE_E4M3(amax / 6), 6 being the largest E2M1 magnitude; the
    division is the exact real one. amax / 6 above 448 saturates to 448
    (codes then clip to +-6); amax / 6 that rounds to 0 gives S = 0 and all
    16 codes 0x0.
  * code_i = RNE_E2M1(x_i / S), exact real division, sign kept.
  * storage: codes[row][C/2] with channel 2j in the low nibble and 2j+1 in the
    high nibble of byte j; scales[row][C/16] as E4M3FN bytes.

Both divisions are done here in fp64. That reproduces the exact-real rounding
decision: an fp64 quotient can sit on a rounding threshold only when the exact
quotient does (the tests check this exhaustively over every bf16 input and
every E4M3 scale).
"""

import numpy as np

from .formats import bf16_decode, e2m1_decode, e2m1_encode, e4m3_decode, e4m3_encode, E2M1_MAX

GROUP = 16


def quant_fp4(x_bits):
    """bf16 rows [T][C] (uint16 bit patterns) -> (codes [T][C/2] u8, scales [T][C/16] u8)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, C = x_bits.shape
    assert C % GROUP == 0
    x = bf16_decode(x_bits).reshape(T, C // GROUP, GROUP)
    amax = np.abs(x).max(axis=-1)                                   # [T][C/16]
    scale_codes = e4m3_encode(amax / E2M1_MAX)
    S = e4m3_decode(scale_codes)                                    # >= 0, finite
    zero = S == 0
    safe_S = np.where(zero, 1.0, S)
    codes = e2m1_encode(x / safe_S[..., None])
    codes = np.where(zero[..., None], np.uint8(0), codes).reshape(T, C)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes.astype(np.uint8)


def unpack_codes(packed, C):
    """codes [T][C/2] u8 -> per-channel 4-bit codes [T][C] u8."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (C,), dtype=np.uint8)
    out[..., 0::2] = packed[..., : C // 2] & 0xF
    out[..., 1::2] = packed[..., : C // 2] >> 4
    return out


def dequant_fp4(packed, scale_codes, C):
    """(codes, scales) -> values [T][C] in fp64: v_i = E2M1(code_i) * S.

    Every such product has at most 6 significant bits and lies in
    [2^-10, 2688], so it is exact in fp32, bf16 and fp16 as well.
    """
    codes = unpack_codes(packed, C)
    T = codes.shape[0]
    S = e4m3_decode(np.asarray(scale_codes, dtype=np.uint8)[:, : C // GROUP])
    v = e2m1_decode(codes).reshape(T, C // GROUP, GROUP) * S[..., None]
    return v.reshape(T, C)


def bytes_per_token(C):
    """Stored bytes for C channels: C/2 code bytes plus C/16 scale bytes."""
    assert C % GROUP == 0
    return C // 2 + C // GROUP
