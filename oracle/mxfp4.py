"""MXFP4: FP4 E2M1 elements with one E8M0 (power-of-two) scale per 32 channels, and its inverse.

[jiwasawa] "FP4 メイン KV Cache と SWA Bounded Replay": the main KV cache is
quantized to FP4 in the OCP-standard MXFP4 format, E2M1 elements. [ezic] key
points gives the other reading (one E4M3 scale per 16 channels, `quant.py`);
this module is the MXFP4 reading, taken from the OCP Microscaling (MX)
format definition the page names: blocks of 32 elements share one scale X
that is a power of two stored as an E8M0 byte (value 2^(byte - 127), byte
0xFF = NaN); the scale of a block is X = 2^(floor(log2(max |x|)) - 2), 2
being the exponent of E2M1's largest normal 6 = 1.5 * 2^2; each element is
x / X rounded to E2M1.

Readings where the definition leaves a step open:
  * element rounding: round-to-nearest-even onto E2M1 with saturation (values
    whose scaled magnitude exceeds 6 become 6), sign kept (as in quant.py);
  * the E8M0 byte is clamped to [0, 254]: a block whose max is 0 or so small
    that its exponent falls below -127 gets byte 0 (X = 2^-127); bf16 inputs
    never need a byte above 252;
  * storage: codes[row][C/2] as in quant.py (channel 2j in the low nibble of
    byte j), scales[row][C/32] as E8M0 bytes.

X is a power of two, so x / X is exact in fp64 and the element rounding is
the same decision as for the exact quotient.
"""

import numpy as np

from .formats import bf16_decode, e2m1_decode, e2m1_encode

BLOCK = 32
E2M1_EMAX = 2                    # exponent of E2M1's largest normal value 6 = 1.5 * 2^2


def e8m0_decode(b):
    """E8M0 byte -> fp64 value 2^(b - 127); 0xFF -> NaN."""
    b = np.asarray(b).astype(np.int64)
    v = np.ldexp(1.0, b - 127)
    return np.where(b == 255, np.nan, v)


def shared_scale_byte(amax):
    """E8M0 byte of a block whose largest magnitude is amax (fp64 array): floor(log2(amax)) - 2 + 127,
    clamped to [0, 254]; 0 for amax == 0."""
    amax = np.asarray(amax, dtype=np.float64)
    m, ex = np.frexp(np.where(amax > 0, amax, 1.0))     # amax = m * 2^ex with m in [0.5, 1)
    e = ex - 1                                          # floor(log2(amax)), exact
    byte = np.clip(e - E2M1_EMAX + 127, 0, 254)
    return np.where(amax > 0, byte, 0).astype(np.uint8)


def quant_mxfp4(x_bits):
    """bf16 rows [T][C] (uint16 bit patterns, C a multiple of 32) -> (codes [T][C/2] u8, scales [T][C/32] u8)."""
    x_bits = np.asarray(x_bits, dtype=np.uint16)
    T, C = x_bits.shape
    assert C % BLOCK == 0
    x = bf16_decode(x_bits).reshape(T, C // BLOCK, BLOCK)
    scale = shared_scale_byte(np.abs(x).max(axis=-1))            # [T][C/32]
    X = e8m0_decode(scale)
    codes = e2m1_encode(x / X[..., None]).reshape(T, C)          # division by a power of two: exact
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    return packed, scale


def dequant_mxfp4(packed, scales, C):
    """(codes, E8M0 scales) -> values [T][C] in fp64: E2M1(code) * 2^(scale - 127) (exact)."""
    packed = np.asarray(packed, dtype=np.uint8)
    T = packed.shape[0]
    codes = np.empty((T, C), dtype=np.uint8)
    codes[:, 0::2] = packed[:, : C // 2] & 0xF
    codes[:, 1::2] = packed[:, : C // 2] >> 4
    X = e8m0_decode(np.asarray(scales, dtype=np.uint8)[:, : C // BLOCK])
    v = e2m1_decode(codes).reshape(T, C // BLOCK, BLOCK) * X[..., None]
    return v.reshape(T, C)


def bytes_per_token(C):
    """Stored bytes for C channels: C/2 code bytes plus C/32 scale bytes."""
    assert C % BLOCK == 0
    return C // 2 + C // BLOCK
