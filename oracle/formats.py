"""Number formats of the FP4 main KV cache, written from their bit-level definitions.

[ezic] key points and "KVを捨てる、共有する、作り直す": the KV body is held in
FP4 E2M1 with one E4M3 scale per 16 channels. [jiwasawa] "FP4 メイン KV Cache":
the FP4 format is the OCP MX element type E2M1. The OCP 8-bit float E4M3 is the
"FN" flavour: bias 7, no infinities, the all-ones pattern is NaN, max 448.

Encoders are the definition of round-to-nearest-even onto the format's finite
value set: find the nearest representable value; on an exact tie take the
code whose least-significant mantissa bit is 0. Values beyond the largest
finite magnitude go to that magnitude (saturation).
"""

import numpy as np

# E2M1 magnitudes indexed by the low three code bits (exponent 2 bits,
# mantissa 1 bit, bias 1; exponent 0 is subnormal: 0 and 0.5).
E2M1_MAGNITUDES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E2M1_MAX = 6.0
E4M3_MAX = 448.0


def e2m1_decode(codes):
    """E2M1 code (low 4 bits) -> value in fp64. Bit 3 is the sign; 0x8 is -0."""
    c = np.asarray(codes).astype(np.uint8) & 0xF
    mag = E2M1_MAGNITUDES[c & 7]
    return np.where((c & 8) != 0, -mag, mag)


def e2m1_encode(r):
    """Round real values (fp64 array) to E2M1 codes, RNE with saturation.

    The sign bit of the code is the sign bit of r, so a negative value that
    rounds to zero gives 0x8 (reading: sign-preserving zero).
    """
    r = np.asarray(r, dtype=np.float64)
    assert np.all(np.isfinite(r)), "E2M1 encode takes finite values"
    # Everything above 6 saturates to 6; clamping first keeps the distances
    # below exact (a huge |r| would otherwise make every distance equal).
    a = np.minimum(np.abs(r), 2 * E2M1_MAX)
    dist = np.abs(a[..., None] - E2M1_MAGNITUDES)          # [..., 8], exact
    dmin = dist.min(axis=-1, keepdims=True)
    is_min = dist == dmin
    # Among the nearest magnitudes (one, or two on an exact tie) prefer the
    # even code (mantissa bit 0).
    idx = np.arange(8)
    even_pick = np.where(is_min & (idx % 2 == 0), idx, 99).min(axis=-1)
    any_pick = np.where(is_min, idx, 99).min(axis=-1)
    mag_code = np.where(even_pick < 99, even_pick, any_pick).astype(np.uint8)
    sign = np.signbit(r).astype(np.uint8) << 3
    return (mag_code | sign).astype(np.uint8)


def _e4m3_value_from_bits(b):
    s = (b >> 7) & 1
    e = (b >> 3) & 0xF
    m = b & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        v = m * 2.0 ** -9                      # subnormal: m/8 * 2^(1-7)
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


# Table of all 256 patterns, built once from the definition above.
E4M3_TABLE = np.array([_e4m3_value_from_bits(b) for b in range(256)], dtype=np.float64)
# Non-negative finite values in code order 0x00..0x7E; this order is ascending.
_E4M3_POS = E4M3_TABLE[:0x7F].copy()
assert np.all(np.diff(_E4M3_POS) > 0)


def e4m3_decode(b):
    """E4M3FN byte -> value in fp64 (NaN for 0x7F / 0xFF)."""
    return E4M3_TABLE[np.asarray(b).astype(np.uint8)]


def e4m3_encode(r):
    """Round real values (fp64 array) to E4M3FN bytes, RNE, saturating at 448.

    Finite inputs only. The two neighbours of |r| in the ascending value
    table are found with a binary search; the nearer one wins, an exact tie
    goes to the even code. |r| > 448 saturates to 0x7E (never NaN).
    """
    r = np.asarray(r, dtype=np.float64)
    assert np.all(np.isfinite(r)), "E4M3 encode takes finite values"
    a = np.abs(r)
    hi = np.clip(np.searchsorted(_E4M3_POS, a, side="left"), 0, 0x7E)   # first value >= a
    lo = np.clip(hi - 1, 0, 0x7E)
    d_hi = np.abs(_E4M3_POS[hi] - a)
    d_lo = np.abs(a - _E4M3_POS[lo])
    pick = np.where(d_lo < d_hi, lo, hi)
    tie = (d_lo == d_hi) & (lo != hi)
    pick = np.where(tie, np.where(lo % 2 == 0, lo, hi), pick)
    pick = np.where(a >= E4M3_MAX, 0x7E, pick)
    sign = np.signbit(r).astype(np.uint8) << 7
    return (pick.astype(np.uint8) | sign).astype(np.uint8)


def bf16_decode(bits):
    """bfloat16 bit patterns (uint16) -> fp64, exact."""
    b = np.asarray(bits).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def f32_decode(bits_or_values):
    """fp32 values (float32 array) -> fp64, exact."""
    return np.asarray(bits_or_values, dtype=np.float32).astype(np.float64)


def decode(arr, dtype):
    """Decode a stored array of dtype 'f32' | 'bf16' | 'e4m3' to fp64."""
    if dtype == "f32":
        return f32_decode(arr)
    if dtype == "bf16":
        return bf16_decode(arr)
    if dtype == "e4m3":
        return e4m3_decode(arr)
    raise ValueError(f"unknown dtype {dtype}")
