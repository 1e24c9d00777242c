"""Pins of the oracle's FP4 quantizer: exhaustive rounding checks, a worked example, invariants.

The scale rule S = RNE_E4M3(amax/6) is a reading (the pages only say "one E4M3
scale per 16 channels"); it is pinned by the invariants below, not by the pages.
"""

from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import quant as Q


def _bf16_bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _all_positive_finite_bf16():
    bits = np.arange(0x0001, 0x7F80, dtype=np.uint16)   # +denormals .. largest finite
    return bits, F.bf16_decode(bits)


def test_worked_group_example(golden_dir):
    lines = {}
    for line in open(f"{golden_dir}/quant_group_example.txt"):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        lines[k.strip()] = v.split()
    x = [float(t) for t in lines["x"]]
    bits = _bf16_bits(x).reshape(1, 16)
    packed, scale = Q.quant_fp4(bits)
    assert packed[0].tolist() == [int(t, 16) for t in lines["packed"]]
    assert scale[0].tolist() == [int(t, 16) for t in lines["scale"]]
    assert Q.unpack_codes(packed, 16)[0].tolist() == [int(t, 16) for t in lines["codes"]]


def test_division_never_moves_a_code_decision():
    """fp64 x/S rounds to E2M1 exactly as the exact real quotient does.

    For every positive finite bf16 x and every nonzero finite E4M3 scale S, the
    oracle's e2m1_encode(x/S) equals the threshold form evaluated with exact
    products t*S (t*S has <= 7 significant bits, so the comparison is exact).
    """
    _, x = _all_positive_finite_bf16()
    scales = F.e4m3_decode(np.arange(1, 0x7F))
    for S in scales:
        got = F.e2m1_encode(x / S)
        a = x
        ref = ((a > 0.25 * S).astype(int) + (a >= 0.75 * S) + (a > 1.25 * S) + (a >= 1.75 * S)
               + (a > 2.5 * S) + (a >= 3.5 * S) + (a > 5.0 * S))
        assert np.array_equal(got, ref.astype(np.uint8)), S


def test_scale_division_matches_exact_rational():
    """e4m3_encode(amax/6 in fp64) equals RNE of the exact rational amax/6, every bf16 amax."""
    bits, a = _all_positive_finite_bf16()
    got = F.e4m3_encode(a / 6.0)
    pos = [Fraction(float(v)) for v in F.e4m3_decode(np.arange(0x7F))]
    for i in range(0, a.size, 37):          # every 37th value: covers all exponents
        r = Fraction(float(a[i])) / 6
        if r >= 448:
            assert got[i] == 0x7E
            continue
        best = min(range(0x7F), key=lambda c: (abs(pos[c] - r), c % 2))
        assert got[i] == best, (a[i], got[i], best)


def test_every_group_code_is_nearest_scaled_value():
    """Brute force: each code is the nearest point of the scaled grid {+-m*S}, ties to even."""
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((4000, 64)) * np.exp(rng.uniform(-9, 9, (4000, 1)))).astype(np.float32)
    bits = _bf16_bits(x)
    packed, scales = Q.quant_fp4(bits)
    codes = Q.unpack_codes(packed, 64)
    xv = F.bf16_decode(bits).reshape(4000, 4, 16)
    S = F.e4m3_decode(scales)
    grid = F.E2M1_MAGNITUDES
    for r in range(0, 4000, 13):
        for g in range(4):
            s = S[r, g]
            for i in range(16):
                c = codes[r, 16 * g + i]
                if s == 0:
                    assert c == 0
                    continue
                a = abs(Fraction(float(xv[r, g, i])))
                dist = [abs(a - Fraction(float(m)) * Fraction(float(s))) for m in grid]
                best = min(range(8), key=lambda k: (dist[k], k % 2))
                assert (c & 7) == best
                assert (c >> 3) == int(np.signbit(xv[r, g, i]))


def test_idempotent_and_error_bound_on_normal_scales():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((20000, 32)) * np.exp(rng.uniform(-4, 6, (20000, 1)))).astype(np.float32)
    bits = _bf16_bits(x)
    packed, scales = Q.quant_fp4(bits)
    v = Q.dequant_fp4(packed, scales, 32)
    S = F.e4m3_decode(scales)
    normal = (S >= 2.0 ** -6) & (scales != 0x7E)
    # error bound |x - v| <= S (half the widest grid gap, 2*S)
    err = np.abs(F.bf16_decode(bits) - v).reshape(20000, 2, 16)
    assert np.all(err[normal] <= S[normal][:, None])
    # idempotence: re-quantizing the dequantized values reproduces codes and scale
    v_bits = _bf16_bits(v.astype(np.float32))
    assert np.array_equal(F.bf16_decode(v_bits), v)                  # exact in bf16
    p2, s2 = Q.quant_fp4(v_bits)
    g_codes = Q.unpack_codes(packed, 32).reshape(20000, 2, 16)
    g_codes2 = Q.unpack_codes(p2, 32).reshape(20000, 2, 16)
    assert np.array_equal(s2[normal], scales[normal])
    assert np.array_equal(g_codes2[normal], g_codes[normal])
    # with a normal unsaturated scale, the group's largest magnitude is code 7 (6*S)
    assert np.all((g_codes[normal] & 7).max(axis=-1) == 7)


def test_zero_and_saturated_scales():
    tiny = np.full((1, 16), 1e-3, dtype=np.float32)          # amax/6 < 2^-10 -> S = 0
    huge = np.full((1, 16), 1e4, dtype=np.float32)           # amax/6 > 448 -> S = 448
    huge[0, 3] = -3e4
    p, s = Q.quant_fp4(_bf16_bits(np.concatenate([tiny, -tiny, huge])))
    assert s[:, 0].tolist() == [0x00, 0x00, 0x7E]
    assert np.all(p[:2] == 0)                                 # zero scale: all codes 0x0
    c = Q.unpack_codes(p[2:], 16)[0]
    assert c[3] == 0xF and np.all(c[np.arange(16) != 3] == 0x7)   # clipped to +-6


def test_dequant_values_exact_in_bf16_and_fp16():
    codes = np.arange(16, dtype=np.uint8)
    for sc in range(0x7F):
        S = F.e4m3_decode(np.array([sc]))[0]
        v = F.e2m1_decode(codes) * S
        assert np.array_equal(v.astype(np.float16).astype(np.float64), v)
        bf = _bf16_bits(v.astype(np.float32))
        assert np.array_equal(F.bf16_decode(bf), v)


def test_bytes_per_token_accounting():
    # 4 bits per element plus one 8-bit scale per 16 channels = 4.5 bits/channel
    assert Q.bytes_per_token(512) == 256 + 32
    assert 2 * Q.bytes_per_token(128) == 144
    for C in (16, 64, 128, 512, 7168):
        assert Q.bytes_per_token(C) * 8 == C * 4.5
    rng = np.random.default_rng(0)
    p, s = Q.quant_fp4(_bf16_bits(rng.standard_normal((3, 512)).astype(np.float32)))
    assert p.nbytes + s.nbytes == 3 * 288
