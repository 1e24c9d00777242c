"""Pins of the oracle's indexer scores: exact-rational brute force and a library matmul."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle import scores as S
from synth import to_bf16_bits, to_e4m3_bytes


def test_round_rational_to_f32_matches_numpy_cast():
    rng = np.random.default_rng(0)
    vals = np.concatenate([
        rng.standard_normal(3000) * np.exp(rng.uniform(-100, 100, 3000)),
        rng.standard_normal(500) * 1e-40,                      # fp32 subnormal range
        [1e-45, 3e38, -3e38, 0.5, 1.0 + 2.0 ** -24, 1.0 + 3 * 2.0 ** -24],   # ties
    ])
    for v in vals:
        assert S.round_rational_to_f32(Fraction(float(v))) == np.float32(v), v
    assert np.isinf(S.round_rational_to_f32(Fraction(2) ** 130))


def _brute(q64, k64):
    out = np.empty(k64.shape[0], dtype=np.float32)
    for t in range(k64.shape[0]):
        tot = sum((Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q64, k64[t])), Fraction(0))
        out[t] = S.round_rational_to_f32(tot)
    return out


@pytest.mark.parametrize("qd,kd", [("f32", "f32"), ("bf16", "e4m3"), ("bf16", "bf16"), ("f32", "e4m3")])
def test_exact_dot_vs_rational_brute_force(qd, kd):
    rng = np.random.default_rng(11)
    d, n = 64, 300
    q = rng.standard_normal(d).astype(np.float32)
    k = rng.standard_normal((n, d)).astype(np.float32)
    q[3] *= 1e-9                                    # widen the exponent spread
    qs = q if qd == "f32" else to_bf16_bits(q)
    ks = k if kd == "f32" else (to_bf16_bits(k) if kd == "bf16" else to_e4m3_bytes(k))
    got = S.index_scores(qs, qd, ks, kd)
    ref = _brute(F.decode(qs, qd), F.decode(ks, kd))
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_fallback_path_is_exercised_and_exact():
    # huge cancellation: fp64 summation would round; the certificate must reject it
    q = np.array([1e30, 1.0, -1e30, 3.0], dtype=np.float32)
    k = np.array([[1.0, 1.0, 1.0, 2.0 ** -20], [3.0, -1.0, 3.0, 1.0]], dtype=np.float32)
    q64, k64 = F.decode(q, "f32"), F.decode(k, "f32")
    assert not S._certified_exact(k64 * q64[None, :]).all()
    got = S.exact_dot_f32(q64, k64)
    assert np.array_equal(got, _brute(q64, k64))
    assert got[0] == np.float32(1.0 + 3 * 2.0 ** -20)


def test_scores_agree_with_library_matmul():
    rng = np.random.default_rng(5)
    q = to_bf16_bits(rng.standard_normal(64).astype(np.float32))
    k = to_e4m3_bytes(rng.standard_normal((5000, 64)).astype(np.float32))
    got = S.index_scores(q, "bf16", k, "e4m3").astype(np.float64)
    ref = np.matmul(F.decode(k, "e4m3"), F.decode(q, "bf16"))      # fp64 BLAS
    ulp = np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)
    assert np.all(np.abs(got - ref) <= 0.5 * ulp + 1e-300)


def test_causal_mask_and_pool_scores():
    rng = np.random.default_rng(2)
    q = rng.standard_normal(64).astype(np.float32)
    k = rng.standard_normal((100, 64)).astype(np.float32)
    s = S.index_scores(q, "f32", k, "f32", q_pos=40)
    assert np.all(np.isneginf(s[41:])) and np.all(np.isfinite(s[:41]))
    pool = np.array([3, 7, 50, -1])
    ps = S.pool_scores(q, "f32", k, "f32", pool)
    full = S.index_scores(q, "f32", k, "f32")
    assert ps[:3].tolist() == full[[3, 7, 50]].tolist() and np.isneginf(ps[3])


def test_non_finite_keys_follow_ieee_addition():
    """IEEE-754 addition on non-finite terms: one NaN product makes the score NaN; infinite products of
    one sign give that infinity; of both signs, NaN. The finite rows of the same call are unaffected."""
    rng = np.random.default_rng(9)
    q = rng.uniform(0.5, 1.0, 64).astype(np.float32)                # positive: products keep the keys' signs
    k = rng.standard_normal((6, 64)).astype(np.float32)
    k[1, 7] = np.nan                                                 # one NaN among finite terms
    k[2, 3] = np.inf                                                 # +inf among finite terms
    k[3, 3], k[3, 9] = np.inf, -np.inf                               # both infinities
    k[4, :] = np.nan                                                 # a whole NaN row
    k[5, 0] = -np.inf
    s = S.index_scores(q, "f32", k, "f32")
    assert np.isnan(s[1]) and np.isnan(s[3]) and np.isnan(s[4])
    assert s[2] == np.inf and s[5] == -np.inf
    assert s[0] == S.index_scores(q, "f32", k[:1], "f32")[0]
    # an E4M3 NaN byte (0x7F) in one channel of a key
    kb = to_e4m3_bytes(rng.standard_normal((3, 64)).astype(np.float32))
    kb[1, 10] = 0x7F
    qb = to_bf16_bits(rng.standard_normal(64).astype(np.float32))
    sb = S.index_scores(qb, "bf16", kb, "e4m3")
    assert np.isfinite(sb[0]) and np.isnan(sb[1]) and np.isfinite(sb[2])
