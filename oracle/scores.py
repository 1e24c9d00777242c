"""Indexer scores: indexer query dotted with indexer keys.

[jiwasawa] CSA2: a Full layer computes its own indexer Q and fresh top-K
positions; a Reindex layer re-scores with its own Q against the indexer K it
shares with an earlier layer. [zaikei] "■CSA2とFP4でキャッシュを圧縮": the
retrieval keys are shared across layers. The pages give no score formula.

Reading: score[t] = sum_d q[d] * k[t][d], the plain dot product (no ReLU, no
head weights, no scaling), taken as the EXACT real sum rounded once to fp32
(round-to-nearest-even). That value is independent of any summation order,
so a kernel that computes it exactly can match it bit for bit, and the top-K
decision is taken on the same fp32 values on both sides.

Computation here:
  1. inputs decoded exactly to fp64;
  2. each product q[d]*k[t][d] is exact in fp64 (the operands have at most
     24 significant bits each, so a product has at most 48 <= 53);
  3. the products are summed in fp64 where that sum is provably exact: if all
     products of a key are integer multiples of a power of two u and the sum
     of their magnitudes is below 2^52 * u, every partial sum is an integer
     multiple of u below 2^53 * u, hence representable, so no addition rounds;
  4. keys without that certificate are summed as exact rationals
     (fractions.Fraction) and rounded to fp32 by hand.
Non-finite inputs (NaN keys, or infinities in fp32 / bf16 operands) follow
IEEE-754 addition: a score is NaN when any product is NaN or products of
both signs are infinite, otherwise the infinity; the fp64 sum of such a row
gives exactly that, whatever the order.
"""

from fractions import Fraction

import numpy as np

from .formats import decode

_CHUNK = 32768


def round_rational_to_f32(x):
    """Exact rational -> nearest fp32 (ties to even), including subnormals."""
    x = Fraction(x)
    if x == 0:
        return np.float32(0.0)
    neg = x < 0
    a = -x if neg else x
    e = a.numerator.bit_length() - a.denominator.bit_length()
    # now 2^(e-1) < a < 2^(e+1); settle on 2^e <= a < 2^(e+1)
    if Fraction(2) ** e > a:
        e -= 1
    if e > 127:
        return np.float32(-np.inf if neg else np.inf)
    e = max(e, -126)                       # below 2^-126 the grid is the subnormal one
    ulp = Fraction(2) ** (e - 23)
    q = a / ulp
    n = q.numerator // q.denominator
    frac = q - n
    if frac > Fraction(1, 2) or (frac == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = n * ulp
    if v >= Fraction(2) ** 128:
        return np.float32(-np.inf if neg else np.inf)
    f = float(v)                            # n <= 2^24 significant bits: exact
    return np.float32(-f if neg else f)


def _certified_exact(prods):
    """Per row of `prods` (exact fp64 products): True if their fp64 sum is exact."""
    a = np.abs(prods)
    m, e = np.frexp(a)                                 # a = m * 2^e, m in [0.5, 1)
    mi = (m * 2.0 ** 53).astype(np.int64)              # integer significand
    low = mi & -mi                                     # lowest set bit of it
    low_e = np.frexp(low.astype(np.float64))[1] - 1    # log2(low), exact
    unit_e = np.where(a > 0, e - 53 + low_e, np.iinfo(np.int32).max)
    u = unit_e.min(axis=1)                              # exponent of the common unit
    total = a.sum(axis=1)
    all_zero = u == np.iinfo(np.int32).max
    bound = np.ldexp(1.0, np.clip(u, -1074, 970).astype(np.int32) + 52)
    return all_zero | (total < bound)


def exact_dot_f32(q64, k64):
    """q64: (d,) fp64, k64: (n, d) fp64 -> (n,) fp32 = RN32(exact dot products)."""
    q64 = np.asarray(q64, dtype=np.float64)
    k64 = np.asarray(k64, dtype=np.float64)
    n = k64.shape[0]
    out = np.empty(n, dtype=np.float32)
    for s in range(0, n, _CHUNK):
        with np.errstate(invalid="ignore"):     # inf - inf and inf * 0 are NaN by intent
            prods = k64[s:s + _CHUNK] * q64[None, :]
            sums = prods.sum(axis=1)
        finite = np.isfinite(prods).all(axis=1)
        # a row with a non-finite product keeps its fp64 sum (IEEE: NaN or the infinity)
        ok = ~finite | _certified_exact(np.where(finite[:, None], prods, 0.0))
        out[s:s + _CHUNK] = sums.astype(np.float32)
        for i in np.nonzero(~ok)[0]:
            total = sum((Fraction(float(p)) for p in prods[i]), Fraction(0))
            out[s + i] = round_rational_to_f32(total)
    return out


def index_scores(q_idx, q_dtype, k_idx, k_dtype, q_pos=None):
    """Scores of one indexer query against keys [n][d_idx].

    q_idx: (d_idx,) stored values (fp32 array or bf16 bits); k_idx: (n, d_idx)
    stored values (fp32, bf16 bits or E4M3 bytes). With q_pos given, positions
    after q_pos are masked to -inf (causal reading for prefill queries).
    Returns fp32 scores (n,).
    """
    q64 = decode(np.asarray(q_idx), q_dtype)
    k64 = decode(np.asarray(k_idx), k_dtype)
    s = exact_dot_f32(q64, k64)
    if q_pos is not None:
        s = s.copy()
        s[np.arange(s.shape[0]) > q_pos] = -np.inf
    return s


def pool_scores(q_idx, q_dtype, k_idx, k_dtype, pool):
    """Reindex scoring: the query against the shared keys at the pool positions only.

    [jiwasawa] CSA2, Hierarchical Sparse Indexer: later Reindex layers search
    only inside the candidate pool. Pool entries of -1 (padding) score -inf.
    """
    pool = np.asarray(pool, dtype=np.int64)
    valid = pool >= 0
    s = np.full(pool.shape[0], -np.inf, dtype=np.float32)
    if valid.any():
        s[valid] = index_scores(q_idx, q_dtype, np.asarray(k_idx)[pool[valid]], k_dtype)
    return s
