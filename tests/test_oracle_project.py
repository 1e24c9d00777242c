"""Pins of the oracle's KV write path (CED projection, bf16 rounding of the activation).

The projection is a library matmul in fp64, checked against exact integer brute force on small
integer-valued inputs; the bf16 rounding against torch's fp32 -> bf16 cast (a library routine) on fp32
values and against exact rationals on fp64 values next to bf16 rounding midpoints."""

from fractions import Fraction

import numpy as np
import torch

from oracle import formats as F
from oracle import project as PJ


def _bf16(vals):
    return torch.tensor(np.asarray(vals, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_projection_equals_integer_brute_force():
    rng = np.random.default_rng(0)
    T, D, C = 5, 37, 9
    h = rng.integers(-20, 21, (T, D))
    w = rng.integers(-9, 10, (D, C))
    got = PJ.project_exact(_bf16(h), _bf16(w))
    for t in range(T):
        for c in range(C):
            assert got[t, c] == sum(int(h[t, k]) * int(w[k, c]) for k in range(D))


def test_round_to_bf16_equals_torch_on_fp32_values():
    rng = np.random.default_rng(1)
    wide = rng.standard_normal(100000) * np.power(10.0, rng.uniform(-40, 38, 100000))
    wide = wide[np.abs(wide) < 3.38e38]
    x = np.concatenate([wide.astype(np.float32), np.arange(0x00000000, 0x00200000, 7, dtype=np.uint32).view(np.float32)])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(PJ.round_to_bf16(x.astype(np.float64)), ref)


def test_round_to_bf16_next_to_midpoints_equals_exact_rationals():
    rng = np.random.default_rng(2)
    base = rng.integers(0x0080, 0x7F00, 2000).astype(np.uint16)       # positive normal bf16 values
    lo = F.bf16_decode(base)
    hi = F.bf16_decode(base + 1)
    mid = (lo + hi) / 2                                               # exact in fp64
    for delta in (-2.0 ** -40, 0.0, 2.0 ** -40):
        x = mid + delta * mid
        got = PJ.round_to_bf16(x)
        for i in range(0, len(x), 97):
            fx, flo, fhi = Fraction(float(x[i])), Fraction(float(lo[i])), Fraction(float(hi[i]))
            if fx - flo < fhi - fx:
                want = base[i]
            elif fx - flo > fhi - fx:
                want = base[i] + 1
            else:
                want = base[i] if base[i] % 2 == 0 else base[i] + 1
            assert got[i] == want, (i, x[i])
    assert PJ.round_to_bf16(np.array([-0.0]))[0] == 0x8000
