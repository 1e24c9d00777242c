"""Pins of the oracle's number formats against the format definitions and torch's casts.

The E2M1 and E4M3 value tables are checked against the OCP tables stored in
tests/golden (cited there), and the encoders against (a) the closed-form
threshold description of round-to-nearest-even and (b) torch's float8_e4m3fn
and bfloat16 casts, which are independent library implementations.
"""

import numpy as np
import pytest
import torch

from oracle import formats as F


def _read_table(path):
    rows = []
    for line in open(path):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        c, v = line.split()
        rows.append((int(c, 16), float(v)))
    return rows


def test_e2m1_table_matches_ocp(golden_dir):
    rows = _read_table(f"{golden_dir}/e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = F.e2m1_decode(np.array([code]))[0]
        assert got == val and np.signbit(got) == np.signbit(val), (code, got, val)


def test_e2m1_all_codes_round_trip():
    codes = np.arange(16, dtype=np.uint8)
    assert np.array_equal(F.e2m1_encode(F.e2m1_decode(codes)), codes)


def _e2m1_threshold_form(r):
    # Closed-form RNE onto {0,.5,1,1.5,2,3,4,6}: midpoints 0.25,0.75,1.25,1.75,2.5,3.5,5;
    # at a midpoint the even code wins, i.e. strict '>' where the lower neighbour is even
    # (0.25, 1.25, 2.5, 5) and '>=' where the upper neighbour is even (0.75, 1.75, 3.5).
    a = np.abs(r)
    m = ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75)
         + (a > 2.5) + (a >= 3.5) + (a > 5.0))
    return (m | (np.signbit(r).astype(int) << 3)).astype(np.uint8)


def test_e2m1_encode_matches_threshold_form():
    mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])
    vals = np.concatenate([
        np.linspace(-8, 8, 200001),
        mids, -mids, np.nextafter(mids, 0), np.nextafter(mids, 10),
        F.E2M1_MAGNITUDES, -F.E2M1_MAGNITUDES, [1e9, -1e9, 6.0000001, -0.0],
    ])
    assert np.array_equal(F.e2m1_encode(vals), _e2m1_threshold_form(vals))


def test_e2m1_negative_to_zero_keeps_sign():
    assert F.e2m1_encode(np.array([-0.1]))[0] == 0x8
    assert F.e2m1_encode(np.array([-0.0]))[0] == 0x8
    assert F.e2m1_encode(np.array([0.1]))[0] == 0x0


def test_e4m3_decode_all_patterns_vs_torch():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = b.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]


def test_e4m3_landmarks(golden_dir):
    for code, val in _read_table(f"{golden_dir}/e4m3_landmarks.txt"):
        got = F.e4m3_decode(np.array([code]))[0]
        if np.isnan(val):
            assert np.isnan(got)
        else:
            assert got == val and np.signbit(got) == np.signbit(val)


def test_e4m3_encode_round_trip_all_finite():
    b = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(b)), b)


def test_e4m3_encode_vs_torch_random_and_ties():
    rng = np.random.default_rng(1)
    pos = F.e4m3_decode(np.arange(0x7F))
    mids = (pos[:-1] + pos[1:]) / 2                      # every rounding midpoint
    vals = np.concatenate([
        rng.standard_normal(200000) * 10, rng.uniform(-448, 448, 200000),
        np.exp(rng.uniform(-12, 6, 100000)), mids, -mids,
        np.nextafter(mids, 0), np.nextafter(mids, 1000), [0.0, -0.0, 448.0, -448.0],
    ]).astype(np.float32).astype(np.float64)             # values torch can take exactly
    ref = torch.from_numpy(vals.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = F.e4m3_encode(vals)
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates():
    got = F.e4m3_encode(np.array([448.0, 460.0, 464.0, 500.0, 1e30, -1e30]))
    assert got.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE]


def test_e4m3_encode_underflow_ties():
    # 2^-10 is the midpoint between 0 and 2^-9: tie -> even code 0x00.
    # 3*2^-10 is the midpoint between 2^-9 (0x01) and 2^-8 (0x02): tie -> 0x02.
    got = F.e4m3_encode(np.array([2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -11]))
    assert got.tolist() == [0x00, 0x02, 0x00]


def test_bf16_decode_all_patterns_vs_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = F.bf16_decode(bits)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])


@pytest.mark.parametrize("dtype", ["f32", "bf16", "e4m3"])
def test_decode_dispatch(dtype):
    if dtype == "f32":
        x = np.array([1.5, -2.25], dtype=np.float32)
        assert F.decode(x, dtype).tolist() == [1.5, -2.25]
    elif dtype == "bf16":
        assert F.decode(np.array([0x3FC0], dtype=np.uint16), dtype).tolist() == [1.5]
    else:
        assert F.decode(np.array([0x3C], dtype=np.uint8), dtype).tolist() == [1.5]
