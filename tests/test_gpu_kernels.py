"""GPU parity of each libcsa2 call against the oracle, at sizes that span several
tiles / chunks and a ragged tail, plus the edge cases of each step."""

import ctypes
import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import formats as F
from oracle import quant as OQ
from oracle import scores as OS
from oracle.attention import sparse_attn as o_attn
from oracle.topk import topk as o_topk
from tests.parity import (ATTN_TOL, compare_topk, dev_bf16, dev_f32, dev_key, dev_u8, host, max_rel_err_rows)

pytestmark = pytest.mark.gpu


def _sync():
    torch.cuda.synchronize()


# ---------------------------------------------------------------- formats

def test_e4m3_key_decode_all_bytes():
    """Every E4M3 byte at every key lane position: score of a unit query = the decoded byte."""
    N, d = 256, 64
    keys = np.repeat(np.arange(256, dtype=np.uint8)[:, None], d, axis=1)[None]      # [1][256][64]
    q = np.eye(d, dtype=np.float32)[None]                                            # [1][64][64]
    s = host(C.index_full(dev_f32(q), dev_u8(keys).view(torch.float8_e4m3fn)))
    ref = F.e4m3_decode(np.arange(256)).astype(np.float32)
    for i in range(d):
        nan = np.isnan(ref)
        assert np.array_equal(np.isnan(s[0, i]), nan)
        assert np.array_equal(s[0, i][~nan], ref[~nan]), i


# ----------------------------------------------------------- quantization

def _finite_bf16_rows(C_):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    b = bits[finite]
    rng = np.random.default_rng(0)
    b = b[rng.permutation(b.size)]
    n = b.size // C_ * C_
    return b[:n].reshape(-1, C_)


@pytest.mark.parametrize("C_", [16, 128, 512])
def test_quant_bit_exact_all_bf16_values(C_):
    x = _finite_bf16_rows(C_)
    codes, scales = C.kv_quant_fp4(dev_bf16(x))
    rc, rs = OQ.quant_fp4(x)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


def test_quant_every_scale_with_every_value_up_to_its_group_max():
    """Every (x, S) pair the quantizer can meet: for each positive finite E4M3 scale S, groups whose
    maximum is 6*S (so the group's scale is S) hold, in their other 15 slots, every finite bf16 x with
    |x| <= 6*S, both signs. Codes and scales must equal the oracle's bit for bit."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    mag = F.bf16_decode(np.where(finite, bits & np.uint16(0x7FFF), 0).astype(np.uint16))
    groups = []
    for sc in range(1, 0x7F):
        S = float(F.e4m3_decode(np.array([sc], dtype=np.uint8))[0])
        top = np.float32(6.0 * S)
        tb = synth.to_bf16_bits(np.array([top], dtype=np.float32))[0]
        if F.bf16_decode(np.array([tb]))[0] != top:      # 6*S not a bf16: this scale is not reached this way
            continue
        vals = bits[finite & (mag <= top)]
        pad = (-vals.size) % 15
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 15)
        groups.append(np.concatenate([np.full((vals.shape[0], 1), tb, dtype=np.uint16), vals], axis=1))
    g = np.concatenate(groups)
    rows = (g.shape[0] + 31) // 32
    g = np.concatenate([g, np.zeros((rows * 32 - g.shape[0], 16), dtype=np.uint16)]).reshape(rows, 512)
    codes, scales = C.kv_quant_fp4(dev_bf16(g))
    rc, rs = OQ.quant_fp4(g)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)
    assert len(set(rs.ravel().tolist())) >= 100            # nearly every scale code occurs


def test_quant_bit_exact_log_uniform_rows_and_dequant():
    cfg = synth.small("quant_1m_x512", row_block=2048)
    x = np.concatenate([synth.quant_rows(cfg, 0), synth.quant_rows(cfg, 7)])[:3001]   # ragged row count
    codes, scales = C.kv_quant_fp4(dev_bf16(x))
    rc, rs = OQ.quant_fp4(x)
    assert np.array_equal(host(scales), rs) and np.array_equal(host(codes), rc)
    hs = host(scales)
    assert (hs == 0).any() and (hs == 0x7E).any()          # both scale extremes are exercised
    y = C.kv_dequant_fp4(codes, scales, 512)
    ref = OQ.dequant_fp4(rc, rs, 512)
    got = host(y.view(torch.int16)).view(np.uint16)
    assert np.array_equal(F.bf16_decode(got), ref)


def test_dequant_every_code_and_scale():
    rng = np.random.default_rng(3)
    T = 4096
    codes = rng.integers(0, 256, (T, 64), dtype=np.uint8)
    scales = rng.integers(0, 0x7F, (T, 8), dtype=np.uint8)        # every finite positive scale
    y = C.kv_dequant_fp4(dev_u8(codes), dev_u8(scales), 128)
    got = F.bf16_decode(host(y.view(torch.int16)).view(np.uint16))
    ref = OQ.dequant_fp4(codes, scales, 128)
    assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref))


def test_quant_strided_into_kv_records():
    rng = np.random.default_rng(5)
    N = 1000
    kb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    vb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32) * 3)
    cache = C.KVCache(1, N)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    kc, ks = OQ.quant_fp4(kb)
    vc, vs = OQ.quant_fp4(vb)
    codes, scales = host(cache.codes), host(cache.scales)
    assert np.array_equal(codes[:, :64], kc) and np.array_equal(codes[:, 64:], vc)
    assert np.array_equal(scales[:, :8], ks) and np.array_equal(scales[:, 8:], vs)


# ------------------------------------------------------------------ scores

@pytest.mark.parametrize("qd,kd,d", [("bf16", "e4m3", 64), ("f32", "f32", 64), ("bf16", "bf16", 128),
                                     ("f32", "e4m3", 128)])
def test_index_full_scores(qd, kd, d):
    cfg = synth.small("full_b64_n131072", N=3001, d_idx=d, q_idx_dtype=qd, k_idx_dtype=kd)
    B, Q = 2, 3
    qs = np.stack([synth.q_idx(cfg, 0, b, Q=Q) for b in range(B)])
    ks = np.stack([synth.k_idx(cfg, b) for b in range(B)])
    q_pos = np.array([[100, 3000, 2047], [0, 1500, 2999]], dtype=np.int64)
    got = host(C.index_full(dev_key(qs, qd), dev_key(ks, kd), q_pos=torch.from_numpy(q_pos).cuda()))
    for b in range(B):
        for i in range(Q):
            ref = OS.index_scores(qs[b, i], qd, ks[b], kd, q_pos=int(q_pos[b, i]))
            assert np.array_equal(got[b, i].view(np.uint32), ref.view(np.uint32)), (b, i)


def test_index_full_scores_with_one_nan_channel():
    """Keys with an E4M3 NaN byte (0x7F or 0xFF) in one channel among finite ones score NaN, as IEEE
    addition gives; every other key keeps its bit-exact score."""
    cfg = synth.small("full_b64_n131072", N=1000, d_idx=64)
    rng = np.random.default_rng(13)
    q = synth.q_idx(cfg, 0, 0, Q=2)
    k = synth.k_idx(cfg, 0).copy()
    rows = rng.choice(1000, size=37, replace=False)
    k[rows, rng.integers(0, 64, 37)] = rng.choice(np.array([0x7F, 0xFF], dtype=np.uint8), 37)
    got = host(C.index_full(dev_key(q[None], "bf16"), dev_key(k[None], "e4m3")))[0]
    for i in range(2):
        ref = OS.index_scores(q[i], "bf16", k, "e4m3")
        nan = np.isnan(ref)
        assert nan.sum() == 37 and np.array_equal(np.isnan(got[i]), nan), i
        assert np.array_equal(got[i][~nan].view(np.uint32), ref[~nan].view(np.uint32)), i


def _near_midpoint_f32_keys(q, n, rng, mode):
    """fp32 keys whose exact dot product with q sits on, or a hair off, a rounding midpoint between two
    fp32 values (built with exact rationals): a plain fp64 sum of 48-bit products rounds these wrongly."""
    from fractions import Fraction
    keys = rng.standard_normal((n, q.size)).astype(np.float32)
    for t in range(n):
        keys[t, -1] = 0.0
        part = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q[:-1], keys[t, :-1]))
        f = np.float32(float(part))
        mid = (Fraction(float(f)) + Fraction(float(np.nextafter(f, np.float32(np.inf))))) / 2
        want = mid - part
        if mode == "above":
            want += Fraction(1, 2 ** 60)
        elif mode == "below":
            want -= Fraction(1, 2 ** 60)
        keys[t, -1] = np.float32(float(want / Fraction(float(q[-1]))))
    return keys


@pytest.mark.parametrize("mode", ["above", "below", "on"])
def test_index_full_f32_scores_near_rounding_midpoints(mode):
    rng = np.random.default_rng({"above": 1, "below": 2, "on": 3}[mode])
    q = rng.standard_normal(64).astype(np.float32)
    q[-1] = np.float32(1.0)
    keys = _near_midpoint_f32_keys(q, 160, rng, mode)
    got = host(C.index_full(dev_f32(q[None, None]), dev_f32(keys[None])))[0, 0]
    ref = OS.index_scores(q, "f32", keys, "f32")
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))


def test_index_reindex_scores_with_padding():
    cfg = synth.small("stack_b32_n262144", N=5000)
    B, P = 3, 777
    rng = np.random.default_rng(9)
    qs = np.stack([synth.q_idx(cfg, 1, b)[0] for b in range(B)])
    ks = np.stack([synth.k_idx(cfg, b) for b in range(B)])
    pool = np.sort(rng.choice(5000, size=(B, P)), axis=1).astype(np.int32)
    pool[:, -5:] = -1
    pool[1, 3] = 5000                                       # out of range -> -inf
    got = host(C.index_reindex(dev_bf16(qs), dev_key(ks, "e4m3"), torch.from_numpy(pool).cuda()))
    for b in range(B):
        ref = OS.pool_scores(qs[b], "bf16", ks[b], "e4m3", np.where(pool[b] >= 5000, -1, pool[b]))
        assert np.array_equal(got[b].view(np.uint32), ref.view(np.uint32))


# ------------------------------------------------------------------- top-K

def _scores_with_ties(rng, rows, n, kind):
    if kind == "ties":
        s = rng.integers(-50, 50, (rows, n)).astype(np.float32)
    elif kind == "few":                                     # thousands of copies of each of 7 values
        s = rng.integers(-3, 4, (rows, n)).astype(np.float32)
    elif kind == "equal":
        s = np.full((rows, n), 1.25, dtype=np.float32)
    elif kind.startswith("bin"):                            # bin20k: 20,000 keys in [1, 1.25), one top-digit bin
        c = int(kind[3:].split("k")[0]) * 1000
        s = (rng.standard_normal((rows, n)) * 0.1).astype(np.float32)
        for r in range(rows):
            at = rng.choice(n, c, replace=False)
            s[r, at] = (1.0 + rng.integers(0, 16, c) / 64.0 if kind.endswith("kt")     # 16 values, many ties
                        else rng.uniform(1.0, 1.25, c)).astype(np.float32)
    elif kind == "inf":                                     # the top-K is a subset of many +inf
        s = rng.standard_normal((rows, n)).astype(np.float32)
        s[rng.random((rows, n)) < 0.3] = np.inf
    else:
        s = rng.standard_normal((rows, n)).astype(np.float32)
    m = rng.random((rows, n))
    s[m < 0.02] = -np.inf
    s[(m >= 0.02) & (m < 0.03)] = np.nan
    s[(m >= 0.03) & (m < 0.04)] = -0.0
    s[(m >= 0.04) & (m < 0.05)] = 0.0
    return s


@pytest.mark.parametrize("rows,n,K,kind", [
    (1, 100, 10, "ties"), (3, 5000, 64, "ties"), (2, 70001, 2048, "normal"), (2, 70001, 2048, "ties"),
    (1, 300000, 8192, "normal"), (4, 40000, 40000, "ties"), (2, 1000, 1500, "normal"),
    (2, 65536, 100, "equal"), (5, 33, 1, "normal"),
    (2, 70001, 50000, "normal"),    # most keys are candidates: waves fall back from extraction
    (2, 70001, 2048, "few"),        # > 1024 keys equal to the threshold: low-bit histogram fallback
    # rows of 2..16 chunks, which exchange suffix sums only
    (32, 70001, 2048, "normal"), (32, 70001, 50000, "normal"), (32, 70001, 2048, "few"),
    (32, 70001, 2048, "inf"), (16, 262144, 100, "equal"), (20, 100000, 3000, "ties"),
    # 16K..32K keys in the threshold's top-digit bin: the row list is resolved in two batches
    (2, 300000, 8192, "bin20k"), (1, 1000000, 2048, "bin30k"), (3, 262144, 8192, "bin24kt"),
    (1, 300000, 8192, "bin40k"),    # more than the list holds: the radix path
    # rows of 16 or more chunks (a multiple of 8): even chunks take more entries than odd ones
    (4, 1043576, 2048, "normal"), (16, 262144, 2048, "ties"), (4, 1048576, 8192, "bin20k")])
def test_topk_matches_oracle(rows, n, K, kind):
    rng = np.random.default_rng(rows * 1000 + n + K)
    s = _scores_with_ties(rng, rows, n, kind)
    idx, sel = C.topk(dev_f32(s), K, want_scores=True)
    idx, sel = host(idx), host(sel)
    for r in range(rows):
        ri, rsel = o_topk(s[r], K)
        assert np.array_equal(idx[r], ri), (r, np.nonzero(idx[r] != ri)[0][:10])
        assert np.array_equal(np.isnan(sel[r]), np.isnan(rsel))
        ok = ~np.isnan(rsel)
        assert np.array_equal(sel[r][ok], rsel[ok])            # -0 and +0 compare equal


def test_topk_candidate_positions_and_strides():
    rng = np.random.default_rng(4)
    rows, n, K = 3, 9000, 300
    s = rng.integers(-20, 20, (rows, n + 17)).astype(np.float32)
    cand = np.stack([np.sort(rng.choice(10 ** 6, n, replace=False)) for _ in range(rows)]).astype(np.int32)
    sd = dev_f32(s)[:, :n]                                   # row stride n+17
    idx = host(C.topk(sd, K, cand=torch.from_numpy(cand).cuda()))
    for r in range(rows):
        ri, _ = o_topk(s[r, :n], K, positions=cand[r])
        assert np.array_equal(idx[r], ri)


def test_topk_repeat_calls_reuse_workspace():
    rng = np.random.default_rng(8)
    s = dev_f32(rng.standard_normal((6, 50000)).astype(np.float32))
    a = host(C.topk(s, 512))
    for _ in range(3):
        assert np.array_equal(host(C.topk(s, 512)), a)
    ws = C.workspace(0, s.device, "topk")
    assert int(ws.view(torch.int32)[:64].abs().sum().item()) == 0        # status word clean


def test_one_workspace_serves_calls_of_any_shape():
    """One zero-filled buffer used in turn by top-K and attention calls of different shapes: the control
    words sit at fixed offsets and every call leaves them zero, so no call sees another's data as counters."""
    rng = np.random.default_rng(21)
    cases = [(2, 65536, 100, "equal"), (6, 50000, 512, "normal"), (1, 300000, 8192, "normal"),
             (40, 9000, 64, "ties"), (2, 65536, 100, "equal")]
    scores = [_scores_with_ties(rng, r, n, kind) for r, n, _, kind in cases]
    N = 6000
    cache, okv = _kv_case(N, 77)
    attn_cases = []
    for Q, K in ((3, 2048), (300, 256), (2, 100)):
        qb = synth.to_bf16_bits(rng.standard_normal((1, Q, 16, 128)).astype(np.float32))
        idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
        attn_cases.append((qb, idx))
    need = []
    for (r, n, K, _) in cases:
        nb = ctypes.c_size_t(0)
        C.lib().csa2_topk_workspace_bytes(r, n, K, ctypes.byref(nb))
        need.append(nb.value)
    for qb, idx in attn_cases:
        nb = ctypes.c_size_t(0)
        C.lib().csa2_sparse_attn_workspace_bytes(1, qb.shape[1], 16, 128, idx.shape[-1], ctypes.byref(nb))
        need.append(nb.value)
    ws = torch.zeros(max(need), dtype=torch.uint8, device="cuda")
    scale = float(np.float32(1 / math.sqrt(128)))
    for i, ((r, n, K, _), s) in enumerate(zip(cases, scores)):
        idx_t = host(C.topk(dev_f32(s), K, ws=ws))
        for row in range(r):
            ri, _ = o_topk(s[row], K)
            assert np.array_equal(idx_t[row], ri), (i, row)
        qb, idx = attn_cases[i % len(attn_cases)]
        out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda(), softmax_scale=scale, ws=ws))
        for qi in (0, qb.shape[1] - 1):
            err = max_rel_err_rows(out[0, qi], o_attn(qb[0, qi], okv, idx[0, qi], scale))
            assert err <= ATTN_TOL, (i, qi, err)
    ctrl_bytes = (64 + 256 * 8256 + 256) * 4                               # the fixed control region
    assert int(ws[:ctrl_bytes].view(torch.int32).abs().sum().item()) == 0


# --------------------------------------------------------------- attention

def _kv_case(N, seed):
    rng = np.random.default_rng(seed)
    kb = synth.to_bf16_bits((rng.standard_normal((N, 128)) * rng.choice([1, 20], (1, 128), p=[.99, .01])).astype(np.float32))
    vb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    cache = C.KVCache(1, N)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    kc, ks = OQ.quant_fp4(kb)
    vc, vs = OQ.quant_fp4(vb)
    return cache, dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs)


@pytest.mark.parametrize("H,K,Q", [(8, 128, 2), (16, 2048, 1), (16, 1, 3), (4, 300, 2)])
def test_sparse_attn_matches_oracle(H, K, Q):
    N = 6000
    cache, okv = _kv_case(N, H * 7 + K)
    rng = np.random.default_rng(K)
    qb = synth.to_bf16_bits(rng.standard_normal((1, Q, H, 128)).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    if K > 4:
        idx[0, 0, -3:] = -1                                   # padding
        idx[0, -1, 1] = N + 5                                 # out of range = padding
    scale = float(np.float32(1 / math.sqrt(128)))
    out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda(), softmax_scale=scale))
    for i in range(Q):
        sel = np.where(idx[0, i] >= N, -1, idx[0, i])
        ref = o_attn(qb[0, i], okv, sel, scale)
        err = max_rel_err_rows(out[0, i], ref)
        assert err <= ATTN_TOL, (i, err)


def test_sparse_attn_all_padding_gives_zeros():
    cache, _ = _kv_case(100, 1)
    qb = synth.to_bf16_bits(np.ones((1, 1, 8, 128), dtype=np.float32))
    idx = torch.full((1, 1, 64), -1, dtype=torch.int32, device="cuda")
    out = C.sparse_attn_fp4(dev_bf16(qb), cache, idx)
    assert float(out.abs().max().item()) == 0.0


def test_sparse_attn_query_magnitudes_outside_f16():
    """Heads whose bf16 queries lie far outside f16's range - above 65504 (up to bf16's largest finite
    values) and below f16's smallest normal 2^-14 - and heads mixing both magnitudes, against the oracle,
    with the library's default softmax scale (softmax_scale=None selects 1/sqrt(d) in the C call)."""
    N, H, K, Q = 3000, 8, 256, 3
    cache, okv = _kv_case(N, 5)
    rng = np.random.default_rng(17)
    x = rng.standard_normal((1, Q, H, 128)).astype(np.float32)
    mult = np.array([1e6, 2.0 ** -20, 3e4, 2.0 ** -40, 1e30, 1.0, 2.0 ** -126, 1e37], dtype=np.float64)
    xf = (x * mult[None, None, :, None]).astype(np.float32)
    xf[0, :, 5, ::9] *= np.float32(2.0 ** -30)              # one head: ~1 and ~2^-30 elements together
    xf[0, :, 2, ::7] *= np.float32(1e3)                     # one head: 3e4 and 3e7 together
    qb = synth.to_bf16_bits(xf)
    assert np.isfinite(F.bf16_decode(qb)).all()
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda()))
    scale = float(np.float32(1 / math.sqrt(128)))
    assert np.isfinite(out).all()
    for i in range(Q):
        ref = o_attn(qb[0, i], okv, idx[0, i], scale)
        err = max_rel_err_rows(out[0, i], ref)
        assert err <= ATTN_TOL, (i, err)
