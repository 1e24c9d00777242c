"""GPU parity of the MXFP4 variant (E2M1 elements, one E8M0 scale per 32 channels) against the oracle:
quantize and dequantize bit for bit (every finite bf16 value, every reachable scale, every code and
scale byte), sparse attention over an MXFP4 cache within ATTN_TOL, and the layer plan end to end."""

import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import formats as F
from oracle import mxfp4 as OM
from oracle import plan as OP
from oracle import scores as OS
from oracle.attention import sparse_attn as o_attn
from tests.parity import ATTN_TOL, compare_topk, dev_bf16, dev_key, dev_u8, host, max_rel_err_rows

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def _finite_bf16_rows(C_):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    b = bits[(bits & 0x7F80) != 0x7F80]
    b = b[np.random.default_rng(1).permutation(b.size)]
    n = b.size // C_ * C_
    return b[:n].reshape(-1, C_)


@pytest.mark.parametrize("C_", [32, 128, 512])
def test_quant_mxfp4_bit_exact_all_bf16_values(C_):
    x = _finite_bf16_rows(C_)
    codes, scales = C.kv_quant_mxfp4(dev_bf16(x))
    rc, rs = OM.quant_mxfp4(x)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)


def test_quant_mxfp4_every_scale_with_every_value_below_its_block_max():
    """For every bf16 exponent field e (so every E8M0 byte the quantizer can produce), blocks whose
    largest magnitude is 2^(e-127) * 1.9921875 (the block's scale byte is max(e - 2, 0)) hold, in their
    other 31 slots, every finite bf16 of smaller magnitude with both signs."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    finite = (bits & 0x7F80) != 0x7F80
    blocks = []
    for e in range(0, 255):
        top = np.uint16((e << 7) | 0x7F)                    # largest bf16 with exponent field e
        vals = bits[finite & ((bits & 0x7FFF) <= top)]
        vals = vals[np.random.default_rng(e).permutation(vals.size)][: 31 * 64]   # a spread of 64 blocks
        pad = (-vals.size) % 31
        vals = np.concatenate([vals, np.zeros(pad, dtype=np.uint16)]).reshape(-1, 31)
        blocks.append(np.concatenate([np.full((vals.shape[0], 1), top, dtype=np.uint16), vals], axis=1))
    g = np.concatenate(blocks)
    rows = (g.shape[0] + 3) // 4
    g = np.concatenate([g, np.zeros((rows * 4 - g.shape[0], 32), dtype=np.uint16)]).reshape(rows, 128)
    codes, scales = C.kv_quant_mxfp4(dev_bf16(g))
    rc, rs = OM.quant_mxfp4(g)
    assert np.array_equal(host(scales), rs)
    assert np.array_equal(host(codes), rc)
    assert len(set(rs.ravel().tolist())) >= 250              # nearly every E8M0 byte occurs


def test_dequant_mxfp4_every_code_and_scale_byte():
    rng = np.random.default_rng(3)
    T = 4096
    codes = rng.integers(0, 256, (T, 64), dtype=np.uint8)
    scales = np.tile(np.arange(256, dtype=np.uint8), T * 4 // 256).reshape(T, 4)
    y = C.kv_dequant_mxfp4(dev_u8(codes), dev_u8(scales), 128)
    got = F.bf16_decode(host(y.view(torch.int16)).view(np.uint16))
    ref = OM.dequant_mxfp4(codes, scales, 128)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    big = np.abs(ref) > 3.3895313892515355e38              # beyond bf16: the hardware gives inf
    assert np.all(np.isinf(got[big & ~nan]))
    ok = ~nan & ~big
    assert np.array_equal(got[ok], ref[ok]) and np.array_equal(np.signbit(got[ok]), np.signbit(ref[ok]))


def test_quant_mxfp4_log_uniform_rows_round_trip():
    cfg = synth.small("quant_1m_x512", row_block=2048)
    x = np.concatenate([synth.quant_rows(cfg, 0), synth.quant_rows(cfg, 9)])[:3001]
    codes, scales = C.kv_quant_mxfp4(dev_bf16(x))
    rc, rs = OM.quant_mxfp4(x)
    assert np.array_equal(host(scales), rs) and np.array_equal(host(codes), rc)
    y = C.kv_dequant_mxfp4(codes, scales, 512)
    got = F.bf16_decode(host(y.view(torch.int16)).view(np.uint16))
    assert np.array_equal(got, OM.dequant_mxfp4(rc, rs, 512))


def _mx_cache(N, seed, outliers=True):
    rng = np.random.default_rng(seed)
    kx = rng.standard_normal((N, 128))
    if outliers:
        kx = kx * rng.choice([1, 20], (1, 128), p=[.99, .01])
    kb = synth.to_bf16_bits(kx.astype(np.float32))
    vb = synth.to_bf16_bits((rng.standard_normal((N, 128)) * np.exp(rng.uniform(-3, 3, (N, 1)))).astype(np.float32))
    cache = C.KVCache(1, N, kv_format="mxfp4")
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    kc, ks = OM.quant_mxfp4(kb)
    vc, vs = OM.quant_mxfp4(vb)
    assert np.array_equal(host(cache.k_codes), kc) and np.array_equal(host(cache.v_scales), vs)
    return cache, dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, format="mxfp4"), rng


@pytest.mark.parametrize("H,K,Q", [(8, 128, 2), (16, 2048, 1), (16, 1, 3), (4, 300, 2), (16, 2048, 40)])
def test_sparse_attn_mxfp4_matches_oracle(H, K, Q):
    N = 6000
    cache, okv, rng = _mx_cache(N, H * 7 + K)
    qb = synth.to_bf16_bits(rng.standard_normal((1, Q, H, 128)).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    if K > 4:
        idx[0, 0, -3:] = -1
        idx[0, -1, 1] = N + 5
    out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda()))
    for i in range(Q):
        ref = o_attn(qb[0, i], okv, np.where(idx[0, i] >= N, -1, idx[0, i]), SCALE)
        err = max_rel_err_rows(out[0, i], ref)
        assert err <= ATTN_TOL, (i, err)


def test_sparse_attn_mxfp4_query_magnitudes():
    N, H, K, Q = 3000, 8, 256, 2
    cache, okv, rng = _mx_cache(N, 5)
    x = rng.standard_normal((1, Q, H, 128)).astype(np.float32)
    mult = np.array([1e6, 2.0 ** -20, 3e4, 2.0 ** -40, 1e30, 1.0, 2.0 ** -126, 1e37])
    qb = synth.to_bf16_bits((x * mult[None, None, :, None]).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda()))
    assert np.isfinite(out).all()
    for i in range(Q):
        assert max_rel_err_rows(out[0, i], o_attn(qb[0, i], okv, idx[0, i], SCALE)) <= ATTN_TOL, i


@pytest.mark.parametrize("B,N,K,P", [(3, 20000, 64, 512), (2, 70001, 2048, 8192)])
def test_plan_stack_over_mxfp4_cache(B, N, K, P):
    """Full -> Reindex -> Reuse -> Reuse over an MXFP4 main KV cache: positions exact, attention within
    ATTN_TOL of the oracle on the GPU's own positions, Reuse bit-identical to attention on the inherited
    positions."""
    cfg = synth.small("stack_b32_n262144", B=B, N=N, K=K, P=P)
    modes = list(cfg["modes"])
    kidx = np.stack([synth.k_idx(cfg, b) for b in range(B)])
    cache = C.KVCache(B, N, k_idx=dev_key(kidx, cfg["k_idx_dtype"]), kv_format="mxfp4")
    ocache = []
    for b in range(B):
        kb, vb = synth.kv_bf16(cfg, b)
        cache.fill(dev_bf16(kb), dev_bf16(vb), row0=b * N)
        ocache.append(dict(k_bf16=kb, v_bf16=vb, k_idx=kidx[b], k_idx_dtype=cfg["k_idx_dtype"], format="mxfp4"))
    layers = []
    for li in range(len(modes)):
        q = np.stack([synth.q_bf16(cfg, li, b)[0] for b in range(B)])
        qi = np.stack([synth.q_idx(cfg, li, b)[0] for b in range(B)])
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, 16, 128, dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, K, dtype=torch.int32, device="cuda")))
    layers[0]["pool_out"] = torch.empty(B, P, dtype=torch.int32, device="cuda")
    plan = C.Plan(modes, K=K, P=P, kv_format="mxfp4")
    plan.run_decode(cache, layers)
    for b in range(B):
        ol = [dict(q=synth.q_bf16(cfg, li, b)[0], q_idx=synth.q_idx(cfg, li, b)[0], q_idx_dtype=cfg["q_idx_dtype"])
              for li in range(len(modes))]
        res = OP.run_decode(modes, ocache[b], ol, K, P, softmax_scale=SCALE)
        prev = None
        for li, mode in enumerate(modes):
            g_idx = prev if mode == "reuse" else host(layers[li]["idx_out"][b])
            if mode != "reuse":
                s = OS.index_scores(ol[li]["q_idx"], cfg["q_idx_dtype"], kidx[b], cfg["k_idx_dtype"])
                assert compare_topk(g_idx, res[li]["idx"], lambda p: s[p], K) == "exact", (b, li)
            prev = g_idx
            err = max_rel_err_rows(host(layers[li]["out"][b]), res[li]["out"])
            assert err <= ATTN_TOL, (b, li, err)
    direct = host(C.sparse_attn_fp4(layers[3]["q"][:, None], cache, layers[1]["idx_out"][:, None]))[:, 0]
    assert np.array_equal(direct, host(layers[3]["out"]))
