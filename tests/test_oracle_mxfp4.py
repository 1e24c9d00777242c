"""Pins of the oracle's MXFP4 quantizer (E2M1 elements, one E8M0 scale per 32 channels).

E8M0 decode against torch's float8_e8m0fnu (a library routine) for all 256 bytes; three blocks worked by
hand (tests/golden/mxfp4_group_example.txt); the properties the OCP MX scale rule fixes (the block maximum
lands in [4, 8) * X, so its code is 4 or 6; every element within X of its value, 2X when saturated);
idempotence; byte accounting (C/2 + C/32)."""

import numpy as np
import torch

from oracle import formats as F
from oracle import mxfp4 as M
from oracle.quant import unpack_codes


def _bf16_bits(vals):
    return torch.tensor(vals, dtype=torch.float32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def test_e8m0_decode_all_bytes_equals_torch():
    b = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(b).view(torch.float8_e8m0fnu).float().double().numpy()
    got = M.e8m0_decode(b)
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])
    assert got[127] == 1.0 and got[0] == 2.0 ** -127 and got[254] == 2.0 ** 127


def test_worked_blocks(golden_dir):
    fields = {}
    for line in open(f"{golden_dir}/mxfp4_group_example.txt"):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        fields[k.strip()] = v.split()
    for blk in ("a", "b", "c"):
        x = np.array([float(t) for t in fields[f"{blk}_x"]]) * float(fields[f"{blk}_mult"][0])
        bits = _bf16_bits(x.tolist()).reshape(1, 32)
        assert np.array_equal(F.bf16_decode(bits)[0], x) and np.array_equal(np.signbit(F.bf16_decode(bits)[0]), np.signbit(x))
        packed, scale = M.quant_mxfp4(bits)
        assert scale[0].tolist() == [int(fields[f"{blk}_scale"][0], 16)], blk
        assert unpack_codes(packed, 32)[0].tolist() == [int(t, 16) for t in fields[f"{blk}_codes"]], blk
        assert packed[0].tolist() == [int(t, 16) for t in fields[f"{blk}_packed"]], blk


def _random_rows(seed, T=512, C=256):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, C)) * np.power(10.0, rng.uniform(-30, 30, (T, 1)))
    x[rng.random((T, C)) < 0.05] = 0.0
    return _bf16_bits(x.astype(np.float32).tolist())


def test_scale_puts_block_max_in_the_top_binades():
    bits = _random_rows(1)
    packed, scale = M.quant_mxfp4(bits)
    x = F.bf16_decode(bits).reshape(bits.shape[0], -1, 32)
    amax = np.abs(x).max(axis=-1)
    X = M.e8m0_decode(scale)
    live = (amax > 0) & (scale > 0)
    r = amax[live] / X[live]
    assert np.all((r >= 4.0) & (r < 8.0))
    mag = unpack_codes(packed, bits.shape[1]).reshape(bits.shape[0], -1, 32) & 7
    assert np.all(np.isin(mag.max(axis=-1)[live], (6, 7)))          # E2M1 4 or 6
    assert np.all(scale[amax == 0] == 0)


def test_error_bound_and_idempotence():
    bits = _random_rows(2)
    C = bits.shape[1]
    packed, scale = M.quant_mxfp4(bits)
    v = M.dequant_mxfp4(packed, scale, C).reshape(bits.shape[0], -1, 32)
    x = F.bf16_decode(bits).reshape(bits.shape[0], -1, 32)
    X = M.e8m0_decode(scale)[..., None]
    sat = np.abs(x) / X > 6.0
    err = np.abs(x - v)
    assert np.all(err[~sat] <= X.repeat(32, -1)[~sat])
    assert np.all(err[sat] <= 2 * X.repeat(32, -1)[sat])
    assert np.array_equal(np.signbit(v), np.signbit(x) | (v == 0) & np.signbit(x))
    # dequantized values are exact in bf16, and quantizing them again gives the same codes and scales
    vb = _bf16_bits(v.reshape(bits.shape[0], C).astype(np.float32).tolist())
    assert np.array_equal(F.bf16_decode(vb), v.reshape(bits.shape[0], C))
    p2, s2 = M.quant_mxfp4(vb)
    assert np.array_equal(s2, scale) and np.array_equal(p2, packed)


def test_byte_accounting():
    assert M.bytes_per_token(128) == 68              # 4.25 bits per channel
    assert 2 * M.bytes_per_token(128) == 136         # K and V of one token
    p, s = M.quant_mxfp4(np.zeros((3, 512), dtype=np.uint16))
    assert p.shape == (3, 256) and s.shape == (3, 16)


def test_attention_reads_mxfp4_planes_and_rows_alike():
    """The oracle's attention over an MXFP4 cache: stored planes and bf16 rows give the same output, and
    a one-position list returns that row of the MXFP4-dequantized V."""
    import synth
    from oracle import attention as A
    rng = np.random.default_rng(4)
    N, H, d = 200, 4, 128
    kb = synth.to_bf16_bits(rng.standard_normal((N, d)).astype(np.float32))
    vb = synth.to_bf16_bits((rng.standard_normal((N, d)) * 5).astype(np.float32))
    kc, ks = M.quant_mxfp4(kb)
    vc, vs = M.quant_mxfp4(vb)
    planes = dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, format="mxfp4")
    rows = dict(k_bf16=kb, v_bf16=vb, format="mxfp4")
    qb = synth.to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))
    idx = np.concatenate([rng.permutation(N)[:50], [-1, -1]])
    assert np.array_equal(A.sparse_attn(qb, planes, idx), A.sparse_attn(qb, rows, idx))
    out = A.sparse_attn(qb, planes, np.array([13, -1]))
    assert np.array_equal(out, np.broadcast_to(M.dequant_mxfp4(vc, vs, d)[13], (H, d)))
