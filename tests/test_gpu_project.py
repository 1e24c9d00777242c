"""GPU parity of the KV write path (csa2_kv_project: C = H W on the matrix cores, rounded to bf16 and
quantized to FP4 in one kernel) against the oracle, stage by stage: the bf16 C within the fp32
accumulation bound of the exact product, and the codes and scales bit for bit equal to the oracle's
quantizer applied to that C; then written straight into a KV cache and read back by attention."""

import math

import numpy as np
import pytest
import torch

import bench
import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import formats as F
from oracle import mxfp4 as OM
from oracle import project as PJ
from oracle import quant as OQ
from oracle.attention import sparse_attn as o_attn
from tests.parity import ATTN_TOL, dev_bf16, host, max_rel_err_rows

pytestmark = pytest.mark.gpu

QUANT = {"fp4_e4m3": OQ.quant_fp4, "mxfp4": OM.quant_mxfp4}


def _check_rows(h, wt, c_bits, codes, scales, fmt):
    """c_bits: the GPU's bf16 C rows; h, wt: the inputs of those rows (bit patterns)."""
    exact = PJ.project_exact(h, wt.T)
    bound = PJ.project_exact(h & np.uint16(0x7FFF), (wt & np.uint16(0x7FFF)).T)     # sum of |products|
    got = F.bf16_decode(c_bits)
    D = h.shape[1]
    # bf16 rounding (half a unit) plus the fp32 accumulation error (D - 1 roundings of partial sums)
    tol = np.abs(exact) * 2.0 ** -8 + bound * (D * 2.0 ** -24)
    assert np.all(np.abs(got - exact) <= tol)
    ref_bits = PJ.round_to_bf16(exact)
    frac_same = float((ref_bits == c_bits).mean())
    rc, rs = QUANT[fmt](c_bits)
    assert np.array_equal(codes, rc) and np.array_equal(scales, rs)
    return frac_same


@pytest.mark.parametrize("fmt", ["fp4_e4m3", "mxfp4"])
@pytest.mark.parametrize("T,D", [(1, 64), (63, 64), (64, 512), (65, 192), (300, 2048)])
def test_kv_project_matches_oracle(T, D, fmt):
    rng = np.random.default_rng(T * 7 + D)
    h = synth.to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32) * np.exp(rng.uniform(-2, 2, (T, 1))).astype(np.float32))
    wt = synth.to_bf16_bits((rng.standard_normal((256, D)) / math.sqrt(D)).astype(np.float32))
    c_out = torch.empty(T, 256, dtype=torch.bfloat16, device="cuda")
    codes, scales = C.kv_project(dev_bf16(h), dev_bf16(wt), fmt, c_out=c_out)
    c_bits = host(c_out.view(torch.int16)).view(np.uint16)
    same = _check_rows(h, wt, c_bits, host(codes), host(scales), fmt)
    assert same > 0.97, same                    # the fp32 sum rounds to the exact product's bf16 almost always


@pytest.mark.parametrize("fmt", ["fp4_e4m3", "mxfp4"])
def test_kv_project_into_cache_then_attention(fmt):
    """Project 700 tokens into positions 300..999 of a 1,200-position cache (the other positions quantized
    from bf16 rows), then attend over positions spanning both: outputs within ATTN_TOL of the oracle."""
    rng = np.random.default_rng(5)
    N, T, D, row0 = 1200, 700, 512, 300
    kb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    vb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    cache = C.KVCache(1, N, kv_format=fmt)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    h = synth.to_bf16_bits(rng.standard_normal((T, D)).astype(np.float32))
    wt = synth.to_bf16_bits((rng.standard_normal((256, D)) / math.sqrt(D)).astype(np.float32))
    c_out = torch.empty(T, 256, dtype=torch.bfloat16, device="cuda")
    C.kv_project(dev_bf16(h), dev_bf16(wt), fmt, codes=cache.codes[row0:row0 + T], scales=cache.scales[row0:row0 + T],
                 c_out=c_out)
    c_bits = host(c_out.view(torch.int16)).view(np.uint16)
    k_all, v_all = kb.copy(), vb.copy()
    k_all[row0:row0 + T], v_all[row0:row0 + T] = c_bits[:, :128], c_bits[:, 128:]
    okv = dict(k_bf16=k_all, v_bf16=v_all, format=fmt)
    rc, rs = QUANT[fmt](k_all)
    assert np.array_equal(host(cache.k_codes), rc) and np.array_equal(host(cache.k_scales), rs)
    H, K, Q = 16, 256, 3
    qb = synth.to_bf16_bits(rng.standard_normal((1, Q, H, 128)).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    out = host(C.sparse_attn_fp4(dev_bf16(qb), cache, torch.from_numpy(idx).cuda()))
    scale = float(np.float32(1 / math.sqrt(128)))
    for i in range(Q):
        assert max_rel_err_rows(out[0, i], o_attn(qb[0, i], okv, idx[0, i], scale)) <= ATTN_TOL


@pytest.mark.timeout(900)
@pytest.mark.parametrize("fmt", ["fp4_e4m3", "mxfp4"])
def test_kv_project_full_size_sampled(fmt):
    """The 16,384 x 4096 projection workload in the benchmark's launch configuration; sampled rows (the
    first and the last 64, 64 across the middle tile boundary, plus random picks; both channel halves of
    each) against the oracle."""
    cfg = dict(synth.WORKLOADS["kvproj_t16384_d4096"])
    dev = torch.device("cuda", 0)
    h_t, wt_t = bench.build_proj_input(cfg, dev)
    T, rb = cfg["T"], cfg["row_block"]
    c_out = torch.empty(T, 256, dtype=torch.bfloat16, device=dev)
    codes, scales = C.kv_project(h_t, wt_t, fmt, c_out=c_out)
    torch.cuda.synchronize()
    wt = synth.proj_weights_t(cfg)
    rows = np.concatenate([np.arange(0, 64), np.arange(8192 - 32, 8192 + 32), np.arange(T - 64, T),
                           np.random.default_rng(0).integers(0, T, 64)])
    blocks = {}
    for r in rows:
        blocks.setdefault(int(r) // rb, []).append(int(r))
    hs, idx = [], []
    for blk, rr in sorted(blocks.items()):
        hb = synth.proj_hidden(cfg, blk)
        hs.append(hb[np.array(rr) - blk * rb])
        idx.extend(rr)
    h = np.concatenate(hs)
    idx = np.array(idx)
    c_bits = host(c_out.view(torch.int16)).view(np.uint16)[idx]
    same = _check_rows(h, wt, c_bits, host(codes)[idx], host(scales)[idx], fmt)
    assert same > 0.97, same
