"""GPU parity of the sliding-window branch beside CSA2 (csa2_sparse_attn_swa and the plan's swa_window):
window rows and selected FP4 positions in one softmax, against the oracle within ATTN_TOL."""

import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import mxfp4 as OM
from oracle import plan as OP
from oracle import quant as OQ
from oracle import scores as OS
from oracle.attention import sparse_attn_swa as o_swa
from tests.parity import ATTN_TOL, compare_topk, dev_bf16, dev_key, host, max_rel_err_rows

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))
QUANT = {"fp4_e4m3": OQ.quant_fp4, "mxfp4": OM.quant_mxfp4}


def _cache(N, fmt, rng):
    kb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    vb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    cache = C.KVCache(1, N, kv_format=fmt)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    return cache, dict(k_bf16=kb, v_bf16=vb, format=fmt)


@pytest.mark.parametrize("fmt", ["fp4_e4m3", "mxfp4"])
@pytest.mark.parametrize("H,K,Q,W", [(16, 2048, 2, 128), (8, 128, 5, 100), (16, 1, 3, 300), (4, 256, 40, 32)])
def test_sparse_attn_swa_matches_oracle(fmt, H, K, Q, W):
    rng = np.random.default_rng(K + W + Q)
    N = 5000
    cache, okv = _cache(N, fmt, rng)
    qb = synth.to_bf16_bits(rng.standard_normal((1, Q, H, 128)).astype(np.float32))
    idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
    if K > 4:
        idx[0, 0, -3:] = -1
    wk = synth.to_bf16_bits((rng.standard_normal((1, Q, W, 128)) * 1.5).astype(np.float32))
    wv = synth.to_bf16_bits(rng.standard_normal((1, Q, W, 128)).astype(np.float32))
    wlen = rng.integers(0, W + 1, Q).astype(np.int32)
    wlen[0] = W
    if Q > 2:
        wlen[1] = 0                                          # a row with an empty window
    out = host(C.sparse_attn_swa(dev_bf16(qb), cache, torch.from_numpy(idx).cuda(), dev_bf16(wk), dev_bf16(wv),
                                 win_len=torch.from_numpy(wlen).cuda()))
    for i in range(Q):
        ref = o_swa(qb[0, i], okv, idx[0, i], wk[0, i, :wlen[i]], wv[0, i, :wlen[i]], SCALE)
        err = max_rel_err_rows(out[0, i], ref)
        assert err <= ATTN_TOL, (i, int(wlen[i]), err)


def test_sparse_attn_swa_window_only_and_no_window():
    """All positions padding: dense attention over the window alone; W = 0 is bit-identical to
    csa2_sparse_attn_fp4."""
    rng = np.random.default_rng(3)
    cache, okv = _cache(2000, "fp4_e4m3", rng)
    qb = synth.to_bf16_bits(rng.standard_normal((1, 2, 16, 128)).astype(np.float32))
    idx = np.full((1, 2, 64), -1, dtype=np.int32)
    wk = synth.to_bf16_bits(rng.standard_normal((1, 2, 77, 128)).astype(np.float32))
    wv = synth.to_bf16_bits(rng.standard_normal((1, 2, 77, 128)).astype(np.float32))
    out = host(C.sparse_attn_swa(dev_bf16(qb), cache, torch.from_numpy(idx).cuda(), dev_bf16(wk), dev_bf16(wv)))
    for i in range(2):
        assert max_rel_err_rows(out[0, i], o_swa(qb[0, i], okv, idx[0, i], wk[0, i], wv[0, i], SCALE)) <= ATTN_TOL
    idx2 = torch.from_numpy(np.sort(rng.choice(2000, (1, 2, 300)), axis=-1).astype(np.int32)).cuda()
    empty = torch.empty(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    a = host(C.sparse_attn_swa(dev_bf16(qb), cache, idx2, empty, empty))
    b = host(C.sparse_attn_fp4(dev_bf16(qb), cache, idx2))
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))


@pytest.mark.parametrize("fmt", ["fp4_e4m3", "mxfp4"])
def test_plan_stack_with_sliding_window(fmt):
    """Full -> Reindex -> Reuse -> Reuse with a 128-row window per layer and sequence (two sequences with
    shorter windows): positions exact, every layer's output within ATTN_TOL of the oracle."""
    B, N, K, P, W = 3, 20000, 256, 1024, 128
    cfg = synth.small("stack_b32_n262144", B=B, N=N, K=K, P=P)
    modes = list(cfg["modes"])
    rng = np.random.default_rng(11)
    kidx = np.stack([synth.k_idx(cfg, b) for b in range(B)])
    cache = C.KVCache(B, N, k_idx=dev_key(kidx, cfg["k_idx_dtype"]), kv_format=fmt)
    ocache = []
    for b in range(B):
        kb, vb = synth.kv_bf16(cfg, b)
        cache.fill(dev_bf16(kb), dev_bf16(vb), row0=b * N)
        ocache.append(dict(k_bf16=kb, v_bf16=vb, k_idx=kidx[b], k_idx_dtype=cfg["k_idx_dtype"], format=fmt))
    wlen = np.array([W, 5, 77], dtype=np.int32)
    layers, wins = [], []
    for li in range(len(modes)):
        q = np.stack([synth.q_bf16(cfg, li, b)[0] for b in range(B)])
        qi = np.stack([synth.q_idx(cfg, li, b)[0] for b in range(B)])
        wk = synth.to_bf16_bits(rng.standard_normal((B, W, 128)).astype(np.float32))
        wv = synth.to_bf16_bits(rng.standard_normal((B, W, 128)).astype(np.float32))
        wins.append((wk, wv))
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, 16, 128, dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, K, dtype=torch.int32, device="cuda"),
                           win_k=dev_bf16(wk), win_v=dev_bf16(wv), win_len=torch.from_numpy(wlen).cuda()))
    plan = C.Plan(modes, K=K, P=P, kv_format=fmt, swa_window=W)
    plan.run_decode(cache, layers)
    for b in range(B):
        ol = [dict(q=synth.q_bf16(cfg, li, b)[0], q_idx=synth.q_idx(cfg, li, b)[0], q_idx_dtype=cfg["q_idx_dtype"],
                   win_k=wins[li][0][b, :wlen[b]], win_v=wins[li][1][b, :wlen[b]]) for li in range(len(modes))]
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
