"""GPU parity of longer plans (several Full layers, each with its own cache and pool) and of prefill
through the whole plan (per-query pools, Reindex and Reuse layers) against the oracle."""

import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import plan as OP
from oracle import quant as OQ
from oracle import scores as OS
from tests.parity import ATTN_TOL, compare_topk, dev_bf16, dev_key, host, max_rel_err_rows

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def _group_caches(cfg, ngroups):
    """One device KVCache (with indexer keys) per group, and the oracle's view of each sequence of each."""
    B, N = cfg["B"], cfg["N"]
    caches, ocaches = [], []
    for gi in range(ngroups):
        cg = dict(cfg, seed=cfg["seed"] + gi)
        kidx = np.stack([synth.k_idx(cg, b) for b in range(B)])
        cache = C.KVCache(B, N, k_idx=dev_key(kidx, cfg["k_idx_dtype"]))
        oc = []
        for b in range(B):
            kb, vb = synth.kv_bf16(cg, b)
            cache.fill(dev_bf16(kb), dev_bf16(vb), row0=b * N)
            kc, ks = OQ.quant_fp4(kb)
            vc, vs = OQ.quant_fp4(vb)
            oc.append(dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, k_idx=kidx[b],
                           k_idx_dtype=cfg["k_idx_dtype"]))
        caches.append(cache)
        ocaches.append(oc)
    return caches, ocaches


def test_decode_plan_with_two_full_layers():
    modes = ["full", "reindex", "reuse", "full", "reindex", "reuse"]
    B, N, K, P = 3, 20000, 128, 512
    cfg = synth.small("stack_b32_n262144", B=B, N=N, K=K, P=P, modes=tuple(modes))
    caches, ocaches = _group_caches(cfg, 2)
    layers = []
    for li in range(len(modes)):
        q = np.stack([synth.q_bf16(cfg, li, b)[0] for b in range(B)])
        qi = np.stack([synth.q_idx(cfg, li, b)[0] for b in range(B)])
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, 16, 128, dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, K, dtype=torch.int32, device="cuda")))
    plan = C.Plan(modes, K=K, P=P)
    plan.run_decode(caches, layers)
    grp = OP.groups(modes)
    for b in range(B):
        ol = [dict(q=synth.q_bf16(cfg, li, b)[0], q_idx=synth.q_idx(cfg, li, b)[0], q_idx_dtype=cfg["q_idx_dtype"])
              for li in range(len(modes))]
        res = OP.run_decode(modes, [ocaches[0][b], ocaches[1][b]], ol, K, P, softmax_scale=SCALE)
        prev = None
        for li, mode in enumerate(modes):
            g_idx = prev if mode == "reuse" else host(layers[li]["idx_out"][b])
            if mode == "full":
                s = OS.index_scores(ol[li]["q_idx"], cfg["q_idx_dtype"], ocaches[grp[li]][b]["k_idx"], cfg["k_idx_dtype"])
                assert compare_topk(g_idx, res[li]["idx"], lambda p: s[p], K) == "exact", (b, li)
            elif mode == "reindex":
                assert np.array_equal(g_idx, res[li]["idx"]), (b, li)
            prev = g_idx
            assert max_rel_err_rows(host(layers[li]["out"][b]), res[li]["out"]) <= ATTN_TOL, (b, li)


def _prefill_case(modes, B, N, K, P, q_pos, ngroups=1):
    cfg = synth.small("stack_b4_n1m", B=B, N=N, K=K, P=P, modes=tuple(modes))
    caches, ocaches = _group_caches(cfg, ngroups)
    Q = q_pos.shape[1]
    layers, olayers = [], []
    for li in range(len(modes)):
        q = np.stack([synth.q_bf16(dict(cfg, H=16), 100 + li, b, Q=Q) for b in range(B)])
        qi = np.stack([synth.q_idx(cfg, 100 + li, b, Q=Q) for b in range(B)])
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, Q, 16, 128, dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, Q, K, dtype=torch.int32, device="cuda")))
        olayers.append((q, qi))
    plan = C.Plan(modes, K=K, P=P)
    plan.run_prefill(caches if ngroups > 1 else caches[0], layers, torch.from_numpy(q_pos).cuda())
    return cfg, caches, ocaches, layers, olayers


def _check_prefill(modes, cfg, ocaches, layers, olayers, q_pos, queries):
    K, P = cfg["K"], cfg["P"]
    grp = OP.groups(modes)
    stats = {"exact": 0, "excused": 0}
    for b in range(q_pos.shape[0]):
        ol = [dict(q=olayers[li][0][b], q_idx=olayers[li][1][b], q_idx_dtype=cfg["q_idx_dtype"])
              for li in range(len(modes))]
        oc = [ocaches[gi][b] for gi in range(len(ocaches))]
        res = OP.run_prefill(modes, oc, ol, q_pos[b], K, P, softmax_scale=SCALE, queries=queries)
        for qi_, i in enumerate(queries):
            prev = None
            for li, mode in enumerate(modes):
                g_idx = prev if mode == "reuse" else host(layers[li]["idx_out"][b, i])
                r_idx = res[li][0][qi_]
                if mode == "full":
                    s = OS.index_scores(ol[li]["q_idx"][i], cfg["q_idx_dtype"], oc[grp[li]]["k_idx"], cfg["k_idx_dtype"],
                                        q_pos=int(q_pos[b, i]))
                    stats[compare_topk(g_idx, r_idx, lambda p: s[p], K)] += 1
                else:
                    assert np.array_equal(g_idx, r_idx), (b, i, li)
                prev = g_idx
                err = max_rel_err_rows(host(layers[li]["out"][b, i]), res[li][1][qi_])
                assert err <= ATTN_TOL, (b, i, li, err)
    return stats


def test_prefill_plan_exact_path():
    modes = ["full", "reindex", "reuse", "reuse"]
    B, N, K, P = 2, 5000, 32, 256
    q_pos = np.array([[0, 5, 31, 32, 100, 255, 256, 1000, 2500, 4000, 4990, 4999]] * B, dtype=np.int64)
    cfg, caches, ocaches, layers, olayers = _prefill_case(modes, B, N, K, P, q_pos)
    stats = _check_prefill(modes, cfg, ocaches, layers, olayers, q_pos, list(range(q_pos.shape[1])))
    assert stats["exact"] == B * q_pos.shape[1], stats


@pytest.mark.timeout(600)
def test_prefill_plan_matrix_core_path():
    """N = 70,001 with bf16 queries and E4M3 keys: the Full layer's top-P pool and top-K come from the
    matrix-core candidate path (two targets of one exact selection); per-query pools feed the Reindex."""
    modes = ["full", "reindex", "reuse", "reuse"]
    B, N, K, P = 2, 70001, 256, 2048
    rng = np.random.default_rng(4)
    q_pos = np.stack([np.sort(np.concatenate([[0, 17, 255, 256, 2047, 2048, 30000, N - 1],
                                              rng.integers(0, N, 56)])) for _ in range(B)]).astype(np.int64)
    cfg, caches, ocaches, layers, olayers = _prefill_case(modes, B, N, K, P, q_pos)
    stats = _check_prefill(modes, cfg, ocaches, layers, olayers, q_pos, list(range(0, 64, 3)) + [63])
    assert stats["excused"] <= 1, stats


def test_prefill_plan_two_groups():
    modes = ["full", "reuse", "full", "reindex"]
    B, N, K, P = 2, 3000, 16, 64
    q_pos = np.array([[2, 15, 63, 64, 700, 2999]] * B, dtype=np.int64)
    cfg, caches, ocaches, layers, olayers = _prefill_case(modes, B, N, K, P, q_pos, ngroups=2)
    stats = _check_prefill(modes, cfg, ocaches, layers, olayers, q_pos, list(range(q_pos.shape[1])))
    assert stats["exact"] == 2 * B * q_pos.shape[1], stats


@pytest.mark.timeout(900)
def test_prefill_plan_large_pool():
    """P = 8192 at N = 262,144 with 256 queries: the Full layer samples at 1.5 times the pool's share, and
    the exact candidate select (one workgroup per query at this many queries) keeps keys and positions in
    LDS for the candidates a query nominates, fewer than its lists' slots. Pools, Reindex and Reuse layers
    and attention match the oracle."""
    modes = ["full", "reindex", "reuse", "reuse"]
    B, N, K, P, Q = 1, 262144, 2048, 8192, 256
    rng = np.random.default_rng(31)
    q_pos = np.sort(np.concatenate([[0, 100, 8191, 8192, 20000, 65535, 65536, 131071, N - 4097, N - 2, N - 1],
                                    rng.integers(0, N, Q - 11)]))[None].astype(np.int64)
    cfg, caches, ocaches, layers, olayers = _prefill_case(modes, B, N, K, P, q_pos)
    check = [0, 2, 3, 5, 60, 130, 200, 250, 254, 255]
    stats = _check_prefill(modes, cfg, ocaches, layers, olayers, q_pos, check)
    assert stats["exact"] + stats["excused"] == len(check) and stats["excused"] <= 1, stats


@pytest.mark.timeout(900)
def test_prefill_plan_more_candidates_than_the_select_holds():
    """20,000 positions share the indexer key that scores highest for the Full layer's query, so every one
    of 256 queries nominates them all: more candidates than the exact candidate select holds (one
    workgroup per query, its LDS sized below the lists' slots; the lists do not overflow). Those queries
    take the exact repair (64 by the multi-workgroup select, the rest one workgroup each); the pool is the
    lowest 8192 tied positions and the top-K the lowest 2048, and every layer matches the oracle."""
    modes = ["full", "reindex", "reuse", "reuse"]
    B, N, K, P, Q = 1, 262144, 2048, 8192, 256
    cfg = synth.small("stack_b4_n1m", B=B, N=N, K=K, P=P, modes=tuple(modes))
    rng = np.random.default_rng(21)
    tied = np.sort(rng.choice(N, 20000, replace=False))
    q0 = synth.q_idx(cfg, 100, 0, Q=1)[0]                       # the Full layer's query, shared by the chunk
    q0f = (np.ascontiguousarray(q0).astype(np.uint32) << 16).view(np.float32)
    key = synth.to_e4m3_bytes(np.where(q0f >= 0, 4.0, -4.0).astype(np.float32))
    kidx = synth.k_idx(cfg, 0)
    kidx[tied] = key
    cache = C.KVCache(B, N, k_idx=dev_key(kidx[None], cfg["k_idx_dtype"]))
    kb, vb = synth.kv_bf16(cfg, 0)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    kc, ks = OQ.quant_fp4(kb)
    vc, vs = OQ.quant_fp4(vb)
    oc = dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, k_idx=kidx, k_idx_dtype=cfg["k_idx_dtype"])
    q_pos = (N - 1 - 20 * np.arange(Q))[None].astype(np.int64)
    layers, olayers = [], []
    for li in range(len(modes)):
        q = synth.q_bf16(dict(cfg, H=16), 100 + li, 0, Q=Q)[None]
        qi = synth.q_idx(cfg, 100 + li, 0, Q=Q)[None]
        if li == 0:
            qi = np.repeat(q0[None, None], Q, axis=1)
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, Q, 16, 128, dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, Q, K, dtype=torch.int32, device="cuda")))
        olayers.append((q, qi))
    plan = C.Plan(modes, K=K, P=P)
    plan.run_prefill(cache, layers, torch.from_numpy(q_pos).cuda())
    full_idx = host(layers[0]["idx_out"][0])
    for i in range(Q):
        causal_tied = tied[tied <= q_pos[0, i]]
        assert np.array_equal(full_idx[i], causal_tied[:K]), i
    check = [0, 1, 63, 64, 65, 200, 255]
    stats = _check_prefill(modes, cfg, [[oc]], layers, olayers, q_pos, check)
    assert stats["exact"] == len(check), stats
