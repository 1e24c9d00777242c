"""Pins of the oracle's top-K, attention and layer plan.

top-K: checked against a rank-count brute force (a different algorithm: an
entry is selected iff fewer than K entries beat it). Attention: against
torch's scaled_dot_product_attention in fp64 (a library routine) with K >= N,
and closed forms (K = 1, equal logits). Plan: the mode invariants the pages
state (Reuse = attention on inherited positions; Reindex over a whole-context
pool = Full; Reindex and Full positions lie inside the pool).
"""

import numpy as np
import pytest
import torch

from oracle import attention as A
from oracle import formats as F
from oracle import plan as PL
from oracle import quant as Q
from oracle.topk import topk
import synth


def _rank_count_topk(s, K, pos):
    s = s.astype(np.float64)
    ok = ~np.isnan(s) & (s > -np.inf)
    chosen = []
    for i in range(len(s)):
        if not ok[i]:
            continue
        beats = sum(1 for j in range(len(s)) if ok[j] and (s[j] > s[i] or (s[j] == s[i] and pos[j] < pos[i])))
        if beats < K:
            chosen.append(pos[i])
    chosen.sort()
    return chosen + [-1] * (K - len(chosen))


@pytest.mark.parametrize("n,K,seed", [(1, 1, 0), (17, 5, 1), (64, 64, 2), (50, 80, 3), (200, 31, 4)])
def test_topk_vs_rank_count(n, K, seed):
    rng = np.random.default_rng(seed)
    s = rng.integers(-4, 5, n).astype(np.float32)          # many exact ties
    s[rng.random(n) < 0.1] = -np.inf
    s[rng.random(n) < 0.05] = np.nan
    s[rng.random(n) < 0.1] = -0.0
    pos = rng.permutation(10 * n)[:n]
    idx, sel = topk(s, K, pos)
    assert idx.tolist() == _rank_count_topk(s, K, pos)
    for p, v in zip(idx, sel):
        if p >= 0:
            assert v == s[list(pos).index(p)]
        else:
            assert np.isnan(v)


def test_topk_all_equal_and_k_ge_n():
    idx, _ = topk(np.full(100, 2.5, dtype=np.float32), 10)
    assert idx.tolist() == list(range(10))
    idx, _ = topk(np.arange(6, dtype=np.float32), 9)
    assert idx.tolist() == [0, 1, 2, 3, 4, 5, -1, -1, -1]


def test_topk_zero_signs_tie():
    idx, _ = topk(np.array([0.0, -0.0, 0.0, -1.0], dtype=np.float32), 2)
    assert idx.tolist() == [0, 1]
    idx, _ = topk(np.array([-0.0, 0.0], dtype=np.float32), 1)
    assert idx.tolist() == [0]


def _kv(rng, N, d=128):
    x = rng.standard_normal((N, d)).astype(np.float32)
    v = rng.standard_normal((N, d)).astype(np.float32)
    kc, ks = Q.quant_fp4(synth.to_bf16_bits(x))
    vc, vs = Q.quant_fp4(synth.to_bf16_bits(v))
    return dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs)


def test_attention_dense_equals_library_sdpa():
    rng = np.random.default_rng(0)
    N, H, d = 40, 8, 128
    kv = _kv(rng, N, d)
    qb = synth.to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))
    out = A.sparse_attn(qb, kv, np.arange(N))
    Kh = torch.from_numpy(Q.dequant_fp4(kv["k_codes"], kv["k_scales"], d))
    Vh = torch.from_numpy(Q.dequant_fp4(kv["v_codes"], kv["v_scales"], d))
    q = torch.from_numpy(F.bf16_decode(qb))
    ref = torch.nn.functional.scaled_dot_product_attention(
        q[None], Kh[None].expand(1, N, d).contiguous(), Vh[None].contiguous())[0].numpy()
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    # K > N padding and any permutation of the list give the same output
    out2 = A.sparse_attn(qb, kv, np.concatenate([np.arange(N)[::-1], [-1] * 9]))
    np.testing.assert_allclose(out2, ref, rtol=1e-12, atol=1e-12)


def test_attention_closed_forms():
    rng = np.random.default_rng(1)
    kv = _kv(rng, 30)
    qb = synth.to_bf16_bits(rng.standard_normal((4, 128)).astype(np.float32))
    Vh = Q.dequant_fp4(kv["v_codes"], kv["v_scales"], 128)
    out = A.sparse_attn(qb, kv, np.array([7, -1, -1]))
    assert np.array_equal(out, np.broadcast_to(Vh[7], (4, 128)))      # K = 1 -> the row itself
    zero_q = np.zeros((4, 128), dtype=np.uint16)
    out = A.sparse_attn(zero_q, kv, np.array([1, 5, 9]))
    np.testing.assert_allclose(out, np.broadcast_to(Vh[[1, 5, 9]].mean(axis=0), (4, 128)), rtol=1e-13)
    assert np.all(A.sparse_attn(qb, kv, np.array([-1, -1])) == 0)


def _stack_case(modes, N=600, K=16, P=64, seed=0):
    cfg = synth.small("stack_b32_n262144", N=N, K=K, P=P, B=1, modes=tuple(modes), seed=seed)
    kb, vb = synth.kv_bf16(cfg, 0)
    kc, ks = Q.quant_fp4(kb)
    vc, vs = Q.quant_fp4(vb)
    cache = dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs,
                 k_idx=synth.k_idx(cfg, 0), k_idx_dtype=cfg["k_idx_dtype"])
    layers = [dict(q=synth.q_bf16(cfg, li, 0)[0], q_idx=synth.q_idx(cfg, li, 0)[0],
                   q_idx_dtype=cfg["q_idx_dtype"]) for li in range(len(modes))]
    return cfg, cache, layers


def test_plan_reuse_equals_attention_on_inherited_positions():
    modes = ["full", "reindex", "reuse", "reuse"]
    cfg, cache, layers = _stack_case(modes)
    res = PL.run_decode(modes, cache, layers, cfg["K"], cfg["P"])
    assert np.array_equal(res[2]["idx"], res[1]["idx"]) and np.array_equal(res[3]["idx"], res[1]["idx"])
    for li in (2, 3):
        direct = A.sparse_attn(layers[li]["q"], cache, res[1]["idx"])
        assert np.array_equal(res[li]["out"], direct)
    pool = set(res[0]["pool"].tolist())
    assert set(res[0]["idx"].tolist()) <= pool and set(res[1]["idx"].tolist()) <= pool
    assert len(pool) == cfg["P"]


def test_plan_reindex_over_whole_context_pool_equals_full():
    modes = ["full", "reindex"]
    cfg, cache, layers = _stack_case(modes, N=500, K=20, P=500)
    res = PL.run_decode(modes, cache, layers, cfg["K"], cfg["P"])
    assert res[0]["pool"].tolist() == list(range(500))
    # a Full layer with the Reindex layer's indexer query selects the same positions
    full2 = PL.run_decode(["full"], cache, [layers[1]], cfg["K"])
    assert np.array_equal(res[1]["idx"], full2[0]["idx"])


def test_plan_validation():
    with pytest.raises(ValueError):
        PL.validate_plan(["reuse", "full"], 4, 8)
    with pytest.raises(ValueError):
        PL.validate_plan(["reindex"], 4, 8)
    with pytest.raises(ValueError):
        PL.validate_plan(["full", "reindex"], 8, 4)
    assert PL.validate_plan(["full", "reuse"], 8) == ["full", "reuse"]


def test_prefill_causal_and_last_query_equals_decode():
    cfg, cache, layers = _stack_case(["full"], N=300, K=12)
    qi = np.stack([synth.q_idx(cfg, 0, 0)[0]] * 3)
    qb = np.stack([synth.q_bf16(cfg, 0, 0)[0]] * 3)
    q_pos = np.array([5, 100, 299])
    idx, out = PL.prefill_full(qi, cfg["q_idx_dtype"], q_pos, qb, cache, cfg["K"])
    for i in range(3):
        v = idx[i][idx[i] >= 0]
        assert np.all(v <= q_pos[i])
    assert (idx[0] >= 0).sum() == 6                 # only 6 positions visible to query 0
    dec = PL.run_decode(["full"], cache, [dict(layers[0], q=qb[2], q_idx=qi[2])], cfg["K"])
    assert np.array_equal(idx[2], dec[0]["idx"]) and np.array_equal(out[2], dec[0]["out"])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_attention_bf16_rows_equals_quantized_planes(seed):
    """The oracle's bf16-rows input (only the listed rows are quantized) against the stored-planes input
    (the whole plane quantized first, then the listed rows dequantized): bit-identical outputs on ragged,
    unsorted, repeating and padded position lists, and each gathered row equals the plane's row."""
    rng = np.random.default_rng(seed)
    N, H, d = 257, 5, 128
    kb = synth.to_bf16_bits((rng.standard_normal((N, d)) * np.exp(rng.uniform(-6, 6, (N, 1)))).astype(np.float32))
    vb = synth.to_bf16_bits((rng.standard_normal((N, d)) * 3).astype(np.float32))
    kc, ks = Q.quant_fp4(kb)
    vc, vs = Q.quant_fp4(vb)
    planes = dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs)
    rows = dict(k_bf16=kb, v_bf16=vb)
    qb = synth.to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))
    lists = [rng.permutation(N)[:37], np.array([N - 1, 0, 3, 3, 200, -1, -1]), rng.integers(0, N, 129),
             np.array([-1, 42, -1]), np.arange(N)[::-1]]
    for idx in lists:
        a = A.sparse_attn(qb, rows, idx)
        b = A.sparse_attn(qb, planes, idx)
        assert np.array_equal(a, b)
        sel = idx[idx >= 0]
        for which, plane in (("k", Q.dequant_fp4(kc, ks, d)), ("v", Q.dequant_fp4(vc, vs, d))):
            assert np.array_equal(A.kv_rows(rows, which, sel, d), plane[sel])
    # a one-position list returns that row of V exactly, from either input form
    out = A.sparse_attn(qb, rows, np.array([-1, 77, -1]))
    assert np.array_equal(out, np.broadcast_to(Q.dequant_fp4(vc, vs, d)[77], (H, d)))


def test_swa_attention_pins():
    """Sliding-window branch: with no window rows it is the sparse attention; with no sparse positions it is
    dense attention over the window (torch SDPA in fp64); a window row equal to a selected main-cache row
    counts twice (two keys of one softmax); both parts together equal SDPA over the concatenated keys."""
    rng = np.random.default_rng(7)
    N, H, d, Wn = 60, 4, 128, 24
    kv = _kv(rng, N, d)
    qb = synth.to_bf16_bits(rng.standard_normal((H, d)).astype(np.float32))
    wk = synth.to_bf16_bits(rng.standard_normal((Wn, d)).astype(np.float32))
    wv = synth.to_bf16_bits(rng.standard_normal((Wn, d)).astype(np.float32))
    idx = np.array([3, 17, -1, 40, 41])
    empty = np.zeros((0, d), dtype=np.uint16)
    assert np.array_equal(A.sparse_attn_swa(qb, kv, idx, empty, empty), A.sparse_attn(qb, kv, idx))
    q = torch.from_numpy(F.bf16_decode(qb))
    Kw, Vw = torch.from_numpy(F.bf16_decode(wk)), torch.from_numpy(F.bf16_decode(wv))
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], Kw[None], Vw[None])[0].numpy()
    np.testing.assert_allclose(A.sparse_attn_swa(qb, kv, np.array([-1, -1]), wk, wv), ref, rtol=1e-12, atol=1e-12)
    Kh = torch.from_numpy(Q.dequant_fp4(kv["k_codes"], kv["k_scales"], d))[[3, 17, 40, 41]]
    Vh = torch.from_numpy(Q.dequant_fp4(kv["v_codes"], kv["v_scales"], d))[[3, 17, 40, 41]]
    ref = torch.nn.functional.scaled_dot_product_attention(q[None], torch.cat([Kh, Kw])[None],
                                                           torch.cat([Vh, Vw])[None])[0].numpy()
    np.testing.assert_allclose(A.sparse_attn_swa(qb, kv, idx, wk, wv), ref, rtol=1e-12, atol=1e-12)
    # a window row identical to main-cache row 3 (as bf16 of its dequantized values) is a second key
    k3 = synth.to_bf16_bits(Q.dequant_fp4(kv["k_codes"], kv["k_scales"], d)[3:4].astype(np.float32))
    v3 = synth.to_bf16_bits(Q.dequant_fp4(kv["v_codes"], kv["v_scales"], d)[3:4].astype(np.float32))
    two = A.sparse_attn_swa(qb, kv, np.array([3]), k3, v3)
    np.testing.assert_allclose(two, A.sparse_attn(qb, kv, np.array([3])), rtol=1e-12)
    assert np.all(A.sparse_attn_swa(qb, kv, np.array([-1]), empty, empty) == 0)


def _group_cache(cfg, b, seed_shift):
    c2 = dict(cfg, seed=cfg["seed"] + seed_shift)
    kb, vb = synth.kv_bf16(c2, b)
    kc, ks = Q.quant_fp4(kb)
    vc, vs = Q.quant_fp4(vb)
    return dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, k_idx=synth.k_idx(c2, b), k_idx_dtype=cfg["k_idx_dtype"])


def test_plan_with_several_full_layers_runs_groups_on_their_own_caches():
    """[Full, Reindex, Reuse, Full, Reindex, Reuse] over two caches (one per Full layer): each half equals
    the three-layer plan on its own cache, so a later Full layer's pool and KV replace the first's."""
    modes = ["full", "reindex", "reuse", "full", "reindex", "reuse"]
    cfg, _, layers = _stack_case(modes, N=700, K=16, P=64)
    caches = [_group_cache(cfg, 0, 0), _group_cache(cfg, 0, 1)]
    res = PL.run_decode(modes, caches, layers, cfg["K"], cfg["P"])
    a = PL.run_decode(modes[:3], caches[0], layers[:3], cfg["K"], cfg["P"])
    b = PL.run_decode(modes[3:], caches[1], layers[3:], cfg["K"], cfg["P"])
    for got, ref in zip(res, a + b):
        assert np.array_equal(got["idx"], ref["idx"]) and np.array_equal(got["out"], ref["out"])
    assert not np.array_equal(res[3]["pool"], res[0]["pool"])
    assert PL.groups(modes) == [0, 0, 0, 1, 1, 1]


def test_prefill_plan_query_equals_decode_on_its_causal_prefix():
    """Every query of a prefill chunk through [Full, Reindex, Reuse, Reuse] equals a decode step of the
    same plan whose context is the query's causal prefix (positions 0..q_pos), layer by layer - including
    queries whose prefix is shorter than the pool (padded pools) or than K."""
    modes = ["full", "reindex", "reuse", "reuse"]
    cfg, cache, _ = _stack_case(modes, N=400, K=12, P=40)
    Qn = 6
    q_pos = np.array([3, 11, 39, 40, 200, 399])
    layers = [dict(q=np.stack([synth.q_bf16(cfg, li * 10 + i, 0)[0] for i in range(Qn)]),
                   q_idx=np.stack([synth.q_idx(cfg, li * 10 + i, 0)[0] for i in range(Qn)]),
                   q_idx_dtype=cfg["q_idx_dtype"]) for li in range(len(modes))]
    res = PL.run_prefill(modes, cache, layers, q_pos, cfg["K"], cfg["P"])
    for i, qp in enumerate(q_pos):
        pre = {k: (v[: qp + 1] if k != "k_idx_dtype" else v) for k, v in cache.items()}
        dec = PL.run_decode(modes, pre, [dict(q=L["q"][i], q_idx=L["q_idx"][i], q_idx_dtype=L["q_idx_dtype"])
                                         for L in layers], cfg["K"], cfg["P"])
        for li in range(len(modes)):
            assert np.array_equal(res[li][0][i], dec[li]["idx"]), (i, li)
            assert np.array_equal(res[li][1][i], dec[li]["out"]), (i, li)
        assert np.all(res[1][0][i][res[1][0][i] >= 0] <= qp)
