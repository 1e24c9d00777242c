"""GPU parity of the layer plan (Full / Reindex / Reuse) and the Full-layer prefill
against the oracle, end to end from bf16 KV rows and indexer inputs."""

import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import plan as OP
from oracle import quant as OQ
from oracle import scores as OS
from oracle.attention import sparse_attn as o_attn
from oracle.topk import topk as o_topk
from tests.parity import ATTN_TOL, compare_topk, dev_bf16, dev_key, host, max_rel_err_rows

pytestmark = pytest.mark.gpu


def build_case(cfg, B=None, with_oracle=True):
    """Device cache + per-layer inputs for a workload, and the oracle's view of the same inputs."""
    B = cfg["B"] if B is None else B
    N, L = cfg["N"], len(cfg["modes"])
    kidx = np.stack([synth.k_idx(cfg, b) for b in range(B)])
    cache = C.KVCache(B, N, k_idx=dev_key(kidx, cfg["k_idx_dtype"]))
    ocache = []
    for b in range(B):
        kb, vb = synth.kv_bf16(cfg, b)
        cache.fill(dev_bf16(kb), dev_bf16(vb), row0=b * N)
        if with_oracle:
            kc, ks = OQ.quant_fp4(kb)
            vc, vs = OQ.quant_fp4(vb)
            ocache.append(dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, k_idx=kidx[b],
                               k_idx_dtype=cfg["k_idx_dtype"]))
    layers, olayers = [], []
    for li in range(L):
        q = np.stack([synth.q_bf16(cfg, li, b)[0] for b in range(B)])          # [B][H][d]
        qi = np.stack([synth.q_idx(cfg, li, b)[0] for b in range(B)])          # [B][d_idx]
        layers.append(dict(q=dev_bf16(q), q_idx=dev_key(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, cfg["H"], cfg["d"], dtype=torch.float32, device="cuda"),
                           idx_out=torch.empty(B, cfg["K"], dtype=torch.int32, device="cuda")))
        olayers.append([dict(q=q[b], q_idx=qi[b], q_idx_dtype=cfg["q_idx_dtype"]) for b in range(B)])
    if cfg.get("P"):
        layers[0]["pool_out"] = torch.empty(B, cfg["P"], dtype=torch.int32, device="cuda")
    return cache, layers, ocache, olayers


def make_plan(cfg):
    return C.Plan(cfg["modes"], K=cfg["K"], P=cfg.get("P") or 0, H=cfg["H"], d=cfg["d"], d_idx=cfg["d_idx"],
                  q_idx_dtype=cfg["q_idx_dtype"], k_idx_dtype=cfg["k_idx_dtype"])


SCALE = float(np.float32(1 / math.sqrt(128)))


def check_against_oracle(cfg, layers, ocache, olayers, seqs):
    stats = {"exact": 0, "excused": 0}
    modes = list(cfg["modes"])
    for b in seqs:
        res = OP.run_decode(modes, ocache[b], [olayers[li][b] for li in range(len(modes))], cfg["K"], cfg.get("P"),
                            softmax_scale=SCALE)
        pool = None
        for li, mode in enumerate(modes):
            g_idx = host(layers[li]["idx_out"][b]) if mode != "reuse" else None
            if mode == "full" and "pool" in res[li]:
                pool = res[li]["pool"]
                g_pool = host(layers[li]["pool_out"][b])
                s_full = OS.index_scores(olayers[li][b]["q_idx"], cfg["q_idx_dtype"], ocache[b]["k_idx"],
                                         cfg["k_idx_dtype"])
                stats[compare_topk(g_pool, pool, lambda p: s_full[p], cfg["P"])] += 1
            if mode == "full":
                s = OS.index_scores(olayers[li][b]["q_idx"], cfg["q_idx_dtype"], ocache[b]["k_idx"], cfg["k_idx_dtype"])
                stats[compare_topk(g_idx, res[li]["idx"], lambda p: s[p], cfg["K"])] += 1
            elif mode == "reindex":
                s = OS.index_scores(olayers[li][b]["q_idx"], cfg["q_idx_dtype"], ocache[b]["k_idx"], cfg["k_idx_dtype"])
                stats[compare_topk(g_idx, res[li]["idx"], lambda p: s[p], cfg["K"])] += 1
            # attention rows are compared where the positions agree exactly
            if mode != "reuse" and not np.array_equal(g_idx, res[li]["idx"]):
                continue
            err = max_rel_err_rows(host(layers[li]["out"][b]), res[li]["out"])
            assert err <= ATTN_TOL, (b, li, err)
    return stats


def test_full_layer_n2048_end_to_end():
    cfg = synth.WORKLOADS["full_n2048"]
    cache, layers, ocache, olayers = build_case(cfg)
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    stats = check_against_oracle(cfg, layers, ocache, olayers, range(cfg["B"]))
    assert stats["exact"] == 1, stats


@pytest.mark.parametrize("B,N,K,P", [(3, 20000, 64, 512), (2, 70001, 2048, 8192), (1, 5000, 100, 100),
                                     (2, 40000, 512, 20000),    # a pool above 16,384: the general select
                                     (20, 20000, 512, 16384)])  # 16 chunks per pool row: two select launches
def test_stack_full_reindex_reuse(B, N, K, P):
    cfg = synth.small("stack_b32_n262144", B=B, N=N, K=K, P=P)
    cache, layers, ocache, olayers = build_case(cfg)
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    stats = check_against_oracle(cfg, layers, ocache, olayers, range(B))
    assert stats["excused"] == 0, stats
    # Reuse layers inherit the Reindex layer's positions bit for bit ...
    idx1 = layers[1]["idx_out"]
    for li in (2, 3):
        direct = C.sparse_attn_fp4(layers[li]["q"][:, None], cache, idx1[:, None], softmax_scale=SCALE)
        assert torch.equal(direct[:, 0], layers[li]["out"])
    # ... Reindex positions lie inside the pool, and so do the Full layer's
    pool = host(layers[0]["pool_out"])
    for b in range(B):
        ps = set(pool[b].tolist())
        assert set(host(idx1[b]).tolist()) - {-1} <= ps
        assert set(host(layers[0]["idx_out"][b]).tolist()) - {-1} <= ps


@pytest.mark.parametrize("N,P,K,zero_q", [(20000, 3001, 1500, False), (20000, 3001, 1500, True),
                                           (9000, 1025, 1025, True), (40000, 16384, 2048, False),
                                           (40000, 16384, 2048, True), (5000, 1030, 7, False)])
def test_reindex_pool_shapes_and_ties(N, P, K, zero_q):
    """Reindex over pools with a ragged tail (P not a multiple of 4 or of 1024), the largest pool
    the single-exchange select takes, K = P, and an all-zero Reindex query, whose scores all tie:
    then the positions are the K lowest pool positions."""
    cfg = synth.small("stack_b32_n262144", B=2, N=N, K=K, P=P, modes=("full", "reindex", "reuse"))
    cache, layers, ocache, olayers = build_case(cfg)
    if zero_q:
        layers[1]["q_idx"].zero_()
        for b in range(2):
            olayers[1][b]["q_idx"] = np.zeros_like(olayers[1][b]["q_idx"])
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    stats = check_against_oracle(cfg, layers, ocache, olayers, range(2))
    assert stats["excused"] == 0, stats
    if zero_q:
        pool = layers[0]["pool_out"]
        assert torch.equal(layers[1]["idx_out"], pool[:, :K])
    idx1 = layers[1]["idx_out"]
    direct = C.sparse_attn_fp4(layers[2]["q"][:, None], cache, idx1[:, None], softmax_scale=SCALE)
    assert torch.equal(direct[:, 0], layers[2]["out"])


def test_pool_with_padding_when_most_scores_are_nan():
    """Keys whose rows hold E4M3 NaN score NaN and are never selected: with 1000 finite scores per row,
    the Full layer's pool (P = 2048) is 1000 positions then -1 padding, and both the Full and the
    Reindex top-K (K = 1500) are 1000 positions then -1."""
    cfg = synth.small("stack_b32_n262144", B=2, N=3000, K=1500, P=2048, modes=("full", "reindex", "reuse"))
    cache, layers, ocache, olayers = build_case(cfg)
    rng = np.random.default_rng(11)
    kdev = cache.k_idx.view(torch.uint8)
    for b in range(2):
        nan_pos = np.sort(rng.choice(3000, size=2000, replace=False))
        ocache[b]["k_idx"] = ocache[b]["k_idx"].copy()
        ocache[b]["k_idx"][nan_pos] = 0x7F
        kdev[b, torch.from_numpy(nan_pos).cuda()] = 0x7F
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    stats = check_against_oracle(cfg, layers, ocache, olayers, range(2))
    assert stats["excused"] == 0, stats
    for li, name in ((0, "pool_out"), (0, "idx_out"), (1, "idx_out")):
        got = host(layers[li][name])
        assert (got[:, :1000] >= 0).all() and (got[:, 1000:] == -1).all(), (li, name)


def test_reindex_over_whole_context_equals_full():
    """A pool of every position: the Reindex layer selects what a Full layer with its query selects.
    The positions agree bit for bit; the outputs - the Reindex layer's attention runs inside its
    select, with another split of the positions, so another summation order - both meet the oracle."""
    cfg = synth.small("stack_b32_n262144", B=2, N=3000, K=50, P=3000, modes=("full", "reindex"))
    cache, layers, ocache, olayers = build_case(cfg)
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    full_only = make_plan(dict(cfg, modes=("full",)))
    l2 = [dict(layers[1], out=torch.empty_like(layers[1]["out"]), idx_out=torch.empty_like(layers[1]["idx_out"]))]
    full_only.run_decode(cache, l2)
    torch.cuda.synchronize()
    assert torch.equal(layers[0]["pool_out"], torch.arange(3000, dtype=torch.int32, device="cuda").expand(2, -1))
    assert torch.equal(layers[1]["idx_out"], l2[0]["idx_out"])
    idx = host(layers[1]["idx_out"])
    for b in range(2):
        ref = o_attn(olayers[1][b]["q"], ocache[b], idx[b], SCALE)
        for got in (layers[1]["out"][b], l2[0]["out"][b]):
            assert max_rel_err_rows(host(got), ref) <= ATTN_TOL, b


def _oracle_seq(cfg, b):
    kb, vb = synth.kv_bf16(cfg, b)
    kc, ks = OQ.quant_fp4(kb)
    vc, vs = OQ.quant_fp4(vb)
    return dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs, k_idx=synth.k_idx(cfg, b),
                k_idx_dtype=cfg["k_idx_dtype"])


@pytest.mark.parametrize("B,N,K,seqs", [
    (40, 32768, 256, (0, 17, 35, 36, 39)),   # 7 chunks per row, 36 rows per launch: two launches of the fused select
    (300, 4096, 64, (0, 150, 299))])        # one chunk per row: the fused attention writes its output directly
def test_full_layer_fused_attention_launch_shapes(B, N, K, seqs):
    """The Full layer's attention runs inside its select: across launches (partial states indexed by
    the launch's rows) and for rows of one chunk (no partial state); positions and outputs against
    the oracle on sampled sequences, including the first and last rows of each launch."""
    cfg = synth.small("stack_b32_n262144", B=B, N=N, K=K, modes=("full",))
    cache, layers, _, olayers = build_case(cfg, with_oracle=False)
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    ocache = {b: _oracle_seq(cfg, b) for b in seqs}
    for b in seqs:
        res = OP.run_decode(["full"], ocache[b], [olayers[0][b]], K, None, softmax_scale=SCALE)
        s = OS.index_scores(olayers[0][b]["q_idx"], cfg["q_idx_dtype"], ocache[b]["k_idx"], cfg["k_idx_dtype"])
        g_idx = host(layers[0]["idx_out"][b])
        assert compare_topk(g_idx, res[0]["idx"], lambda p: s[p], K) == "exact", b
        assert max_rel_err_rows(host(layers[0]["out"][b]), res[0]["out"]) <= ATTN_TOL, b


def test_plan_is_deterministic():
    cfg = synth.small("stack_b32_n262144", B=4, N=40000, K=256, P=1024)
    cache, layers, _, _ = build_case(cfg, with_oracle=False)
    plan = make_plan(cfg)
    plan.run_decode(cache, layers)
    first = [(L["idx_out"].clone(), L["out"].clone()) for L in layers]
    for _ in range(2):
        plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    for (i0, o0), L in zip(first, layers):
        assert torch.equal(i0, L["idx_out"]) and torch.equal(o0, L["out"])


def test_prefill_full_causal():
    cfg = synth.small("stack_b4_n1m", B=2, N=5000, K=32, modes=("full",))
    cache, layers, ocache, _ = build_case(cfg)
    Q = 12
    q_pos = np.array([[0, 5, 31, 32, 100, 1000, 2500, 4000, 4990, 4997, 4998, 4999]] * 2, dtype=np.int64)
    qi = np.stack([synth.prefill_q_idx(cfg, b, Q) for b in range(2)])
    qb = np.stack([synth.prefill_q_bf16(cfg, b, Q) for b in range(2)])
    plan = make_plan(cfg)
    idx, out = plan.prefill_full(cache, dev_key(qi, cfg["q_idx_dtype"]), dev_bf16(qb), torch.from_numpy(q_pos).cuda())
    torch.cuda.synchronize()
    idx, out = host(idx), host(out)
    for b in range(2):
        r_idx, r_out = OP.prefill_full(qi[b], cfg["q_idx_dtype"], q_pos[b], qb[b], ocache[b], cfg["K"],
                                       softmax_scale=SCALE)
        for i in range(Q):
            s = OS.index_scores(qi[b, i], cfg["q_idx_dtype"], ocache[b]["k_idx"], cfg["k_idx_dtype"], q_pos=int(q_pos[b, i]))
            assert compare_topk(idx[b, i], r_idx[i], lambda p: s[p], cfg["K"]) == "exact"
            assert max_rel_err_rows(out[b, i], r_out[i]) <= ATTN_TOL
        assert (idx[b, 0] >= 0).sum() == 1 and idx[b, 0, 0] == 0       # query at position 0 sees only itself


def _prefill_inputs(cfg, B, Q, q_pos):
    qi = np.stack([synth.prefill_q_idx(cfg, b, Q) for b in range(B)])
    qb = np.stack([synth.prefill_q_bf16(cfg, b, Q) for b in range(B)])
    return qi, qb, torch.from_numpy(np.ascontiguousarray(q_pos)).cuda()


def test_prefill_matrix_core_indexer_matches_oracle():
    """N >= 65536 with bf16 queries and E4M3 keys takes the matrix-core candidate path; every row is
    compared with the oracle's exact top-K (near-ties excused and counted) and sampled rows' attention."""
    cfg = synth.small("stack_b4_n1m", B=2, N=70001, K=256, modes=("full",))
    cache, _, ocache, _ = build_case(cfg)
    B, Q, N, K = 2, 160, cfg["N"], cfg["K"]
    rng = np.random.default_rng(5)
    q_pos = np.stack([np.concatenate([[0, 10, 31, 32, 100, 255, 256, 4000, 40000, N - 1],
                                      np.sort(rng.integers(N - 3000, N, Q - 10))]) for _ in range(B)]).astype(np.int64)
    qi, qb, qp = _prefill_inputs(cfg, B, Q, q_pos)
    plan = make_plan(cfg)
    idx, out = plan.prefill_full(cache, dev_key(qi, cfg["q_idx_dtype"]), dev_bf16(qb), qp)
    assert plan.prefill_status(cache, Q) == 0
    idx, out = host(idx), host(out)
    stats = {"exact": 0, "excused": 0}
    for b in range(B):
        for i in range(Q):
            s = OS.index_scores(qi[b, i], cfg["q_idx_dtype"], ocache[b]["k_idx"], cfg["k_idx_dtype"],
                                q_pos=int(q_pos[b, i]))
            r_idx, _ = o_topk(s, K)
            res = compare_topk(idx[b, i], r_idx, lambda p: s[p], K)
            assert res in stats, (b, i, res)
            stats[res] += 1
            if i % 16 == 0:
                ref = o_attn(qb[b, i], ocache[b], r_idx if res == "exact" else idx[b, i], SCALE)
                assert max_rel_err_rows(out[b, i], ref) <= ATTN_TOL, (b, i)
    assert stats["exact"] >= B * Q - 2, stats


def _tied_cache(N, B=1):
    """Indexer keys all equal (every score of a query ties): candidate lists overflow."""
    kb = np.zeros((N, 128), dtype=np.uint16)
    cache = C.KVCache(B, N, k_idx=dev_key(np.full((B, N, 64), 0x38, dtype=np.uint8), "e4m3"))   # 1.0 everywhere
    for b in range(B):
        cache.fill(dev_bf16(kb), dev_bf16(kb), row0=b * N)
    return cache


def test_prefill_repair_pass_takes_lowest_positions_on_ties():
    cfg = synth.small("stack_b4_n1m", B=1, N=70001, K=256, modes=("full",))
    N, K, Q = cfg["N"], cfg["K"], 40
    cache = _tied_cache(N)
    q_pos = np.array([[N - 1 - 7 * i for i in range(Q)]], dtype=np.int64)
    qi, qb, qp = _prefill_inputs(cfg, 1, Q, q_pos)
    plan = make_plan(cfg)
    idx, _ = plan.prefill_full(cache, dev_key(qi, "bf16"), dev_bf16(qb), qp)
    assert plan.prefill_status(cache, Q) == 0
    idx = host(idx)
    for i in range(Q):
        assert np.array_equal(idx[0, i], np.arange(K)), i          # ties go to the lowest positions


def test_prefill_exact_for_every_queued_row():
    """100 queries whose candidates cannot be certified (all scores tie) - more than the 64 the
    multi-workgroup repair pass takes: every one still gets the exact top-K (ties to the lowest positions)."""
    cfg = synth.small("stack_b4_n1m", B=1, N=70001, K=256, modes=("full",))
    N, K, Q = cfg["N"], cfg["K"], 100
    cache = _tied_cache(N)
    q_pos = np.stack([np.concatenate([np.full(60, N - 1), N - 1 - 997 * np.arange(1, 41)])]).astype(np.int64)
    qi, qb, qp = _prefill_inputs(cfg, 1, Q, q_pos)
    plan = make_plan(cfg)
    idx, _ = plan.prefill_full(cache, dev_key(qi, "bf16"), dev_bf16(qb), qp)
    assert plan.prefill_status(cache, Q) == 0
    idx = host(idx)
    for i in range(Q):
        assert np.array_equal(idx[0, i], np.arange(K)), i


@pytest.mark.timeout(600)
def test_prefill_early_positions_in_a_long_context():
    """A chunk of queries at early positions of a 524,288-position cache (K = 2048): each query's
    candidates spread over the key ranges of its own causal span, so no list overflows and every
    query's top-K is exact without the repair fallback."""
    cfg = synth.small("stack_b4_n1m", B=1, N=524288, K=2048, modes=("full",))
    N, K, Q = cfg["N"], cfg["K"], 160
    cache, _, ocache, _ = build_case(cfg)
    rng = np.random.default_rng(11)
    q_pos = np.sort(np.concatenate([[0, 1, 2047, 2048, 4095, 4096, 65535, 65536],
                                    rng.integers(0, N // 4, Q - 8)]))[None].astype(np.int64)
    qi, qb, qp = _prefill_inputs(cfg, 1, Q, q_pos)
    plan = make_plan(cfg)
    idx, _ = plan.prefill_full(cache, dev_key(qi, cfg["q_idx_dtype"]), dev_bf16(qb), qp)
    assert plan.prefill_status(cache, Q) == 0
    idx = host(idx)
    for i in range(Q):
        s = OS.index_scores(qi[0, i], cfg["q_idx_dtype"], ocache[0]["k_idx"], cfg["k_idx_dtype"], q_pos=int(q_pos[0, i]))
        r_idx, _ = o_topk(s, K)
        assert compare_topk(idx[0, i], r_idx, lambda p: s[p], K) == "exact", i
