"""GPU parity at the full sizes of the decode and prefill workloads, in the launch
configuration the benchmark times (the same input builder and the same plan
calls), on sampled sequences and queries that the oracle computes one by one; the
decode index sets (Full top-K and pool, Reindex top-K) of every sequence of the
batch, which need only the indexer keys, are checked too.

Top-K position sets must match bit for bit; a mismatch is excused (and counted)
only for near-ties at the K-th score. Attention is compared stage-wise, on the
GPU's own positions, within ATTN_TOL.
"""

import math

import numpy as np
import pytest
import torch

import bench
import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import formats as F
from oracle import plan as OP
from oracle import quant as OQ
from oracle import scores as OS
from oracle.attention import sparse_attn as o_attn
from oracle.topk import topk as o_topk
from tests.parity import ATTN_TOL, compare_topk, host, max_rel_err_rows

pytestmark = pytest.mark.gpu

SCALE = float(np.float32(1 / math.sqrt(128)))


def _oracle_sequence(cfg, b):
    """Sequence b of the workload as the oracle sees it: bf16 KV rows (quantized where read) and indexer keys."""
    kb, vb = synth.kv_bf16(cfg, b)
    return dict(k_bf16=kb, v_bf16=vb, k_idx=synth.k_idx(cfg, b), k_idx_dtype=cfg["k_idx_dtype"])


def _plan(cfg, modes):
    return C.Plan(modes, K=cfg["K"], P=cfg.get("P") or 0, H=cfg["H"], d=cfg["d"], d_idx=cfg["d_idx"],
                  q_idx_dtype=cfg["q_idx_dtype"], k_idx_dtype=cfg["k_idx_dtype"])


def _check_index_sets_every_sequence(cfg, modes, layers):
    """Every sequence of the batch, not only the sampled ones: the Full layer's top-K (and pool) and the
    Reindex layer's top-K against the oracle's exact selection from the indexer scores alone (these need
    no KV rows, so the whole batch stays cheap). Stage-wise: the Reindex reference scores the GPU's own
    pool. Returns the counts of exact and excused sets."""
    K, P = cfg["K"], cfg.get("P")
    stats = {"exact": 0, "excused": 0}
    for b in range(cfg["B"]):
        kidx = synth.k_idx(cfg, b)
        pool = None
        for li, mode in enumerate(modes):
            if mode == "reuse":
                continue
            qi = synth.q_idx(cfg, li, b)[0]
            g_idx = host(layers[li]["idx_out"][b])
            if mode == "full":
                s = OS.index_scores(qi, cfg["q_idx_dtype"], kidx, cfg["k_idx_dtype"])
                r_idx, _ = o_topk(s, K)
                stats[compare_topk(g_idx, r_idx, lambda p: s[p], K)] += 1
                if "pool_out" in layers[li]:
                    pool = host(layers[li]["pool_out"][b])
                    r_pool, _ = o_topk(s, P)
                    stats[compare_topk(pool, r_pool, lambda p: s[p], P)] += 1
                    # the pool holds the layer's own top-K
                    assert np.isin(g_idx, pool).all(), (b, li)
            else:
                sp = OS.pool_scores(qi, cfg["q_idx_dtype"], kidx, cfg["k_idx_dtype"], pool)
                r_idx, _ = o_topk(sp, K, positions=pool)
                at = dict(zip(pool.tolist(), sp.tolist()))
                stats[compare_topk(g_idx, r_idx, lambda p: at[int(p)], K)] += 1
                assert np.isin(g_idx, pool).all(), (b, li)
    return stats


@pytest.mark.timeout(1500)
@pytest.mark.parametrize("workload,seqs", [("full_b64_n131072", (0, 21, 42, 63)),
                                           ("stack_b32_n262144", (0, 9, 18, 31)),
                                           ("stack_b4_n1m", (0, 2))])
def test_decode_step_full_size_sampled(workload, seqs):
    cfg = dict(synth.WORKLOADS[workload])
    modes = list(cfg["modes"])
    dev = torch.device("cuda", 0)
    cache, layers = bench.build_inputs(cfg, dev)
    plan = _plan(cfg, cfg["modes"])
    plan.run_decode(cache, layers)
    torch.cuda.synchronize()
    for li in range(len(modes)):
        assert torch.isfinite(layers[li]["out"]).all(), (workload, li)
    print(f"{workload}: top-K sets of every sequence {_check_index_sets_every_sequence(cfg, modes, layers)}")
    K, P = cfg["K"], cfg.get("P")
    stats = {"exact": 0, "excused": 0}
    for b in seqs:
        oc = _oracle_sequence(cfg, b)
        ol = [dict(q=synth.q_bf16(cfg, li, b)[0], q_idx=synth.q_idx(cfg, li, b)[0], q_idx_dtype=cfg["q_idx_dtype"])
              for li in range(len(modes))]
        res = OP.run_decode(modes, oc, ol, K, P if "reindex" in modes else None, softmax_scale=SCALE)
        prev = None
        for li, mode in enumerate(modes):
            if mode == "reuse":
                g_idx = prev
            else:
                g_idx = host(layers[li]["idx_out"][b])
                s = OS.index_scores(ol[li]["q_idx"], cfg["q_idx_dtype"], oc["k_idx"], cfg["k_idx_dtype"])
                stats[compare_topk(g_idx, res[li]["idx"], lambda p: s[p], K)] += 1
                if "pool" in res[li]:
                    g_pool = host(layers[li]["pool_out"][b])
                    stats[compare_topk(g_pool, res[li]["pool"], lambda p: s[p], P)] += 1
            prev = g_idx
            ref = res[li]["out"] if np.array_equal(g_idx, res[li]["idx"]) else o_attn(ol[li]["q"], oc, g_idx, SCALE)
            err = max_rel_err_rows(host(layers[li]["out"][b]), ref)
            assert err <= ATTN_TOL, (workload, b, li, err)
    print(f"{workload}: top-K sets {stats}")


@pytest.mark.timeout(1500)
def test_prefill_full_size_sampled():
    """The 4 x 1M-context prefill chunk (4096 queries per sequence at the last positions) through the
    matrix-core indexer path; 59 sampled queries (both ends of the chunk and 12 seeded random ones per
    sequence) against the oracle's exact causal top-K and attention."""
    cfg = dict(synth.WORKLOADS["stack_b4_n1m"])
    B, N, Q, K = cfg["B"], cfg["N"], cfg["prefill_Q"], cfg["K"]
    dev = torch.device("cuda", 0)
    cache, _ = bench.build_inputs(cfg, dev)
    qi = np.stack([synth.prefill_q_idx(cfg, b, Q) for b in range(B)])
    qb = np.stack([synth.prefill_q_bf16(cfg, b, Q) for b in range(B)])
    qi_t = torch.from_numpy(np.ascontiguousarray(qi).view(np.int16)).view(torch.bfloat16).to(dev)
    qb_t = torch.from_numpy(np.ascontiguousarray(qb).view(np.int16)).view(torch.bfloat16).to(dev)
    q_pos = np.stack([np.arange(N - Q, N, dtype=np.int64)] * B)
    plan = _plan(cfg, ("full",))
    idx, out = plan.prefill_full(cache, qi_t, qb_t, torch.from_numpy(q_pos).to(dev))
    assert plan.prefill_status(cache, Q) == 0
    idx, out = host(idx), host(out)
    stats = {"exact": 0, "excused": 0}
    fixed = {0: (0, 1000, 2049, 4095), 1: (7, 3333), 2: (512, 4094), 3: (1, 2222, 4095)}
    for b in range(B):
        # the fixed queries (both ends of the chunk) plus 12 seeded random ones per sequence
        extra = np.random.default_rng([7, b]).choice(Q, 12, replace=False)
        queries = sorted(set(fixed[b]) | set(int(i) for i in extra))
        oc = _oracle_sequence(cfg, b)
        for i in queries:
            s = OS.index_scores(qi[b, i], cfg["q_idx_dtype"], oc["k_idx"], cfg["k_idx_dtype"], q_pos=int(q_pos[b, i]))
            r_idx, _ = o_topk(s, K)
            stats[compare_topk(idx[b, i], r_idx, lambda p: s[p], K)] += 1
            err = max_rel_err_rows(out[b, i], o_attn(qb[b, i], oc, idx[b, i], SCALE))
            assert err <= ATTN_TOL, (b, i, err)
    print(f"prefill: top-K sets {stats}")


@pytest.mark.timeout(900)
def test_quant_dequant_full_size_sampled():
    """kv_quant_fp4 and kv_dequant_fp4 over the whole 1,048,576 x 512 quantize workload in the benchmark's
    launch configuration, compared bit for bit with the oracle on row blocks at the start, the end and
    between: each of the 16,384 workgroups of both kernels owns 64 consecutive rows (2048 groups or
    4096 half-groups, four passes of 256 lanes), so every block spans the ranges of several workgroups,
    the first and the last included."""
    cfg = dict(synth.WORKLOADS["quant_1m_x512"])
    T, Cc, rb = cfg["T"], cfg["C"], cfg["row_block"]
    dev = torch.device("cuda", 0)
    x = bench.build_quant_input(cfg, dev)
    codes, scales = C.kv_quant_fp4(x)
    y = C.kv_dequant_fp4(codes, scales, Cc)
    torch.cuda.synchronize()
    nb = T // rb
    blocks = sorted({0, 1, nb // 4, nb // 2, nb // 2 + 1, 3 * nb // 4, nb - 2, nb - 1})
    for blk in blocks:
        xb = synth.quant_rows(cfg, blk)
        rc, rs = OQ.quant_fp4(xb)
        sl = slice(blk * rb, (blk + 1) * rb)
        assert np.array_equal(host(scales[sl]), rs), blk
        assert np.array_equal(host(codes[sl]), rc), blk
        got = F.bf16_decode(host(y[sl].view(torch.int16)).view(np.uint16))
        ref = OQ.dequant_fp4(rc, rs, Cc)
        assert np.array_equal(got, ref) and np.array_equal(np.signbit(got), np.signbit(ref)), blk
    print(f"quant full size: {len(blocks)} row blocks of {rb} bit-exact")
