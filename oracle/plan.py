"""The CSA2 layer plan (Full / Reindex / Reuse) for one sequence, and the Full-layer prefill.

[zaikei] "■CSA2とFP4でキャッシュを圧縮": each CSA2 layer is fixed to one of Full,
Reindex, Reuse. Full computes KV data and reference positions afresh; Reindex
reuses the preceding layers' KV data and re-selects positions; Reuse inherits
both KV data and positions. [jiwasawa] CSA2: modes are assigned statically;
Full computes the main KV and its own indexer Q and fresh Top-K indices;
Reindex shares main KV and indexer K from an earlier layer and re-scores with
its own Q; Reuse shares main KV and the Top-K indices and skips the indexer.
Hierarchical Sparse Indexer: the first Full layer picks a candidate pool from
the whole context and later Reindex layers search only inside it.

Readings:
  * the pool is the top-P of the first Full layer's scores under the same
    order as top-K (so it contains that layer's top-K);
  * a Reindex layer scores the pool positions with its own indexer query and
    the first Full layer's indexer keys, and selects top-K from the pool;
  * a Reuse layer takes the positions of the immediately preceding layer;
  * every Full layer computes KV afresh, so it opens a group: its main KV
    cache and indexer keys, and the pool it picks (when a Reindex layer
    follows in the group), serve the Reindex and Reuse layers after it up to
    the next Full layer; with one Full layer this is the single shared cache
    and "the first Full layer's pool";
  * plan validity: the first layer is Full; a Reindex needs an earlier Full
    (and a pool, so P >= K); a Reuse needs a predecessor.
"""

import numpy as np

from .attention import sparse_attn, sparse_attn_swa
from .scores import index_scores, pool_scores
from .topk import topk

FULL, REINDEX, REUSE = "full", "reindex", "reuse"


def validate_plan(modes, K, P=None):
    modes = list(modes)
    if not modes or modes[0] != FULL:
        raise ValueError("first layer must be Full")
    for m in modes:
        if m not in (FULL, REINDEX, REUSE):
            raise ValueError(f"unknown mode {m}")
    if REINDEX in modes:
        if P is None or P < K:
            raise ValueError("a Reindex layer needs a pool with P >= K")
    return modes


def groups(modes):
    """Group index of each layer: the number of Full layers up to and including it, minus one."""
    out, gi = [], -1
    for m in modes:
        gi += m == FULL
        out.append(gi)
    return out


def _group_needs_pool(modes):
    """Per group: whether a Reindex layer follows its Full layer."""
    g = groups(modes)
    need = [False] * (g[-1] + 1)
    for m, gi in zip(modes, g):
        need[gi] |= m == REINDEX
    return need


def run_decode(modes, cache, layers, K, P=None, softmax_scale=None):
    """One decode step of the stack for ONE sequence.

    cache: dict with 'k_codes', 'k_scales', 'v_codes', 'v_scales' (main KV,
    [N][d/2] and [N][d/16]), 'k_idx' ([N][d_idx] stored), 'k_idx_dtype' - or a
    list of such dicts, one per Full layer (group).
    layers: list (one per layer) of dicts with 'q' ((H, d) bf16 bits) and, for
    Full and Reindex layers, 'q_idx' ((d_idx,) stored) and 'q_idx_dtype'; a
    layer with a sliding-window branch also has 'win_k', 'win_v' ((w, d) bf16
    bits: its window's valid rows).
    Returns a list of dicts per layer: 'idx' (K,), 'out' (H, d) fp64 and, for
    the first Full layer when the plan has a Reindex, 'pool' (P,).
    """
    modes = validate_plan(modes, K, P)
    caches = cache if isinstance(cache, (list, tuple)) else [cache]
    grp, need_pool = groups(modes), _group_needs_pool(modes)
    pool = None
    prev_idx = None
    results = []
    for mode, layer, gi in zip(modes, layers, grp):
        res = {}
        cache = caches[gi]
        if mode == FULL:
            s = index_scores(layer["q_idx"], layer["q_idx_dtype"], cache["k_idx"], cache["k_idx_dtype"])
            pool = None
            if need_pool[gi]:
                pool, _ = topk(s, P)
                res["pool"] = pool
            idx, _ = topk(s, K)
        elif mode == REINDEX:
            s = pool_scores(layer["q_idx"], layer["q_idx_dtype"], cache["k_idx"], cache["k_idx_dtype"], pool)
            idx, _ = topk(s, K, positions=pool)
        else:
            idx = prev_idx.copy()
        res["idx"] = idx
        if layer.get("win_k") is not None:      # the layer's sliding-window branch, in the same softmax
            res["out"] = sparse_attn_swa(layer["q"], cache, idx, layer["win_k"], layer["win_v"], softmax_scale)
        else:
            res["out"] = sparse_attn(layer["q"], cache, idx, softmax_scale)
        results.append(res)
        prev_idx = idx
    return results


def run_prefill(modes, cache, layers, q_pos, K, P=None, softmax_scale=None, queries=None):
    """A prefill chunk of Q queries of ONE sequence through every layer of the plan.

    Each query is a decode step at its own position: the causal rule of
    prefill_full (positions <= q_pos[i]) in its Full layers, and its own pool,
    Reindex selection and Reuse inheritance. cache: as run_decode. layers: one
    dict per layer with 'q' ((Q, H, d) bf16 bits) and, for Full and Reindex
    layers, 'q_idx' ((Q, d_idx) stored) and 'q_idx_dtype'. Returns per layer
    (idx (Q', K), out (Q', H, d)) for the queries taken (all, or `queries`).
    """
    modes = validate_plan(modes, K, P)
    caches = cache if isinstance(cache, (list, tuple)) else [cache]
    grp, need_pool = groups(modes), _group_needs_pool(modes)
    rows = range(len(q_pos)) if queries is None else list(queries)
    res = [([], []) for _ in modes]
    for i in rows:
        pool, prev_idx = None, None
        for li, (mode, layer, gi) in enumerate(zip(modes, layers, grp)):
            cache = caches[gi]
            if mode == FULL:
                s = index_scores(layer["q_idx"][i], layer["q_idx_dtype"], cache["k_idx"], cache["k_idx_dtype"],
                                 q_pos=int(q_pos[i]))
                pool = topk(s, P)[0] if need_pool[gi] else None
                idx, _ = topk(s, K)
            elif mode == REINDEX:
                s = pool_scores(layer["q_idx"][i], layer["q_idx_dtype"], cache["k_idx"], cache["k_idx_dtype"], pool)
                idx, _ = topk(s, K, positions=pool)
            else:
                idx = prev_idx.copy()
            res[li][0].append(idx)
            res[li][1].append(sparse_attn(layer["q"][i], cache, idx, softmax_scale))
            prev_idx = idx
    return [(np.stack(a), np.stack(b)) for a, b in res]


def prefill_full(q_idx, q_idx_dtype, q_pos, q, cache, K, softmax_scale=None, queries=None):
    """Full-layer prefill for a chunk of queries of ONE sequence.

    q_idx: (Q, d_idx) stored; q_pos: (Q,) positions; q: (Q, H, d) bf16 bits.
    Reading (causal): query i may select only positions <= q_pos[i].
    `queries` restricts the work to a subset of query rows (sampling).
    Returns (idx (Q', K), out (Q', H, d)).
    """
    rows = range(len(q_pos)) if queries is None else list(queries)
    idx_all, out_all = [], []
    for i in rows:
        s = index_scores(q_idx[i], q_idx_dtype, cache["k_idx"], cache["k_idx_dtype"], q_pos=int(q_pos[i]))
        idx, _ = topk(s, K)
        idx_all.append(idx)
        out_all.append(sparse_attn(q[i], cache, idx, softmax_scale))
    return np.stack(idx_all), np.stack(out_all)
