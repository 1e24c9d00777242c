"""Helpers shared by the GPU parity tests: moving seeded inputs to the device and the
comparison rules (bit-exact codes and positions with the near-tie excusal for
top-K, max relative error per output row for attention)."""

import numpy as np
import torch

ATTN_TOL = 2e-3          # max relative error per (query, head) row
TIE_REL = 1e-5           # near-tie excusal for top-K sets


def dev_bf16(bits):
    """uint16 bf16 bit patterns (numpy) -> torch.bfloat16 on the GPU."""
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda()


def dev_key(a, dtype):
    """Stored indexer values -> device tensor of the matching torch dtype."""
    if dtype == "f32":
        return dev_f32(a)
    if dtype == "bf16":
        return dev_bf16(a)
    return dev_u8(a).view(torch.float8_e4m3fn)


def host(t):
    return t.detach().cpu().numpy()


def compare_topk(gpu_idx, ref_idx, ref_scores_at, K):
    """Compare one row's position sets.

    Returns "exact" or "excused"; raises AssertionError otherwise. A mismatch is
    excused only if every position in the symmetric difference has an oracle
    score within TIE_REL * |s_K| of the oracle's K-th score s_K.
    """
    g = np.asarray(gpu_idx)
    r = np.asarray(ref_idx)
    if np.array_equal(g, r):
        return "exact"
    gs, rs = set(g[g >= 0].tolist()), set(r[r >= 0].tolist())
    diff = gs ^ rs
    ref_valid = r[r >= 0]
    s_ref = np.array([ref_scores_at(p) for p in ref_valid], dtype=np.float64)
    s_k = s_ref.min() if s_ref.size else 0.0
    for p in diff:
        s = ref_scores_at(p)
        assert abs(s - s_k) <= TIE_REL * max(abs(s_k), 1e-30), (p, s, s_k)
    assert len(gs) == len(rs), (len(gs), len(rs))
    assert np.all(np.diff(g[g >= 0]) > 0), "positions not ascending"
    return "excused"


def max_rel_err_rows(got, ref):
    """max over rows of max|got-ref| / max|ref| (rows = last axis slices)."""
    got = np.asarray(got, dtype=np.float64).reshape(-1, got.shape[-1])
    ref = np.asarray(ref, dtype=np.float64).reshape(-1, ref.shape[-1])
    den = np.abs(ref).max(axis=1)
    num = np.abs(got - ref).max(axis=1)
    rel = np.where(den > 0, num / np.where(den > 0, den, 1), num)
    return float(rel.max())
