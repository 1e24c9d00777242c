"""The allocation-free attention entry point (csa2_sparse_attn_fp4_noalloc, scratch in a fixed device
array) against the workspace entry point csa2_sparse_attn_fp4, through the C ABI: bit-identical outputs
on two calls in a row, the second with a smaller input, plus the oracle on sampled rows."""

import math

import numpy as np
import pytest
import torch

import fp4_compressed_sparse_kv_amd as C
import synth
from oracle import quant as OQ
from oracle.attention import sparse_attn as o_attn
from tests.parity import ATTN_TOL, dev_bf16, host, max_rel_err_rows

pytestmark = pytest.mark.gpu


def _case(N, seed):
    rng = np.random.default_rng(seed)
    kb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    vb = synth.to_bf16_bits(rng.standard_normal((N, 128)).astype(np.float32))
    cache = C.KVCache(1, N)
    cache.fill(dev_bf16(kb), dev_bf16(vb))
    kc, ks = OQ.quant_fp4(kb)
    vc, vs = OQ.quant_fp4(vb)
    return cache, dict(k_codes=kc, k_scales=ks, v_codes=vc, v_scales=vs), rng


@pytest.mark.parametrize("first,second", [((32, 16, 2048), (5, 8, 300)), ((255, 16, 512), (1, 4, 2048)),
                                          ((300, 16, 256), (64, 16, 2048))])
def test_noalloc_attention_matches_workspace_entry_point(first, second):
    N = 20000
    cache, okv, rng = _case(N, sum(first))
    scale = float(np.float32(1 / math.sqrt(128)))
    for Q, H, K in (first, second):                        # two calls in a row, the second smaller
        qb = synth.to_bf16_bits(rng.standard_normal((1, Q, H, 128)).astype(np.float32))
        idx = np.stack([np.sort(rng.choice(N, K, replace=False)) for _ in range(Q)]).astype(np.int32)[None]
        idx[0, 0, -2:] = -1
        q_t, idx_t = dev_bf16(qb), torch.from_numpy(idx).cuda()
        ref = host(C.sparse_attn_fp4(q_t, cache, idx_t))
        got = host(C.sparse_attn_fp4_noalloc(q_t, cache, idx_t))
        assert np.array_equal(got.view(np.uint32), ref.view(np.uint32)), (Q, H, K)
        for i in (0, Q - 1):
            err = max_rel_err_rows(got[0, i], o_attn(qb[0, i], okv, idx[0, i], scale))
            assert err <= ATTN_TOL, (Q, i, err)
