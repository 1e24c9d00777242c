"""The C-ABI library loads, exports every call include/csa2.h declares, and rejects bad
arguments on the host before any HIP call (runs without a GPU)."""

import ctypes
import os
import re

import pytest

import fp4_compressed_sparse_kv_amd as C

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "csa2.h")

pytestmark = pytest.mark.skipif(not os.path.exists(C.LIB_PATH), reason="libcsa2.so not built")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?(?:int|void|char\s*\*|const char\s*\*)\s*\*?\s*(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_boundary_calls():
    names = _declared_functions()
    for n in ["kv_quant_fp4", "kv_dequant_fp4", "csa2_index_full", "csa2_index_reindex", "csa2_topk",
              "csa2_sparse_attn_fp4", "csa2_plan_create", "csa2_plan_run_decode", "csa2_prefill_full",
              "csa2_last_error", "kv_quant_mxfp4", "kv_dequant_mxfp4", "csa2_sparse_attn_mxfp4", "csa2_kv_project"]:
        assert n in names, n


def test_library_exports_every_declared_symbol():
    h = ctypes.CDLL(C.LIB_PATH)
    missing = [n for n in _declared_functions() if not hasattr(h, n)]
    assert not missing, missing
    assert C.lib().csa2_version() >= 100


def _err(rc, code, fragment):
    assert rc == code, (rc, C.lib().csa2_last_error())
    assert fragment in C.lib().csa2_last_error().decode()


def test_quant_validation():
    L = C.lib()
    p = ctypes.c_void_p(4096)
    _err(L.kv_quant_fp4(p, 10, 24, 24, p, 12, p, 2, None), 1, "multiple of 16")
    _err(L.kv_quant_fp4(p, 10, 32, 16, p, 16, p, 2, None), 1, "stride")
    _err(L.kv_quant_fp4(None, 10, 32, 32, p, 16, p, 2, None), 1, "null")
    _err(L.kv_quant_fp4(ctypes.c_void_p(4098), 10, 32, 32, p, 16, p, 2, None), 1, "aligned")
    _err(L.kv_quant_fp4(p, -1, 32, 32, p, 16, p, 2, None), 1, "rows")
    assert L.kv_quant_fp4(None, 0, 32, 32, None, 16, None, 2, None) == 0          # empty: no-op
    _err(L.kv_dequant_fp4(p, 4, p, 2, 10, 32, p, 32, None), 1, "code row stride")


def test_mxfp4_validation():
    L = C.lib()
    p = ctypes.c_void_p(4096)
    _err(L.kv_quant_mxfp4(p, 10, 48, 48, p, 24, p, 2, None), 1, "multiple of 32")
    _err(L.kv_quant_mxfp4(p, 10, 64, 64, ctypes.c_void_p(4104), 32, p, 2, None), 1, "16-byte aligned")
    _err(L.kv_quant_mxfp4(p, 10, 64, 64, p, 32, p, 1, None), 1, "scale row stride")
    assert L.kv_quant_mxfp4(None, 0, 64, 64, None, 32, None, 2, None) == 0
    _err(L.kv_dequant_mxfp4(p, 16, p, 2, 10, 64, p, 64, None), 1, "code row stride")
    _err(L.csa2_sparse_attn_mxfp4(p, 1, 1, 8, 128, p, ctypes.c_void_p(4098), p, p, 10, 128, 8, p, 4, 0.1, p, p,
                                  1 << 20, None), 1, "4-byte aligned")
    _err(L.csa2_sparse_attn_mxfp4(p, 1, 1, 8, 128, p, p, p, p, 10, 128, 2, p, 4, 0.1, p, p, 1 << 20, None),
         1, "stride")
    params = C.PlanParams(K=16, P=64, H=8, d=128, d_idx=64, q_idx_dtype=1, k_idx_dtype=2, softmax_scale=0.0,
                          kv_format=7)
    arr = (ctypes.c_int32 * 1)(C.FULL)
    h = ctypes.c_void_p(None)
    _err(L.csa2_plan_create(arr, 1, ctypes.byref(params), ctypes.byref(h)), 1, "kv_format")


def test_kv_project_validation():
    L = C.lib()
    p = ctypes.c_void_p(4096)
    _err(L.csa2_kv_project(p, 10, 96, 96, p, 96, 0, p, 128, p, 16, None, 0, None), 1, "multiple of 64")
    _err(L.csa2_kv_project(p, 10, 128, 128, p, 128, 3, p, 128, p, 16, None, 0, None), 1, "kv_format")
    _err(L.csa2_kv_project(p, 10, 128, 128, p, 128, 0, p, 64, p, 16, None, 0, None), 1, "code row stride")
    _err(L.csa2_kv_project(p, 10, 128, 128, p, 128, 1, ctypes.c_void_p(4104), 128, p, 8, None, 0, None), 1,
         "16-byte aligned")
    _err(L.csa2_kv_project(None, 10, 128, 128, p, 128, 0, p, 128, p, 16, None, 0, None), 1, "null")
    assert L.csa2_kv_project(None, 0, 128, 128, None, 128, 0, None, 128, None, 16, None, 0, None) == 0


def test_index_validation():
    L = C.lib()
    p = ctypes.c_void_p(4096)
    _err(L.csa2_index_full(p, 2, p, 2, 1, 1, 100, 64, None, p, None), 2, "query dtype")
    _err(L.csa2_index_full(p, 1, p, 7, 1, 1, 100, 64, None, p, None), 2, "key dtype")
    _err(L.csa2_index_full(p, 1, p, 2, 1, 1, 100, 48, None, p, None), 1, "d_idx")
    _err(L.csa2_index_full(p, 1, ctypes.c_void_p(4100), 2, 1, 1, 100, 64, None, p, None), 1, "16-byte")
    _err(L.csa2_index_full(p, 1, p, 2, 300, 300, 100, 64, None, p, None), 1, "65535")
    assert L.csa2_index_full(p, 1, p, 2, 0, 1, 100, 64, None, p, None) == 0
    _err(L.csa2_index_reindex(p, 1, p, 2, 1, 100, 64, None, 8, p, None), 1, "null")


def test_topk_and_attn_validation():
    L = C.lib()
    p = ctypes.c_void_p(4096)
    _err(L.csa2_topk(p, 1, 100, 100, None, 0, p, None, p, 1 << 20, None), 1, "K >= 1")
    _err(L.csa2_topk(p, 1, 100, 50, None, 5, p, None, p, 1 << 20, None), 1, "score_stride")
    _err(L.csa2_topk(None, 1, 100, 100, None, 5, p, None, p, 1 << 20, None), 1, "null")
    _err(L.csa2_sparse_attn_fp4(p, 1, 1, 17, 128, p, p, p, p, 10, 128, 16, p, 4, 0.1, p, p, 1 << 20, None),
         1, "H must")
    _err(L.csa2_sparse_attn_fp4(p, 1, 1, 8, 64, p, p, p, p, 10, 128, 16, p, 4, 0.1, p, p, 1 << 20, None),
         1, "head dim")
    _err(L.csa2_sparse_attn_fp4(p, 1, 1, 8, 128, p, p, p, p, 10, 32, 16, p, 4, 0.1, p, p, 1 << 20, None),
         1, "stride")
    _err(L.csa2_sparse_attn_fp4(p, 1, 1, 8, 128, p, p, p, p, 10, 128, 16, p, 4, -1.0, p, p, 1 << 20, None),
         1, "softmax_scale")
    sz = ctypes.c_size_t(0)
    _err(L.csa2_sparse_attn_workspace_bytes(1, 1, 0, 128, 4, ctypes.byref(sz)), 1, "bad sizes")
    # the allocation-free variant checks the same arguments on the host before any HIP call
    _err(L.csa2_sparse_attn_fp4_noalloc(p, 1, 1, 17, 128, p, p, p, p, 10, 128, 16, p, 4, 0.1, p, None), 1, "H must")
    _err(L.csa2_sparse_attn_fp4_noalloc(p, 1, 1, 8, 128, p, p, p, p, 10, 128, 16, None, 4, 0.1, p, None), 1, "null")
    _err(L.csa2_sparse_attn_fp4_noalloc(p, 1, 1, 8, 128, p, p, p, p, 10, 128, 16, p, 4, float("nan"), p, None),
         1, "softmax_scale")
    assert L.csa2_sparse_attn_fp4_noalloc(p, 0, 1, 8, 128, p, p, p, p, 10, 128, 16, p, 4, 0.0, p, None) == 0


def _plan(modes, **kw):
    prm = dict(K=16, P=64, H=8, d=128, d_idx=64, q_idx_dtype=1, k_idx_dtype=2, softmax_scale=0.0)
    prm.update(kw)
    arr = (ctypes.c_int32 * len(modes))(*modes)
    params = C.PlanParams(**prm)
    h = ctypes.c_void_p(None)
    rc = C.lib().csa2_plan_create(arr, len(modes), ctypes.byref(params), ctypes.byref(h))
    return rc, h


def test_plan_rules():
    rc, h = _plan([C.FULL, C.REINDEX, C.REUSE, C.REUSE])
    assert rc == 0 and h.value
    C.lib().csa2_plan_destroy(h)
    rc, _ = _plan([C.REUSE, C.FULL])
    _err(rc, 3, "first layer must be Full")
    rc, _ = _plan([C.REINDEX])
    _err(rc, 3, "first layer must be Full")
    rc, _ = _plan([C.FULL, C.REINDEX], K=128, P=64)
    _err(rc, 3, "P >= K")
    rc, _ = _plan([C.FULL, 9])
    _err(rc, 3, "unknown mode")
    rc, _ = _plan([C.FULL], H=0)
    _err(rc, 1, "H must")
    rc, _ = _plan([C.FULL], k_idx_dtype=5)
    _err(rc, 2, "key dtype")
    rc, h = _plan([C.FULL, C.REUSE], P=0)          # no Reindex: P unused
    assert rc == 0
    C.lib().csa2_plan_destroy(h)


def test_python_binding_rejects_cpu_tensors():
    import torch
    with pytest.raises(C.Csa2Error):
        C.kv_quant_fp4(torch.zeros(4, 32, dtype=torch.bfloat16))
