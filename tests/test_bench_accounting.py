"""CPU checks of the benchmark's accounting: the algorithmic bytes of a decode step follow the
per-layer byte counts of the method (indexer query and keys, pool and top-K positions, gathered
FP4 K/V rows at C/2 + C/16 bytes per C channels, query and output), worked out by hand below, and
a multi-GPU request is refused."""

import json
import os
import subprocess
import sys

import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def _attn(K, H, d):
    # positions (4K) + bf16 query (2Hd) + K gathered K/V records (2 * (d/2 + d/16) bytes) + fp32 output (4Hd)
    return 4 * K + 2 * H * d + K * 2 * (d // 2 + d // 16) + 4 * H * d


def test_kv_record_is_144_bytes_per_token():
    assert 2 * (128 // 2 + 128 // 16) == 144


def test_stack_b32_n262144_bytes():
    cfg = synth.WORKLOADS["stack_b32_n262144"]
    A = _attn(2048, 16, 128)
    assert A == 315_392
    full = 2 * 64 + 262_144 * 64 + 4 * 8192 + 4 * 2048 + A      # bf16 q_I, E4M3 keys, pool, top-K
    reindex = 2 * 64 + 4 * 8192 + 8192 * 64 + 4 * 2048 + A    # pool in, pool keys gathered
    per_seq = full + reindex + 2 * A
    assert per_seq == 18_645_248
    step, full_sel = bench.alg_bytes(cfg)
    assert step == 32 * per_seq == 596_647_936
    assert full_sel == 32 * (full - A) == 538_185_728


def test_full_b64_n131072_bytes():
    step, full_sel = bench.alg_bytes(synth.WORKLOADS["full_b64_n131072"])
    per_seq = 2 * 64 + 131_072 * 64 + 4 * 2048 + _attn(2048, 16, 128)   # no pool without a Reindex layer
    assert step == 64 * per_seq == 557_588_480
    assert full_sel == 64 * (per_seq - _attn(2048, 16, 128))


def test_stack_b4_n1m_decode_bytes():
    step, _ = bench.alg_bytes(synth.WORKLOADS["stack_b4_n1m"])
    A = _attn(2048, 16, 128)
    per_seq = (2 * 64 + 1_048_576 * 64 + 4 * 8192 + 4 * 2048 + A) + (2 * 64 + 4 * 8192 + 8192 * 64 + 4 * 2048 + A) + 2 * A
    assert step == 4 * per_seq == 275_907_584


def test_quantize_workload_bytes():
    cfg = synth.WORKLOADS["quant_1m_x512"]
    T, C = cfg["T"], cfg["C"]
    assert T * C * 2 + T * (C // 2 + C // 16) == 1_375_731_712        # bf16 rows + 256 + 32 B/token


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU" in msg["error"]
