#!/usr/bin/env python3
"""Benchmark of one decode step of the CSA2 layer stack over an FP4 E2M1 KV cache on one MI355X.

Default workload: stack_b32_n262144 - layers Full, Reindex, Reuse, Reuse; 32
sequences x 262,144 positions; 16 query heads of dim 128 on one shared FP4 KV
head (E4M3 scale per 16 channels); indexer dim 64 with E4M3 keys and bf16
queries; pool P = 8192; top-K = 2048. One step = the whole stack for all 32
sequences (one query each), inputs resident in HBM.

Prints ONE JSON line: queries/s, ms per step, algorithmic HBM GB/s of the step,
a roofline entry for the dominant kernel (the Full layer's fused scan + select,
timed with HIP events on its own stream inside this process) and the CPU
oracle timed on a bounded sample of the same workload (cpu_baseline).

  python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu]
  python bench.py --copy-calibration   # also runs a known-size copy kernel (for PMC scaling)
  python bench.py --workload stack_b4_n1m --prefill --steps 3 --warmup 1   # the prefill chunk
  python bench.py --workload quant_1m_x512 --steps 20                       # kv_quant_fp4 / dequant
  python bench.py --workload kvproj_t16384_d4096 --steps 50                 # KV write path (projection + FP4)
  python bench.py --kv mxfp4 ...                                            # MXFP4 cache (E8M0 per 32 channels)
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode queries/s per CSA2 layer stack + achieved HBM GB/s (% of peak)"
# HBM traffic per launch from committed rocprofv3 PMC passes (profiles/traffic_<kernel>_<workload>.json),
# each tied to a hash of the sources its kernel is built from and ignored once they change.
TRAFFIC_KERNELS = {
    "full_select": ["select.hip", "dot.hpp", "device.hpp", "attn_core.hpp"],
    "quant": ["quant.hip", "fp4q.hpp", "device.hpp"],
    "quant_mx": ["quant.hip", "fp4q.hpp", "device.hpp"],
    "kv_project": ["project.hip", "fp4q.hpp", "device.hpp"],
    "kv_project_mx": ["project.hip", "fp4q.hpp", "device.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def alg_bytes(cfg, kv="fp4_e4m3", swa=0):
    """Algorithmic bytes of one step (per sequence sums x B) and of the Full selection kernel.

    Full    = 2*d_I + N*d_I*b_k + 4P (when a Reindex follows) + 4K + A
    Reindex = 2*d_I + 4P + P*d_I*b_k + 4K + A
    Reuse   = A,  A = 4K + 2*H*d + K*2*(d/2 + d/g) + 4*H*d
    with g = 16 channels per scale (E4M3 scales) or 32 (MXFP4); a sliding window of W bf16 rows
    per layer adds 2*W*d*2 (its K and V rows) to A.
    """
    B, N, K, H, d, dI = cfg["B"], cfg["N"], cfg["K"], cfg["H"], cfg["d"], cfg["d_idx"]
    P = cfg.get("P") or 0
    bk = {"e4m3": 1, "bf16": 2, "f32": 4}[cfg["k_idx_dtype"]]
    bq = {"bf16": 2, "f32": 4}[cfg["q_idx_dtype"]]
    modes = list(cfg["modes"])
    has_re = "reindex" in modes
    g = 32 if kv == "mxfp4" else 16
    A = 4 * K + 2 * H * d + K * 2 * (d // 2 + d // g) + 4 * H * d + 2 * swa * d * 2
    per_seq = 0
    full_sel = 0
    first_full = True
    for m in modes:
        if m == "full":
            sel = bq * dI + N * dI * bk + (4 * P if (has_re and first_full) else 0) + 4 * K
            if first_full:
                full_sel = sel
            first_full = False
            per_seq += sel + A
        elif m == "reindex":
            per_seq += bq * dI + 4 * P + P * dI * bk + 4 * K + A
        else:
            per_seq += A
    return B * per_seq, B * full_sel


def kernel_hash(kernel="full_select"):
    h = hashlib.sha256()
    for f in TRAFFIC_KERNELS[kernel]:
        with open(os.path.join(ROOT, "fp4_compressed_sparse_kv_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed PMC runs, or None when
    there are none or they were taken on other kernel sources."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        t = json.load(fh)
    if t.get("kernel_hash") != kernel_hash(kernel) or t.get("workload") != workload:
        return None
    return t.get("traffic_bytes_per_launch")


def copy_calibration(dev):
    """A known-size copy kernel for scaling the PMC byte counters: reads and writes 1 GiB."""
    import torch
    x = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    y = torch.empty_like(x)
    torch.add(x, 0.0, out=y)
    torch.cuda.synchronize()
    del x, y


def build_inputs(cfg, dev, query_set=0, kv="fp4_e4m3", swa=0):
    import numpy as np
    import torch

    import fp4_compressed_sparse_kv_amd as C
    import synth

    B, N, L = cfg["B"], cfg["N"], len(cfg["modes"])

    def bf(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)

    def key_t(a, dt):
        t = torch.from_numpy(np.ascontiguousarray(a))
        if dt == "e4m3":
            return t.to(dev).view(torch.float8_e4m3fn)
        if dt == "bf16":
            return t.view(torch.int16).to(dev).view(torch.bfloat16)
        return t.to(dev)

    dI = cfg["d_idx"]
    kdt = {"e4m3": torch.uint8, "bf16": torch.int16, "f32": torch.float32}[cfg["k_idx_dtype"]]
    kidx = torch.empty(B, N, dI, dtype=kdt, device=dev)
    cache = C.KVCache(B, N, device=dev, kv_format=kv)
    for b in range(B):
        kb, vb = synth.kv_bf16(cfg, b)
        cache.fill(bf(kb), bf(vb), row0=b * N)
        ki = synth.k_idx(cfg, b)
        kidx[b].copy_(torch.from_numpy(np.ascontiguousarray(ki).view(
            {"e4m3": np.uint8, "bf16": np.int16, "f32": np.float32}[cfg["k_idx_dtype"]])))
    if cfg["k_idx_dtype"] == "e4m3":
        cache.k_idx = kidx.view(torch.float8_e4m3fn)
    elif cfg["k_idx_dtype"] == "bf16":
        cache.k_idx = kidx.view(torch.bfloat16)
    else:
        cache.k_idx = kidx
    layers = []
    for li in range(L):
        ql = query_set * L + li                 # set 0 is the workload's own queries (the parity tests' set)
        q = np.stack([synth.q_bf16(cfg, ql, b)[0] for b in range(B)])
        qi = np.stack([synth.q_idx(cfg, ql, b)[0] for b in range(B)])
        layers.append(dict(q=bf(q), q_idx=key_t(qi, cfg["q_idx_dtype"]),
                           out=torch.empty(B, cfg["H"], cfg["d"], dtype=torch.float32, device=dev),
                           idx_out=torch.empty(B, cfg["K"], dtype=torch.int32, device=dev)))
        if swa:
            wk, wv = synth.window_kv(cfg, ql, swa)
            layers[-1]["win_k"], layers[-1]["win_v"] = bf(wk), bf(wv)
    if cfg.get("P") and "reindex" in cfg["modes"]:
        layers[0]["pool_out"] = torch.empty(B, cfg["P"], dtype=torch.int32, device=dev)
    torch.cuda.synchronize()
    return cache, layers


def query_sets(cfg, dev, layers, nsets):
    """nsets sets of per-layer queries (set 0 = `layers`), each another seeded draw of the same
    distribution, sharing the output buffers of `layers`. Timed steps rotate through them so that
    consecutive steps select different positions and the gathers are not served from caches warmed
    by the previous step with the same queries."""
    import numpy as np

    import synth

    B, L = cfg["B"], len(cfg["modes"])
    sets = [layers]
    for qs in range(1, nsets):
        cur = []
        for li in range(L):
            ql = qs * L + li
            q = np.stack([synth.q_bf16(cfg, ql, b)[0] for b in range(B)])
            qi = np.stack([synth.q_idx(cfg, ql, b)[0] for b in range(B)])
            d = dict(layers[li])
            d["q"] = _to_dev_bf16(q, dev)
            d["q_idx"] = _to_dev_key(qi, cfg["q_idx_dtype"], dev)
            if "win_k" in d:
                wk, wv = synth.window_kv(cfg, ql, d["win_k"].shape[1])
                d["win_k"], d["win_v"] = _to_dev_bf16(wk, dev), _to_dev_bf16(wv, dev)
            cur.append(d)
        sets.append(cur)
    return sets


def _to_dev_bf16(bits, dev):
    import numpy as np
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(dev)


def _to_dev_key(a, dt, dev):
    import numpy as np
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dt == "e4m3":
        return t.to(dev).view(torch.float8_e4m3fn)
    if dt == "bf16":
        return t.view(torch.int16).to(dev).view(torch.bfloat16)
    return t.to(dev)


def host_cores():
    """Host threads this process may run on (its CPU affinity)."""
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, budget_s, kv="fp4_e4m3", swa=0):
    """The oracle, as it stands, on whole sequences of the same workload until ~budget_s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import plan as OP

    modes = list(cfg["modes"])
    scale = float(np.float32(1 / math.sqrt(cfg["d"])))
    done, spent = 0, 0.0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        for b in range(cfg["B"]):
            kb, vb = synth.kv_bf16(cfg, b)                           # untimed: input generation
            cache = dict(k_bf16=kb, v_bf16=vb, k_idx=synth.k_idx(cfg, b), k_idx_dtype=cfg["k_idx_dtype"], format=kv)
            layers = [dict(q=synth.q_bf16(cfg, li, b)[0], q_idx=synth.q_idx(cfg, li, b)[0],
                           q_idx_dtype=cfg["q_idx_dtype"]) for li in range(len(modes))]
            if swa:
                for li, L in enumerate(layers):
                    wk, wv = synth.window_kv(cfg, li, swa)
                    L["win_k"], L["win_v"] = wk[b], wv[b]
            t0 = time.perf_counter()
            OP.run_decode(modes, cache, layers, cfg["K"], cfg.get("P"), softmax_scale=scale)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    return {"value": done / spent, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {cfg['B']} sequences, one decode step of the whole stack each "
                      f"(N={cfg['N']}), {spent:.1f} s with BLAS on {cores} host threads (the process's CPU "
                      f"affinity); KV rows quantized by the oracle only where attention reads them"}


def build_quant_input(cfg, dev):
    """The quantize workload's T x C bf16 rows on the device, block by block from the seeded generator."""
    import numpy as np
    import torch

    import synth

    T, Cc, rb = cfg["T"], cfg["C"], cfg["row_block"]
    x = torch.empty(T, Cc, dtype=torch.bfloat16, device=dev)
    for blk in range(T // rb):
        xb = synth.quant_rows(cfg, blk)
        x[blk * rb:(blk + 1) * rb].copy_(torch.from_numpy(xb.view(np.int16)).view(torch.bfloat16))
    torch.cuda.synchronize()
    return x


def build_proj_input(cfg, dev):
    """The projection workload's hidden state [T][D] and transposed weights [C][D] on the device (bf16)."""
    import numpy as np
    import torch

    import synth

    T, D, rb = cfg["T"], cfg["D"], cfg["row_block"]
    h = torch.empty(T, D, dtype=torch.bfloat16, device=dev)
    for blk in range(T // rb):
        h[blk * rb:(blk + 1) * rb].copy_(torch.from_numpy(synth.proj_hidden(cfg, blk).view(np.int16)).view(torch.bfloat16))
    wt = torch.from_numpy(synth.proj_weights_t(cfg).view(np.int16)).view(torch.bfloat16).to(dev)
    torch.cuda.synchronize()
    return h, wt


def run_proj(args, cfg, dev):
    """The KV write path: C = H W (bf16, matrix cores) rounded to bf16 and quantized to FP4 in one kernel,
    T tokens x D hidden into the 256 channels of one KV head; the oracle on a bounded sample of rows."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import fp4_compressed_sparse_kv_amd as C
    import synth
    from oracle import mxfp4 as OM
    from oracle import project as PJ
    from oracle import quant as OQ

    T, D, Cc, rb = cfg["T"], cfg["D"], cfg["C"], cfg["row_block"]
    mx = args.kv == "mxfp4"
    t0 = time.perf_counter()
    h, wt = build_proj_input(cfg, dev)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    codes = torch.empty(T, 128, dtype=torch.uint8, device=dev)
    scales = torch.empty(T, 8 if mx else 16, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        C.kv_project(h, wt, args.kv, codes=codes, scales=scales)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        C.kv_project(h, wt, args.kv, codes=codes, scales=scales)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    if args.copy_calibration:
        copy_calibration(dev)
    nbytes = T * D * 2 + Cc * D * 2 + T * (Cc // 2 + Cc // (32 if mx else 16))
    flop = 2.0 * T * D * Cc
    gbs = nbytes / (ms * 1e-3) / 1e9
    tflops = flop / (ms * 1e-3) / 1e12
    out = {
        "metric": "KV write path tokens/s (CED projection GEMM + fused FP4 quantize) + HBM GB/s",
        "value": round(T / (ms * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 MFMA (fp32 accumulate)", "data": "synthetic",
        "config": {"workload": args.workload + (":mxfp4" if mx else ""), "T": T, "D": D, "C": Cc,
                   "kv": "mxfp4 (e2m1 + e8m0 per 32 ch)" if mx else "fp4_e2m1 + e4m3 scale per 16 ch"},
        "alg_bytes_per_call": nbytes, "flop_per_call": flop, "tflops": round(tflops, 1),
        "mfma_frac": round(tflops / 2500.0, 4),
        # the HBM floor (bytes / 8 TB/s) is above the matrix-core floor (FLOP / 2.5 PFLOP/s) at C = 256
        "roofline": {"bound": "hbm", "kernel": "k_kv_project", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("kv_project_mx" if mx else "kv_project", args.workload)},
    }
    if not args.no_cpu:
        done, spent = 0, 0.0
        cores = host_cores()
        wt_h = synth.proj_weights_t(cfg)
        quant = OM.quant_mxfp4 if mx else OQ.quant_fp4
        with threadpool_limits(limits=cores):
            for blk in range(T // rb):
                hb = synth.proj_hidden(cfg, blk)                 # untimed: input generation
                t1 = time.perf_counter()
                quant(PJ.round_to_bf16(PJ.project_exact(hb, wt_h.T)))
                spent += time.perf_counter() - t1
                done += rb
                if spent >= args.cpu_seconds:
                    break
        out["cpu_baseline"] = {"value": round(done / spent, 1), "unit": "tokens/s", "cores": cores, "kind": "oracle",
                               "sample": f"{done} of {T} tokens ({done // rb} blocks of {rb}), {spent:.1f} s with "
                                         f"BLAS on {cores} host threads"}
    print(json.dumps(out), flush=True)


def run_quant(args, cfg, dev):
    """The quantize workload: kv_quant_fp4 and kv_dequant_fp4 over T x C bf16 rows (each call timed alone,
    back to back, K calls between two events), with the oracle's quantizer on a bounded sample of rows."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_limits

    import fp4_compressed_sparse_kv_amd as C
    import synth
    from oracle import mxfp4 as OM
    from oracle import quant as OQ

    mx = args.kv == "mxfp4"
    T, Cc, rb = cfg["T"], cfg["C"], cfg["row_block"]
    blk = 32 if mx else 16
    quant, dequant = (C.kv_quant_mxfp4, C.kv_dequant_mxfp4) if mx else (C.kv_quant_fp4, C.kv_dequant_fp4)
    oquant = OM.quant_mxfp4 if mx else OQ.quant_fp4
    t0 = time.perf_counter()
    x = build_quant_input(cfg, dev)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    codes = torch.empty(T, Cc // 2, dtype=torch.uint8, device=dev)
    scales = torch.empty(T, Cc // blk, dtype=torch.uint8, device=dev)
    y = torch.empty_like(x)
    stream = torch.cuda.current_stream()

    def timed(fn):
        for _ in range(args.warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(args.steps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / args.steps

    q_ms = timed(lambda: quant(x, codes, scales))
    d_ms = timed(lambda: dequant(codes, scales, Cc, y))
    if args.copy_calibration:
        copy_calibration(dev)
    nbytes = T * Cc * 2 + T * (Cc // 2 + Cc // blk)           # bf16 rows + codes + scales, each direction
    groups = T * Cc // blk
    s_zero = int((scales == 0).sum().item())
    s_sat = int((scales == 0x7E).sum().item()) if not mx else None
    out = {
        "metric": ("kv_quant_mxfp4 HBM GB/s (bf16 rows in, FP4 codes + E8M0 scales out)" if mx else
                   "kv_quant_fp4 HBM GB/s (bf16 rows in, FP4 codes + E4M3 scales out)"),
        "value": round(nbytes / (q_ms * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(q_ms, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32 compares / u8", "data": "synthetic",
        "config": {"workload": args.workload + (":mxfp4" if mx else ""), "T": T, "C": Cc,
                   "kv": "mxfp4 (e2m1 + e8m0 per 32 ch)" if mx else "fp4_e2m1 + e4m3 scale per 16 ch"},
        "rows_per_s": round(T / (q_ms * 1e-3), 1),
        "dequant_ms": round(d_ms, 5), "dequant_gbs": round(nbytes / (d_ms * 1e-3) / 1e9, 1),
        "alg_bytes_per_call": nbytes, "groups": groups, "groups_scale_zero": s_zero, "groups_scale_448": s_sat,
        "roofline": {"bound": "hbm", "kernel": "k_quant_mx" if mx else "k_quant",
                     "achieved": round(nbytes / (q_ms * 1e-3) / 1e9, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(nbytes / (q_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("quant_mx" if mx else "quant", args.workload)},
    }
    if not args.no_cpu:
        done, spent = 0, 0.0
        cores = host_cores()
        with threadpool_limits(limits=cores):
            for blk in range(T // rb):
                xb = synth.quant_rows(cfg, blk)                   # untimed: input generation
                t1 = time.perf_counter()
                oquant(xb)
                spent += time.perf_counter() - t1
                done += rb
                if spent >= args.cpu_seconds:
                    break
        out["cpu_baseline"] = {"value": round(done / spent, 1), "unit": "rows/s", "cores": cores, "kind": "oracle",
                               "sample": f"{done} of {T} rows ({done // rb} blocks of {rb}), {spent:.1f} s with "
                                         f"BLAS on {cores} host threads (numpy's elementwise work runs on one)"}
    print(json.dumps(out), flush=True)


def run_prefill(args, cfg, dev):
    """Full-layer prefill of the workload's chunk: prefill_Q queries per sequence at the last
    positions of the context (causal), through the matrix-core indexer, exact top-K and attention."""
    import numpy as np
    import torch

    import fp4_compressed_sparse_kv_amd as C
    import synth

    B, N, Q, K = cfg["B"], cfg["N"], cfg["prefill_Q"], cfg["K"]
    t0 = time.perf_counter()
    cache, _ = build_inputs(cfg, dev)
    qi = np.stack([synth.prefill_q_idx(cfg, b, Q) for b in range(B)])
    qb = np.stack([synth.prefill_q_bf16(cfg, b, Q) for b in range(B)])
    qi_t = torch.from_numpy(np.ascontiguousarray(qi).view(np.int16)).view(torch.bfloat16).to(dev)
    qb_t = torch.from_numpy(np.ascontiguousarray(qb).view(np.int16)).view(torch.bfloat16).to(dev)
    q_pos = torch.arange(N - Q, N, dtype=torch.int64, device=dev).repeat(B, 1).contiguous()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    plan = C.Plan(("full",), K=K, P=0, H=cfg["H"], d=cfg["d"], d_idx=cfg["d_idx"],
                  q_idx_dtype=cfg["q_idx_dtype"], k_idx_dtype=cfg["k_idx_dtype"])
    idx = torch.empty(B, Q, K, dtype=torch.int32, device=dev)
    out = torch.empty(B, Q, cfg["H"], cfg["d"], dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.prefill_full(cache, qi_t, qb_t, q_pos, idx_out=idx, out=out, check=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.prefill_full(cache, qi_t, qb_t, q_pos, idx_out=idx, out=out, check=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    status = plan.prefill_status(cache, Q)
    causal = float((q_pos + 1).sum().item())
    flop = 2.0 * cfg["d_idx"] * causal                  # indexer dot products, causal positions only
    res = {
        "metric": "Full-layer prefill queries/s (indexer + exact top-K + FP4 sparse attention)",
        "value": round(B * Q / (ms * 1e-3), 1) if status == 0 else None, "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16 MFMA (candidates) / f64 (exact scores) / f32", "data": "synthetic",
        "config": {"workload": args.workload + ":prefill", "B": B, "N": N, "Q": Q, "K": K, "H": cfg["H"],
                   "d_idx": cfg["d_idx"], "indexer_keys": cfg["k_idx_dtype"], "indexer_query": cfg["q_idx_dtype"]},
        "indexer_tflop": round(flop / 1e12, 3),
        "indexer_mfma_frac_of_whole_prefill": round(flop / (ms * 1e-3) / 2.5e15, 4),
        "status_word": status,
        # conservative: the indexer's FLOP over the whole prefill time (all kernels), dense bf16 peak
        "roofline": {"bound": "mfma", "kernel": "k_pf_tiles (indexer candidates), whole-prefill time",
                     "achieved": round(flop / (ms * 1e-3) / 1e12, 1), "peak": 2500.0, "unit": "TFLOP/s",
                     "frac": round(flop / (ms * 1e-3) / 2.5e15, 4), "traffic": None},
    }
    if not args.no_cpu:
        res["cpu_baseline"] = prefill_cpu_baseline(cfg, args.cpu_seconds)
    print(json.dumps(res), flush=True)


def run_prefill_plan(args, cfg, dev):
    """The workload's prefill chunk through every layer of its plan (csa2_plan_run_prefill): per query a
    causal Full layer with its own pool, Reindex over that pool, Reuse, and attention in every layer."""
    import numpy as np
    import torch

    import fp4_compressed_sparse_kv_amd as C
    import synth

    B, N, Q, K, P = cfg["B"], cfg["N"], cfg["prefill_Q"], cfg["K"], cfg["P"]
    modes = list(cfg["modes"])
    t0 = time.perf_counter()
    cache, _ = build_inputs(cfg, dev)
    layers = []
    for li in range(len(modes)):
        qi = np.stack([synth.q_idx(cfg, 100 + li, b, Q=Q) for b in range(B)])
        qb = np.stack([synth.q_bf16(cfg, 100 + li, b, Q=Q) for b in range(B)])
        layers.append(dict(q=_to_dev_bf16(qb, dev), q_idx=_to_dev_key(qi, cfg["q_idx_dtype"], dev),
                           out=torch.empty(B, Q, cfg["H"], cfg["d"], dtype=torch.float32, device=dev)))
    q_pos = torch.arange(N - Q, N, dtype=torch.int64, device=dev).repeat(B, 1).contiguous()
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    plan = C.Plan(modes, K=K, P=P, H=cfg["H"], d=cfg["d"], d_idx=cfg["d_idx"], q_idx_dtype=cfg["q_idx_dtype"],
                  k_idx_dtype=cfg["k_idx_dtype"])
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        plan.run_prefill(cache, layers, q_pos, check=False)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        plan.run_prefill(cache, layers, q_pos, check=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    ws = C.workspace(0, dev, ("plan_prefill", id(plan)))
    status = C.status_word(ws)
    res = {
        "metric": "prefill queries/s through the CSA2 layer stack (per-query pools, Reindex, Reuse, attention)",
        "value": round(B * Q / (ms * 1e-3), 1) if status == 0 else None, "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16 MFMA (candidates) / f64 (exact scores) / f32",
        "data": "synthetic",
        "config": {"workload": args.workload + ":prefill_plan", "B": B, "N": N, "Q": Q, "K": K, "P": P,
                   "modes": modes},
        "status_word": status,
    }
    causal = float((q_pos + 1).sum().item())
    flop = 2.0 * cfg["d_idx"] * causal * modes.count("full")      # the Full layers' indexer dot products
    res["indexer_tflop"] = round(flop / 1e12, 3)
    # conservative: the Full layers' indexer FLOP over the whole prefill time (all layers), dense bf16 peak
    res["roofline"] = {"bound": "mfma", "kernel": "k_pf_tiles (indexer candidates), whole-plan prefill time",
                       "achieved": round(flop / (ms * 1e-3) / 1e12, 1), "peak": 2500.0, "unit": "TFLOP/s",
                       "frac": round(flop / (ms * 1e-3) / 2.5e15, 4), "traffic": None}
    if not args.no_cpu:
        from threadpoolctl import threadpool_limits

        from oracle import plan as OP
        scale = float(np.float32(1 / math.sqrt(cfg["d"])))
        kb, vb = synth.kv_bf16(cfg, 0)                               # untimed: input generation
        oc = dict(k_bf16=kb, v_bf16=vb, k_idx=synth.k_idx(cfg, 0), k_idx_dtype=cfg["k_idx_dtype"])
        ol = [dict(q=synth.q_bf16(cfg, 100 + li, 0, Q=Q), q_idx=synth.q_idx(cfg, 100 + li, 0, Q=Q),
                   q_idx_dtype=cfg["q_idx_dtype"]) for li in range(len(modes))]
        qp = np.arange(N - Q, N)
        cores = host_cores()
        done, spent = 0, 0.0
        with threadpool_limits(limits=cores):
            for i in range(0, Q, 97):
                t1 = time.perf_counter()
                OP.run_prefill(modes, oc, ol, qp, K, P, softmax_scale=scale, queries=[i])
                spent += time.perf_counter() - t1
                done += 1
                if spent >= args.cpu_seconds:
                    break
        res["cpu_baseline"] = {"value": done / spent, "unit": "queries/s", "cores": cores, "kind": "oracle",
                               "sample": f"{done} of {Q} queries of sequence 0 (every 97th position) through all "
                                         f"{len(modes)} layers, N={N}, {spent:.1f} s with BLAS on {cores} host threads"}
    print(json.dumps(res), flush=True)


def prefill_cpu_baseline(cfg, budget_s):
    """The oracle on sampled prefill queries of sequence 0 (exact causal scores over the whole context,
    top-K, fp64 attention) until ~budget_s of CPU work."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    import synth
    from oracle import scores as OS
    from oracle.attention import sparse_attn as o_attn
    from oracle.topk import topk as o_topk

    N, Q, K = cfg["N"], cfg["prefill_Q"], cfg["K"]
    scale = float(np.float32(1 / math.sqrt(cfg["d"])))
    kb, vb = synth.kv_bf16(cfg, 0)                                   # untimed: input generation
    cache = dict(k_bf16=kb, v_bf16=vb, k_idx=synth.k_idx(cfg, 0), k_idx_dtype=cfg["k_idx_dtype"])
    qi = synth.prefill_q_idx(cfg, 0, Q)
    qb = synth.prefill_q_bf16(cfg, 0, Q)
    done, spent = 0, 0.0
    cores = host_cores()
    with threadpool_limits(limits=cores):
        for i in range(0, Q, 97):                                    # a spread of query positions
            t0 = time.perf_counter()
            s = OS.index_scores(qi[i], cfg["q_idx_dtype"], cache["k_idx"], cfg["k_idx_dtype"], q_pos=N - Q + i)
            idx, _ = o_topk(s, K)
            o_attn(qb[i], cache, idx, scale)
            spent += time.perf_counter() - t0
            done += 1
            if spent >= budget_s:
                break
    return {"value": done / spent, "unit": "queries/s", "cores": cores, "kind": "oracle",
            "sample": f"{done} of {Q} queries of sequence 0 (every 97th position), N={N}, {spent:.1f} s with BLAS "
                      f"on {cores} host threads; KV rows quantized by the oracle only where attention reads them"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=300)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first: a few hundred bring the GPU from idle clocks to steady state")
    ap.add_argument("--workload", default="stack_b32_n262144")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--kv", default="fp4_e4m3", choices=["fp4_e4m3", "mxfp4"],
                    help="main KV cache format: E4M3 scale per 16 channels, or MXFP4 (E8M0 per 32)")
    ap.add_argument("--swa", type=int, default=0,
                    help="decode: every layer also attends to a sliding window of this many bf16 rows")
    ap.add_argument("--query-sets", type=int, default=4,
                    help="decode: timed steps rotate through this many seeded query sets")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--prefill", action="store_true",
                    help="time the workload's Full-layer prefill chunk instead of the decode step")
    ap.add_argument("--prefill-plan", action="store_true",
                    help="time the workload's prefill chunk through every layer of its plan")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only: the decode stack shards by sequence "
                                   "(each GPU runs the same kernels on its own sequences) and no multi-GPU run "
                                   "is provided", "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import fp4_compressed_sparse_kv_amd as C
    import synth

    cfg = dict(synth.WORKLOADS[args.workload])
    if args.prefill or args.prefill_plan:
        if "prefill_Q" not in cfg:
            raise SystemExit(f"{args.workload} has no prefill chunk")
        torch.cuda.set_device(0)
        if args.prefill_plan:
            return run_prefill_plan(args, cfg, torch.device("cuda", 0))
        return run_prefill(args, cfg, torch.device("cuda", 0))
    if "D" in cfg:
        torch.cuda.set_device(0)
        return run_proj(args, cfg, torch.device("cuda", 0))
    if "T" in cfg:
        torch.cuda.set_device(0)
        return run_quant(args, cfg, torch.device("cuda", 0))
    if "modes" not in cfg:
        raise SystemExit(f"{args.workload} is not a decode workload")
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t0 = time.perf_counter()
    cache, layers = build_inputs(cfg, dev, kv=args.kv, swa=args.swa)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    plan = C.Plan(cfg["modes"], K=cfg["K"], P=cfg.get("P") or 0, H=cfg["H"], d=cfg["d"], d_idx=cfg["d_idx"],
                  q_idx_dtype=cfg["q_idx_dtype"], k_idx_dtype=cfg["k_idx_dtype"], kv_format=args.kv,
                  swa_window=args.swa)
    stream = torch.cuda.current_stream()
    sets = query_sets(cfg, dev, layers, args.query_sets)
    ws = plan.decode_workspace(cache)

    for i in range(args.warmup):
        plan.run_decode(cache, sets[i % len(sets)], ws=ws, check=False)
    torch.cuda.synchronize()

    # timed region: exactly K steps between two events, synchronized on both sides
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(args.steps):
        plan.run_decode(cache, sets[i % len(sets)], ws=ws, check=False)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / args.steps
    status = C.status_word(ws)
    log(f"step {ms * 1e3:.1f} us, status word {status}")

    # per-kernel durations over a second pass of up to 100 steps (events around each kernel, same stream)
    prof_steps = min(args.steps, 100)
    plan.profile_begin(prof_steps)
    for i in range(prof_steps):
        plan.run_decode(cache, sets[i % len(sets)], ws=ws, check=False)
    torch.cuda.synchronize()
    slot_ms, runs = plan.profile_read()
    plan.profile_begin(0)
    log("kernel slots (ms): " + ", ".join(f"{s:.4f}" for s in slot_ms))

    # cold-cache steps: a 1 GiB write between steps evicts L2 and MALL; each step timed alone
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    cold = []
    for i in range(min(args.steps, 10)):
        flush.fill_(1)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        plan.run_decode(cache, sets[i % len(sets)], ws=ws, check=False)
        b.record(stream)
        torch.cuda.synchronize()
        cold.append(a.elapsed_time(b))
    del flush
    status |= C.status_word(ws)

    # achievable reference: a device-to-device copy of 1 GiB (2 GiB moved)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst

    if args.copy_calibration:
        copy_calibration(dev)

    step_bytes, sel_bytes = alg_bytes(cfg, args.kv, args.swa)
    # the Full layer's attention runs inside its select when its own slot stays empty: that launch
    # then also reads the query, the selected KV rows and writes the output (its positions stay on chip)
    full_fused = len(slot_ms) > 1 and slot_ms[1] == 0.0
    if full_fused:
        H, d, K = cfg["H"], cfg["d"], cfg["K"]
        g = 32 if args.kv == "mxfp4" else 16
        sel_bytes += cfg["B"] * (2 * H * d + K * 2 * (d // 2 + d // g) + 4 * H * d)
    qps = cfg["B"] / (ms * 1e-3)
    sel_ms = slot_ms[0]
    achieved = sel_bytes / (sel_ms * 1e-3) / 1e9
    traffic = measured_traffic("full_select", args.workload)
    out = {
        "metric": METRIC,
        "value": round(qps, 1) if status == 0 else None,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f64/f32",
        "data": "synthetic",
        "config": {"workload": args.workload + (":mxfp4" if args.kv == "mxfp4" else "") +
                               (f":swa{args.swa}" if args.swa else ""), "B": cfg["B"], "swa_window": args.swa,
                   "N": cfg["N"], "modes": list(cfg["modes"]),
                   "H": cfg["H"], "d": cfg["d"], "d_idx": cfg["d_idx"], "K": cfg["K"], "P": cfg.get("P"),
                   "kv": "mxfp4 (e2m1 + e8m0 per 32 ch)" if args.kv == "mxfp4" else "fp4_e2m1 + e4m3 scale per 16 ch",
                   "indexer_keys": cfg["k_idx_dtype"],
                   "indexer_query": cfg["q_idx_dtype"]},
        "status_word": status,
        "query_sets": len(sets),
        "hbm_frac_basis": f"ms_per_step: timed steps rotate through {len(sets)} seeded query sets",
        "hbm_gbs_step": round(step_bytes / (ms * 1e-3) / 1e9, 1),
        "hbm_frac_step": round(step_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
        "alg_bytes_step": step_bytes,
        "cold_ms_per_step": round(sorted(cold)[len(cold) // 2], 5) if cold else None,
        "cold_ms_p10_p90": [round(float(np.percentile(cold, 10)), 5), round(float(np.percentile(cold, 90)), 5)] if cold else None,
        "achievable_copy_gbs": round(copy_gbs, 1),
        # per-kernel slots: 2l is layer l's select launch, 2l + 1 its attention launch (empty when fused)
        "kernel_ms": {"full_select": round(sel_ms, 5),
                      **{f"L{i // 2}_{cfg['modes'][i // 2]}_{'attn' if i % 2 else 'select'}": round(v, 5)
                         for i, v in enumerate(slot_ms) if i > 0 and v > 0 and i // 2 < len(cfg["modes"])}},
        "roofline": {"bound": "hbm", "kernel": "k_select<SrcScan> (Full layer: scan + pool/top-K select" +
                               (" + attention)" if full_fused else ")"),
                     "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "alg_bytes_per_launch": sel_bytes,
                     "traffic": traffic},
    }
    if not args.no_cpu:
        t0 = time.perf_counter()
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_seconds, args.kv, args.swa)
        log(f"cpu baseline in {time.perf_counter() - t0:.1f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
