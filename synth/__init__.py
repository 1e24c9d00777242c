"""Seeded synthetic inputs for the CSA2 workloads (shared by tests, bench and the oracle).

This module only draws random numbers and stores them in the input formats
(bf16 bit patterns, fp32, E4M3 bytes via torch's own casts). It holds none of
the method's arithmetic: no quantization, scoring, selection or attention.

Streams: numpy PCG64 seeded with SeedSequence([seed, workload_id, tensor_id,
index]) so that any one sequence (or row block) can be regenerated alone.

Workloads (one decode query per sequence and layer; context positions 0..N-1):
  full_n2048         1 Full layer, B=1, N=2048, KV 1 head K,V 128 channels from
                     bf16 N(0,1) with 1% of channels x20; 8 query heads d=128
                     bf16 N(0,1); indexer d=64 fp32 N(0,1) query and keys; K=128.
  quant_1m_x512      1,048,576 rows x 512 channels bf16, N(0,1) times a per-row
                     scale 10^U(-3,3).
  full_b64_n131072   1 Full layer, B=64, N=131,072, 16 heads d=128, indexer
                     d=64 with bf16 query and E4M3 keys, K=2048, 0.5% outliers.
  stack_b32_n262144  Full, Reindex, Reuse, Reuse; B=32, N=262,144, pool P=8192,
                     K=2048, other shapes as full_b64_n131072.
  stack_b4_n1m       the stack at B=4, N=1,048,576 plus a prefill chunk of the
                     last 4096 positions of each sequence through the Full
                     layer (causal), K=2048.
  kvproj_t16384_d4096  the KV write path of that prefill chunk: 4 x 4096 tokens
                     of encoder hidden state (D = 4096, bf16 N(0,1)) projected
                     by one decoder layer's KV weights (256 x 4096 bf16,
                     N(0, 1/D)) into K and V of the shared head.
"""

import numpy as np
import torch

WORKLOADS = {
    "full_n2048": dict(wid=0, B=1, N=2048, H=8, d=128, d_idx=64, K=128, P=None,
                       modes=("full",), q_idx_dtype="f32", k_idx_dtype="f32",
                       outlier_frac=0.01, seed=0),
    "quant_1m_x512": dict(wid=1, T=1048576, C=512, seed=0, row_block=4096),
    "full_b64_n131072": dict(wid=2, B=64, N=131072, H=16, d=128, d_idx=64, K=2048, P=None,
                             modes=("full",), q_idx_dtype="bf16", k_idx_dtype="e4m3",
                             outlier_frac=0.005, seed=0),
    "stack_b32_n262144": dict(wid=3, B=32, N=262144, H=16, d=128, d_idx=64, K=2048, P=8192,
                              modes=("full", "reindex", "reuse", "reuse"), q_idx_dtype="bf16",
                              k_idx_dtype="e4m3", outlier_frac=0.005, seed=0),
    "kvproj_t16384_d4096": dict(wid=5, T=16384, D=4096, C=256, seed=0, row_block=1024),
    "stack_b4_n1m": dict(wid=4, B=4, N=1048576, H=16, d=128, d_idx=64, K=2048, P=8192,
                         modes=("full", "reindex", "reuse", "reuse"), q_idx_dtype="bf16",
                         k_idx_dtype="e4m3", outlier_frac=0.005, seed=0, prefill_Q=4096),
}

# tensor ids for the substreams
_T_K, _T_V, _T_KOUT, _T_VOUT, _T_Q, _T_QIDX, _T_KIDX, _T_ROWS, _T_PQ, _T_PQIDX, _T_HID, _T_WKV, _T_WIN = range(13)


def rng(seed, wid, tensor, index=0):
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, wid, tensor, index])))


def to_bf16_bits(x_f32):
    """fp32 array -> bf16 bit patterns (uint16) via torch's round-to-nearest-even cast."""
    t = torch.from_numpy(np.ascontiguousarray(x_f32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def to_e4m3_bytes(x_f32):
    """fp32 array -> E4M3FN bytes via torch's cast (inputs kept inside +-448)."""
    x = np.clip(np.asarray(x_f32, dtype=np.float32), -448.0, 448.0)
    t = torch.from_numpy(np.ascontiguousarray(x))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def outlier_channels(cfg, tensor, C):
    """Channels scaled x20 for one KV tensor: max(1, round(frac*C)) of them, fixed across tokens."""
    n = max(1, int(round(cfg["outlier_frac"] * C)))
    g = rng(cfg["seed"], cfg["wid"], _T_KOUT if tensor == "k" else _T_VOUT)
    return np.sort(g.choice(C, size=n, replace=False))


def kv_bf16(cfg, b, n0=0, n1=None):
    """Main-KV rows of sequence b, positions [n0, n1): (K bits [n][d], V bits [n][d]).

    Values N(0,1) in fp32, outlier channels x20, then cast to bf16. Rows are
    drawn from the sequence's own stream, so any slice regenerates exactly.
    """
    N, d = cfg["N"], cfg["d"]
    n1 = N if n1 is None else n1
    out = []
    for tid, name in ((_T_K, "k"), (_T_V, "v")):
        g = rng(cfg["seed"], cfg["wid"], tid, b)
        if n0:
            g.standard_normal((n0, d), dtype=np.float32)     # advance the stream
        x = g.standard_normal((n1 - n0, d), dtype=np.float32)
        x[:, outlier_channels(cfg, name, d)] *= np.float32(20.0)
        out.append(to_bf16_bits(x))
    return out[0], out[1]


def q_bf16(cfg, layer, b, Q=1):
    """Attention query of sequence b for one layer: (Q, H, d) bf16 bits, N(0,1)."""
    g = rng(cfg["seed"], cfg["wid"], _T_Q, layer * 1_000_000 + b)
    return to_bf16_bits(g.standard_normal((Q, cfg["H"], cfg["d"]), dtype=np.float32))


def q_idx(cfg, layer, b, Q=1):
    """Indexer query of sequence b for one layer: (Q, d_idx) fp32 or bf16 bits, N(0,1)."""
    g = rng(cfg["seed"], cfg["wid"], _T_QIDX, layer * 1_000_000 + b)
    x = g.standard_normal((Q, cfg["d_idx"]), dtype=np.float32)
    return x if cfg["q_idx_dtype"] == "f32" else to_bf16_bits(x)


def k_idx(cfg, b, n0=0, n1=None):
    """Indexer keys of sequence b, positions [n0, n1): fp32 or E4M3 bytes, from N(0,1)."""
    N, di = cfg["N"], cfg["d_idx"]
    n1 = N if n1 is None else n1
    g = rng(cfg["seed"], cfg["wid"], _T_KIDX, b)
    if n0:
        g.standard_normal((n0, di), dtype=np.float32)
    x = g.standard_normal((n1 - n0, di), dtype=np.float32)
    if cfg["k_idx_dtype"] == "f32":
        return x
    if cfg["k_idx_dtype"] == "bf16":
        return to_bf16_bits(x)
    return to_e4m3_bytes(x)


def prefill_q_bf16(cfg, b, Q):
    g = rng(cfg["seed"], cfg["wid"], _T_PQ, b)
    return to_bf16_bits(g.standard_normal((Q, cfg["H"], cfg["d"]), dtype=np.float32))


def prefill_q_idx(cfg, b, Q):
    g = rng(cfg["seed"], cfg["wid"], _T_PQIDX, b)
    x = g.standard_normal((Q, cfg["d_idx"]), dtype=np.float32)
    return x if cfg["q_idx_dtype"] == "f32" else to_bf16_bits(x)


def quant_rows(cfg, block):
    """Rows of block `block` of the quantize workload: (row_block, C) bf16 bits.

    N(0,1) times a per-row scale 10^U(-3,3), in fp32, cast to bf16.
    """
    rb, C = cfg["row_block"], cfg["C"]
    g = rng(cfg["seed"], cfg["wid"], _T_ROWS, block)
    scale = np.power(np.float32(10.0), g.uniform(-3.0, 3.0, size=(rb, 1)).astype(np.float32))
    x = g.standard_normal((rb, C), dtype=np.float32) * scale.astype(np.float32)
    return to_bf16_bits(x)


def window_kv(cfg, layer, W):
    """A layer's sliding-window K and V rows for all B sequences: ([B][W][d], [B][W][d]) bf16 bits, N(0,1)."""
    g = rng(cfg["seed"], cfg["wid"], _T_WIN, layer)
    k = g.standard_normal((cfg["B"], W, cfg["d"]), dtype=np.float32)
    v = g.standard_normal((cfg["B"], W, cfg["d"]), dtype=np.float32)
    return to_bf16_bits(k), to_bf16_bits(v)


def proj_hidden(cfg, block):
    """Rows [block*row_block, (block+1)*row_block) of the projection workload's hidden state: bf16 N(0,1)."""
    g = rng(cfg["seed"], cfg["wid"], _T_HID, block)
    return to_bf16_bits(g.standard_normal((cfg["row_block"], cfg["D"]), dtype=np.float32))


def proj_weights_t(cfg):
    """The KV projection weights, transposed ([C][D], row c = output channel c): bf16 N(0, 1/D)."""
    g = rng(cfg["seed"], cfg["wid"], _T_WKV, 0)
    x = g.standard_normal((cfg["C"], cfg["D"]), dtype=np.float32) * np.float32(1.0 / np.sqrt(cfg["D"]))
    return to_bf16_bits(x)


def small(cfg_name, **over):
    """A copy of a workload with some sizes overridden (for parity tests at small sizes)."""
    cfg = dict(WORKLOADS[cfg_name])
    cfg.update(over)
    return cfg
