"""Plain CPU oracle for the CSA2 decode step over an FP4 E2M1 main KV cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package. The HIP product path (``fp4_compressed_sparse_kv_amd``) never
imports it, and this package imports nothing from the product path. The two
share only the seeded input generators in ``synth`` (which hold none of the
method's arithmetic).

Everything here is numpy on the host, in fp64 or exact integer/rational
arithmetic, written to be read against the pages, not to be fast.

Pages cited (by title and section):

* [ezic] "DeepSeek-V4.1-Flash: KVキャッシュ1トークン890バイト" (ai2.x.ezic.info),
  sections "先に要点だけ" (key points) and "KVを捨てる、共有する、作り直す"
  (drop / share / rebuild the KV).
* [zaikei] "DeepSeek-V4.1-Flash、KVキャッシュを約4分の1に圧縮" (zaikei.co.jp),
  section "■CSA2とFP4でキャッシュを圧縮".
* [jiwasawa] "DeepSeek-V4.1-Flash" technical-report digest (jiwasawa.github.io),
  sections "Compressed Sparse Attention 2 (CSA2) による極限のKV cache圧縮" and
  "FP4 メイン KV Cache と SWA Bounded Replay".

What the pages fix: the main KV is stored as FP4 E2M1 elements with one E4M3
scale per 16 channels and is dequantized before attention ([ezic] key points,
[zaikei] CSA2とFP4, [jiwasawa] FP4 main KV cache); each CSA2 layer is statically
Full, Reindex or Reuse; Full computes the indexer query and fresh top-K
positions, Reindex reuses the main KV and indexer keys of an earlier layer and
re-scores with its own query, Reuse inherits KV and top-K positions and skips
the indexer ([zaikei] CSA2とFP4, [jiwasawa] CSA2); the first Full layer picks a
candidate pool from the whole context that later Reindex layers search
([jiwasawa] CSA2, Hierarchical Sparse Indexer).

Readings taken where the pages are silent (each is repeated at its function):
scale = RNE_E4M3(amax / 6) saturating at 448, zero scale -> all codes 0x0;
E2M1 rounding is round-to-nearest-even with saturation and keeps the sign;
indexer score = plain dot product of indexer query and key, taken as the
exact sum rounded once to fp32; top-K order is (score desc, position asc),
non-finite scores never selected, output ascending by position and padded
with -1; pool = top-P of the first Full layer's scores; Reuse inherits the
immediately preceding layer's positions; attention uses scale 1/sqrt(d), all
heads share one KV head and one position list.

Parity unpinned by the pages: the scale rule above (a reading; pinned only
by internal invariants: idempotence, error bound, byte accounting) and the
890 B/token whole-model figure (not decomposed on the pages).
"""

from . import formats, quant, scores, topk, attention, plan  # noqa: F401

__all__ = ["formats", "quant", "scores", "topk", "attention", "plan"]
