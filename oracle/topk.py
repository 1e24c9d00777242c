"""Top-K position selection.

[jiwasawa] CSA2: Full and Reindex layers produce fresh Top-K indices; Reuse
layers take the Top-K indices of an earlier layer. [zaikei] "■CSA2とFP4で
キャッシュを圧縮": the selected token positions are shared across layers.

Readings (the pages state neither tie rule nor output order):
  * order: a before b iff score_a > score_b, or the scores are equal and
    pos_a < pos_b (lowest position wins a tie); -0 and +0 are equal;
  * NaN and -inf scores are never selected;
  * the first min(K, #selectable) entries of that order are taken and
    returned sorted by ascending position, padded with -1 up to K.
"""

import numpy as np


def topk(scores, K, positions=None):
    """scores: (n,) fp32; positions: (n,) ints or None (= 0..n-1).

    Returns (idx int32 [K], sel_scores fp32 [K]); padding slots hold -1 and NaN.
    """
    s = np.asarray(scores, dtype=np.float32)
    n = s.shape[0]
    pos = np.arange(n, dtype=np.int64) if positions is None else np.asarray(positions, dtype=np.int64)
    ok = ~np.isnan(s) & (s > -np.inf)
    s_ok = s[ok].astype(np.float64)
    p_ok = pos[ok]
    order = np.lexsort((p_ok, -s_ok))          # primary: score desc; secondary: position asc
    take = order[:K]
    chosen = p_ok[take]
    chosen_s = s[ok][take]
    asc = np.argsort(chosen, kind="stable")
    idx = np.full(K, -1, dtype=np.int32)
    sel = np.full(K, np.nan, dtype=np.float32)
    idx[: chosen.shape[0]] = chosen[asc]
    sel[: chosen.shape[0]] = chosen_s[asc]
    return idx, sel
