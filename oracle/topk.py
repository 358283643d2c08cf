"""Top-k selection over index scores.

Test infrastructure: see the package docstring.

[P5] section "두 가지 압축 전략: CSA 및 HCA": the indexer keeps the most relevant
top-k entries (typically about 128). Readings taken: order by score descending,
ties broken by the lower entry index, -0 equal to +0; only entries visible to
the query take part; when fewer than k are visible the list is padded with -1
(score -inf). The order is strict, so the result is unique.
"""
import numpy as np


def topk(scores, k):
    """scores [T, N] fp64 (-inf = not visible) -> (idx int32 [T, k], score fp32 [T, k])."""
    T, N = scores.shape
    idx = np.full((T, k), -1, dtype=np.int32)
    sc = np.full((T, k), -np.inf, dtype=np.float32)
    for t in range(T):
        row = scores[t] + 0.0
        vis = np.nonzero(np.isfinite(row))[0]
        if vis.size == 0:
            continue
        if vis.size > k:
            # the first k entries in (score desc, index asc) order all score at least the k-th
            # largest visible score, so only those entries need sorting
            kth = np.partition(row[vis], vis.size - k)[vis.size - k]
            vis = vis[row[vis] >= kth]
        order = np.lexsort((vis, -row[vis]))   # primary: score desc; secondary: index asc
        take = vis[order[:k]]
        idx[t, :take.size] = take
        sc[t, :take.size] = row[take]
    return idx, sc
