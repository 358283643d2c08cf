"""Lightning-indexer scores over compressed entries, computed exactly.

Test infrastructure: see the package docstring.

[P5] section "두 가지 압축 전략: CSA 및 HCA": a light indexer running in FP4
scores the compressed entries against the query. [P1] section "주요 댓글": the
DSA indexer scores all stored KV to find the tokens that matter to each query.
The pages give no formula. Reading taken: the published DSA lightning-indexer
form, s(t, j) = sum_h w[t, h] * ReLU(q[t, h] . k[j]), with q and k in MXFP4
(e2m1 elements, one E8M0 scale per 32 elements) and w = 1 unless given.

Every product of two e2m1 elements with power-of-two scales is dyadic, so the
score is a dyadic rational; the oracle evaluates it in fp64 and asserts that
it is exactly representable in fp32 (it is, when the scale spread per score
keeps all partial sums below 2^24 units of the smallest term).
"""
import numpy as np

from . import formats


def scores(iq, iq_scale, ik, ik_scale, n_valid, head_w=None):
    """One sequence.

    iq [T, H_I, D_I/2] packed e2m1, iq_scale [T, H_I, D_I/32] E8M0,
    ik [N, D_I/2], ik_scale [N, D_I/32], n_valid [T] visible entries per query,
    head_w [T, H_I] or None (= 1).  Returns fp64 [T, N]; entries j >= n_valid[t]
    are -inf.
    """
    # fp64 evaluation is exact while every term is a multiple of the smallest
    # one and the sum stays below 2^53 of those units: H*D*36*2^spread < 2^53.
    qs = np.asarray(iq_scale, dtype=np.int64)
    ks = np.asarray(ik_scale, dtype=np.int64)
    if ks.size and qs.size:
        spread = int(qs.max() - qs.min() + ks.max() - ks.min())
        assert spread <= 30, "MXFP4 scale spread too wide for an exact fp64 evaluation"
    q = formats.mxfp4_to_f64(iq, iq_scale)      # [T, H, D]
    k = formats.mxfp4_to_f64(ik, ik_scale)      # [N, D]
    return scores_decoded(q, k, n_valid, head_w)


def scores_decoded(q, k, n_valid, head_w=None):
    """The same scores from decoded (exact fp64) MXFP4 values: q [T, H_I, D_I], k [N, D_I].

    Callers that score many queries against one key set decode the keys once. The dot products
    are one matrix product (every product and partial sum is a dyadic rational that fp64 holds
    exactly, so the summation order does not change the result)."""
    T, H, D = q.shape
    N = k.shape[0]
    dots = (q.reshape(T * H, D) @ k.T).reshape(T, H, N)
    relu = np.maximum(dots, 0.0)
    w = np.ones((T, H)) if head_w is None else np.asarray(head_w, dtype=np.float64)
    s = np.einsum("th,thn->tn", w, relu)
    s = s + 0.0                                  # canonicalise -0 to +0
    assert np.array_equal(s.astype(np.float32).astype(np.float64), s), "index score not exact in fp32"
    j = np.arange(N)[None, :]
    nv = np.asarray(n_valid).reshape(T, 1)
    return np.where(j < nv, s, -np.inf)
