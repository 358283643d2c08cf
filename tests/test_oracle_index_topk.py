"""Pins of oracle.indexer and oracle.topk: exact rational brute force and library sorts."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats, indexer, topk


def rand_mxfp4(rng, shape, e_lo=125, e_hi=128):
    """Random packed e2m1 codes [..., D/2] and E8M0 scales [..., D/32] in [e_lo, e_hi]."""
    *lead, D = shape
    packed = rng.integers(0, 256, tuple(lead) + (D // 2,), dtype=np.uint8)
    scales = rng.integers(e_lo, e_hi + 1, tuple(lead) + (D // 32,), dtype=np.uint8)
    return packed, scales


def frac_e2m1(c):
    mag = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]
    v = mag[c & 7]
    return -v if c & 8 else v


def frac_vec(packed, scales):
    out = []
    for d in range(packed.shape[-1] * 2):
        byte = int(packed[d // 2])
        code = byte & 15 if d % 2 == 0 else byte >> 4
        out.append(frac_e2m1(code) * Fraction(2) ** (int(scales[d // 32]) - 127))
    return out


@pytest.mark.parametrize("H,D", [(2, 32), (3, 64)])
def test_scores_equal_exact_rational_brute_force(H, D):
    rng = np.random.default_rng(H * 100 + D)
    T, N = 3, 7
    iq, iqs = rand_mxfp4(rng, (T, H, D))
    ik, iks = rand_mxfp4(rng, (N, D))
    w = np.array([[1.0, -0.5, 2.0][:H]] * T)
    s = indexer.scores(iq, iqs, ik, iks, np.array([7, 3, 0]), head_w=w)
    for t in range(T):
        for j in range(N):
            if j >= [7, 3, 0][t]:
                assert s[t, j] == -np.inf
                continue
            kv = frac_vec(ik[j], iks[j])
            tot = Fraction(0)
            for h in range(H):
                qv = frac_vec(iq[t, h], iqs[t, h])
                dot = sum(a * b for a, b in zip(qv, kv))
                tot += Fraction(w[t, h]) * max(dot, Fraction(0))
            assert Fraction(s[t, j]) == tot


def test_scores_are_exact_in_fp32_at_config_shape():
    rng = np.random.default_rng(11)
    iq, iqs = rand_mxfp4(rng, (1, 8, 128), 124, 127)
    ik, iks = rand_mxfp4(rng, (2048, 128), 124, 127)
    s = indexer.scores(iq, iqs, ik, iks, np.array([2048]))
    assert np.array_equal(s.astype(np.float32).astype(np.float64), s)


def test_exactness_guard_fires_outside_the_span():
    # two blocks with scales 2^30 apart: 32*2^30 + 32 is exact in fp64, not in fp32
    iq = np.zeros((1, 1, 32), np.uint8); iq[..., :] = 0x22      # all 1.0
    iqs = np.array([[[127, 127]]], np.uint8)
    ik = np.zeros((1, 32), np.uint8); ik[..., :] = 0x22
    iks = np.array([[157, 127]], np.uint8)
    with pytest.raises(AssertionError):
        indexer.scores(iq, iqs, ik, iks, np.array([1]))


def test_key_scale_shift_keeps_topk():
    rng = np.random.default_rng(12)
    iq, iqs = rand_mxfp4(rng, (2, 4, 64))
    ik, iks = rand_mxfp4(rng, (300, 64))
    a = topk.topk(indexer.scores(iq, iqs, ik, iks, np.array([300, 250])), 16)[0]
    b = topk.topk(indexer.scores(iq, iqs, ik, (iks + 1).astype(np.uint8), np.array([300, 250])), 16)[0]
    assert np.array_equal(a, b)


def test_topk_matches_python_sorted_with_ties_and_padding():
    rng = np.random.default_rng(13)
    T, N, k = 6, 200, 32
    s = rng.integers(0, 12, (T, N)).astype(np.float64) * 0.25     # many ties
    s[0, :5] = -0.0
    nv = np.array([200, 150, 32, 10, 1, 0])
    masked = np.where(np.arange(N)[None] < nv[:, None], s, -np.inf)
    idx, sc = topk.topk(masked, k)
    for t in range(T):
        want = sorted(range(nv[t]), key=lambda j: (-s[t, j], j))[:k]
        assert idx[t, :len(want)].tolist() == want
        assert np.all(idx[t, len(want):] == -1) and np.all(np.isneginf(sc[t, len(want):]))
        assert np.array_equal(sc[t, :len(want)], s[t, want].astype(np.float32))


def test_topk_equals_lexsort_truncation():
    rng = np.random.default_rng(14)
    s = rng.standard_normal((1, 5000))
    idx, _ = topk.topk(s, 128)
    order = np.lexsort((np.arange(5000), -s[0]))[:128]
    assert np.array_equal(idx[0], order)


def test_topk_with_k_at_least_n_returns_all_visible_in_key_order():
    s = np.array([[0.5, 2.0, 2.0, -1.0, 0.0]])
    idx, _ = topk.topk(s, 8)
    assert idx[0].tolist() == [1, 2, 0, 4, 3, -1, -1, -1]


def test_topk_permutation_and_low_entry_invariance():
    rng = np.random.default_rng(15)
    s = rng.integers(0, 50, (1, 400)).astype(np.float64)
    idx, _ = topk.topk(s, 20)
    perm = rng.permutation(400)
    sp = s[:, perm]
    idx_p, _ = topk.topk(sp, 20)
    # permuted indices map back to the same entries whenever no tie straddles the cut
    kth = s[0, idx[0, -1]]
    if np.sum(s[0] == kth) == np.sum(s[0, idx[0]] == kth):
        assert set(perm[idx_p[0]].tolist()) == set(idx[0].tolist())
    s2 = np.concatenate([s, np.full((1, 1), s[0, idx[0, -1]] - 1)], axis=1)
    assert np.array_equal(topk.topk(s2, 20)[0], idx)


def test_topk_selection_prefilter_keeps_ties_at_the_cut():
    """Rows longer than k go through a selection of the entries scoring at least the k-th largest
    score: with few distinct scores the cut falls inside a run of ties, which must be resolved by
    the lower index exactly as a full sort does (Python sorted over every visible entry)."""
    rng = np.random.default_rng(16)
    for T, N, k, levels in ((4, 3000, 128, 3), (3, 700, 1, 2), (2, 129, 128, 1), (5, 4000, 77, 40)):
        s = rng.integers(0, levels, (T, N)).astype(np.float64)
        nv = rng.integers(k, N + 1, T)
        masked = np.where(np.arange(N)[None] < nv[:, None], s, -np.inf)
        idx, _ = topk.topk(masked, k)
        for t in range(T):
            want = sorted(range(nv[t]), key=lambda j: (-s[t, j], j))[:k]
            assert idx[t].tolist() == want, (T, N, k, levels, t)


def test_decoded_scores_match_the_packed_entry_point():
    rng = np.random.default_rng(17)
    iq, iqs = rand_mxfp4(rng, (3, 4, 64))
    ik, iks = rand_mxfp4(rng, (500, 64))
    hw = rng.choice([1.0, -0.5, 2.0], (3, 4))
    nv = np.array([500, 17, 0])
    a = indexer.scores(iq, iqs, ik, iks, nv, hw)
    b = indexer.scores_decoded(formats.mxfp4_to_f64(iq, iqs), formats.mxfp4_to_f64(ik, iks), nv, hw)
    assert np.array_equal(a, b)
