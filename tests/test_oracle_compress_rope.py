"""Pins of oracle.rope and oracle.compress: closed forms, invariants, brute force."""
import math
import os

import numpy as np
import torch

from oracle import compress, formats, rope

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(rng, shape, std=1.0):
    return formats.f64_to_bf16(rng.standard_normal(shape) * std)


# ------------------------------------------------------------------ RoPE
def test_rope_matches_complex_rotation():
    rng = np.random.default_rng(0)
    D, dr, base = 12, 8, 10000.0
    u = rng.standard_normal((5, D))
    pos = np.array([0, 1, 7, 1000, 2 ** 20 + 3])
    got = rope.apply(u, pos, dr, base)
    # textbook complex form: (u_2i + i u_2i+1) * exp(i p base^(-2i/dr)) on the last dr dims
    z = u[:, D - dr::2] + 1j * u[:, D - dr + 1::2]
    theta = np.array([base ** (-(2.0 * i) / dr) for i in range(dr // 2)])
    zr = z * np.exp(1j * pos[:, None] * theta[None, :])
    assert np.allclose(got[:, :D - dr], u[:, :D - dr], rtol=0, atol=0)
    assert np.allclose(got[:, D - dr::2], zr.real, rtol=0, atol=1e-12)
    assert np.allclose(got[:, D - dr + 1::2], zr.imag, rtol=0, atol=1e-12)


def test_rope_position_zero_and_no_rope_are_identity():
    u = np.random.default_rng(1).standard_normal((3, 16))
    assert np.array_equal(rope.apply(u, np.zeros(3, np.int64), 8, 10000.0), u)
    assert np.array_equal(rope.apply(u, np.arange(3) * 99, 0, 10000.0), u)


def test_rope_preserves_pair_norms():
    u = np.random.default_rng(2).standard_normal((4, 64))
    r = rope.apply(u, np.array([3, 50, 9999, 123456]), 64, 10000.0)
    assert np.allclose(np.hypot(r[:, 0::2], r[:, 1::2]), np.hypot(u[:, 0::2], u[:, 1::2]), atol=1e-13)


def test_rope_dot_depends_only_on_position_difference():
    rng = np.random.default_rng(3)
    q, k = rng.standard_normal(32), rng.standard_normal(32)
    for a, b, d in [(5, 2, 1000), (100, 0, 77777), (2 ** 20, 2 ** 20 - 128, 12345)]:
        d0 = rope.apply(q, np.array(a), 32, 10000.0) @ rope.apply(k, np.array(b), 32, 10000.0)
        d1 = rope.apply(q, np.array(a + d), 32, 10000.0) @ rope.apply(k, np.array(b + d), 32, 10000.0)
        # fp64 angles of size ~2^20 carry ~1e-10 absolute error
        assert abs(d0 - d1) < 1e-9 * (1 + abs(d0))


# ------------------------------------------------------------------ pooling
def test_identical_tokens_pool_to_that_token_rotated():
    rng = np.random.default_rng(4)
    m, D, dr = 4, 16, 8
    tok = _bf16(rng, (3, D))
    x = np.repeat(tok, m, axis=0)
    z = rng.standard_normal(3 * m).astype(np.float32)
    e, _, _ = compress.compress(x, z, 40, m, dr, 10000.0, "bf16")
    want = rope.apply(formats.bf16_to_f64(tok), 40 + np.arange(3) * m, dr, 10000.0)
    assert np.allclose(e, want, rtol=0, atol=1e-14)


def test_uniform_logits_give_the_mean_and_logit_shift_is_invisible():
    rng = np.random.default_rng(5)
    m, D = 128, 24
    x = _bf16(rng, (2 * m, D))
    e, _, _ = compress.compress(x, np.zeros(2 * m, np.float32), 0, m, 0, 10000.0, "bf16")
    want = formats.bf16_to_f64(x).reshape(2, m, D).mean(axis=1)
    assert np.allclose(e, want, rtol=0, atol=1e-15)
    z = (np.round(rng.standard_normal(2 * m) * 1024) / 1024).astype(np.float32)  # exact after +shift
    e1, _, _ = compress.compress(x, z, 0, m, 0, 10000.0, "bf16")
    zs = (z.astype(np.float64) + np.repeat([3.0, -7.5], m)).astype(np.float32)
    e2, _, _ = compress.compress(x, zs, 0, m, 0, 10000.0, "bf16")
    assert np.allclose(e1, e2, rtol=0, atol=1e-14)


def test_pooled_entry_lies_in_the_convex_hull_per_dim():
    rng = np.random.default_rng(6)
    m, D = 4, 32
    x = _bf16(rng, (64 * m, D))
    z = (rng.standard_normal(64 * m) * 3).astype(np.float32)
    e, _, _ = compress.compress(x, z, 0, m, 0, 10000.0, "bf16")
    xb = formats.bf16_to_f64(x).reshape(64, m, D)
    assert np.all(e <= xb.max(axis=1) + 1e-15) and np.all(e >= xb.min(axis=1) - 1e-15)


def test_block_of_one_is_the_rotated_token():
    rng = np.random.default_rng(7)
    x = _bf16(rng, (9, 16))
    e, _, _ = compress.compress(x, rng.standard_normal(9).astype(np.float32), 100, 1, 8, 10000.0, "bf16")
    assert np.allclose(e, rope.apply(formats.bf16_to_f64(x), 100 + np.arange(9), 8, 10000.0), atol=1e-15)


def test_compress_matches_loop_brute_force():
    rng = np.random.default_rng(8)
    m, D, dr, base, pos0 = 4, 8, 4, 500.0, 17
    x = _bf16(rng, (3 * m, D))
    z = rng.standard_normal(3 * m).astype(np.float32)
    e, stored, _ = compress.compress(x, z, pos0, m, dr, base, "bf16")
    xf = formats.bf16_to_f64(x)
    for j in range(3):
        zz = [float(z[j * m + i]) for i in range(m)]
        den = sum(math.exp(v) for v in zz)
        pooled = [sum(math.exp(zz[i]) / den * xf[j * m + i, d] for i in range(m)) for d in range(D)]
        p = pos0 + j * m
        for i in range(dr // 2):
            ang = p * base ** (-2.0 * i / dr)
            a, b = pooled[D - dr + 2 * i], pooled[D - dr + 2 * i + 1]
            pooled[D - dr + 2 * i] = a * math.cos(ang) - b * math.sin(ang)
            pooled[D - dr + 2 * i + 1] = a * math.sin(ang) + b * math.cos(ang)
        assert np.allclose(e[j], pooled, rtol=1e-12, atol=1e-14)
    assert np.array_equal(stored, formats.f64_to_bf16(e))


def test_fp8_storage_scale_and_rounding_bound():
    rng = np.random.default_rng(9)
    m, D = 128, 64
    x = _bf16(rng, (4 * m, D), 1 / 8)
    z = rng.standard_normal(4 * m).astype(np.float32)
    e, codes, s = compress.compress(x, z, 2 ** 20, m, 16, 10000.0, "fp8")
    assert s.dtype == np.float32
    amax = np.abs(e).max(axis=1)
    assert np.allclose(s, amax / 448.0, rtol=1e-7, atol=0)
    dec = formats.e4m3_to_f64(codes)
    assert np.all(np.abs(dec).max(axis=1) == 448.0)        # the largest element maps to the top code
    # RNE: error at most half a step of the e4m3 grid around each value (step 2^(e-3), subnormal 2^-9)
    v = e / s.astype(np.float64)[:, None]
    ex = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -6)))
    assert np.all(np.abs(dec - v) <= 2.0 ** (ex - 3) / 2 + 1e-12)


def test_zero_entry_gets_unit_scale():
    x = np.zeros((4, 8), np.uint16)
    _, codes, s = compress.compress(x, np.zeros(4, np.float32), 0, 4, 0, 10000.0, "fp8")
    assert s[0] == 1.0 and np.all(codes == 0)


def test_page_entry_counts():
    consts = {}
    for line in open(os.path.join(GOLD, "page_constants.txt")):
        if line.strip() and not line.startswith("#"):
            name, val = line.split()[:2]
            consts[name] = int(val)
    assert 4096 // consts["csa_block"] == 1024
    assert 65536 // consts["csa_block"] == 16384
    n_hca = 2 ** 20 // consts["hca_block"]
    assert n_hca == 8192 and abs(n_hca - consts["hca_entries_1m_approx"]) / 8000 < 0.03
    assert consts["hca_block"] // consts["csa_block"] == consts["hca_vs_csa_memory"]


def test_index_keys_pool_with_the_entry_weights():
    """Pooled indexer keys: identical tokens give that token's key (exactly, with equal logits: the
    weights are exactly 1/m); uniform logits give the mean (np.mean); the weights are those of the
    entries (keys equal to the KV rows pool to the un-rotated entries)."""
    rng = np.random.default_rng(7)
    m, D_I = 4, 64
    tok = formats.f64_to_bf16(rng.normal(0, 1, (1, D_I)))
    xk = np.repeat(tok, 3 * m, axis=0)
    k, p, s = compress.index_keys(xk, np.zeros(3 * m), m)
    assert np.array_equal(k, np.repeat(formats.bf16_to_f64(tok), 3, axis=0))
    p1, s1 = formats.f64_to_mxfp4(formats.bf16_to_f64(tok))
    assert np.array_equal(p, np.repeat(p1, 3, axis=0)) and np.array_equal(s, np.repeat(s1, 3, axis=0))
    k, _, _ = compress.index_keys(xk, rng.normal(0, 2, 3 * m), m)
    assert np.allclose(k, np.repeat(formats.bf16_to_f64(tok), 3, axis=0), rtol=1e-15, atol=0)
    xk = formats.f64_to_bf16(rng.normal(0, 1, (3 * m, D_I)))
    k, _, _ = compress.index_keys(xk, np.zeros(3 * m), m)
    assert np.allclose(k, formats.bf16_to_f64(xk).reshape(3, m, D_I).mean(axis=1), rtol=1e-15, atol=0)
    z = rng.normal(0, 2, 3 * m)
    k, _, _ = compress.index_keys(xk, z, m)
    e, _, _ = compress.compress(xk, z, 0, m, 0, 10000.0, "bf16")
    assert np.array_equal(k, e)


def test_rms_norm_matches_torch_and_has_unit_mean_square():
    """The entry normalisation against torch's rms_norm (fp64) and its closed-form mean square."""
    rng = np.random.default_rng(21)
    e = rng.standard_normal((7, 96)) * rng.uniform(0.01, 10, (7, 1))
    eps = 1e-6
    got = compress.rms_norm(e, eps)
    want = torch.nn.functional.rms_norm(torch.from_numpy(e), (96,), eps=eps).numpy()
    assert np.allclose(got, want, rtol=1e-13, atol=0)
    ms = np.mean(e * e, axis=1)
    assert np.allclose(np.mean(got * got, axis=1), ms / (ms + eps), rtol=1e-13)
    # scale invariance: (c e, c^2 eps) normalises to the same vector
    assert np.allclose(compress.rms_norm(3.0 * e, 9.0 * eps), got, rtol=1e-13)


def test_compress_with_rms_norm_is_normalise_then_rotate():
    """Normalising before or after the rotation gives the same entry (pairs keep their norm);
    rms_eps = 0 leaves the pooling unchanged."""
    rng = np.random.default_rng(22)
    m, D, dr, n = 4, 64, 32, 5
    x = formats.f64_to_bf16(rng.standard_normal((n * m, D)) * 0.3)
    z = rng.standard_normal(n * m).astype(np.float32)
    e_plain, _, _ = compress.compress(x, z, 100, m, dr, 10000.0, "bf16")
    e_norm, _, _ = compress.compress(x, z, 100, m, dr, 10000.0, "bf16", rms_eps=1e-6)
    assert np.allclose(e_norm, compress.rms_norm(e_plain, 1e-6), rtol=1e-12, atol=1e-15)
    pooled = compress.pool(formats.bf16_to_f64(x), z.astype(np.float64), m)
    rot = rope.apply(compress.rms_norm(pooled, 1e-6), 100 + np.arange(n) * m, dr, 10000.0)
    assert np.allclose(e_norm, rot, rtol=1e-12, atol=1e-15)


def test_compress_mxfp4_is_the_encoding_of_the_exact_entry():
    rng = np.random.default_rng(24)
    m, D, dr, n = 4, 128, 64, 6
    x = formats.f64_to_bf16(rng.standard_normal((n * m, D)) * 0.2)
    z = rng.standard_normal(n * m).astype(np.float32)
    e, codes, scales = compress.compress(x, z, 12, m, dr, 10000.0, "mxfp4")
    want_c, want_s = formats.f64_to_mxfp4(e, -127, 127)
    assert np.array_equal(codes, want_c) and np.array_equal(scales, want_s)
    e_bf, _, _ = compress.compress(x, z, 12, m, dr, 10000.0, "bf16")
    assert np.array_equal(e, e_bf)      # same exact entry, only the storage differs
