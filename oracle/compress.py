"""KV compression: softmax-weighted pooling of m consecutive tokens into one entry.

Test infrastructure: see the package docstring.

[P5] section "두 가지 압축 전략: CSA 및 HCA": CSA merges 4 consecutive tokens
into one KV entry by softmax-weighted pooling; HCA merges 128 tokens into one.
[P3] section "쉽게 이해하기": the merge is learned (each token's contribution is
learned), not a plain mean.

Readings taken where the pages are silent:
  * one scalar pooling logit z per token; softmax over the m tokens of a block;
  * blocks are aligned and non-overlapping: block j = tokens [j*m, j*m+m);
  * the pooled vector is rotated (partial RoPE) AFTER pooling, at position
    p_j = pos0 + j*m + entry_pos_offset (offset 0: the block's first token);
  * storage: bf16 by RNE, or e4m3fn with one fp32 scale per entry,
    s = max|e|/448 (s = 1 when the entry is all zero), code = RNE_sat(e/s), or
    OCP MXFP4 (next-row N4; [P4]: the main KV cache kept at FP4 precision) with
    the block exponent over the whole E8M0 range [-127, 127];
  * optional KV normalisation ([P5] section "두 가지 압축 전략: CSA 및 HCA": both
    branches normalise queries and KV): when rms_eps > 0 the pooled entry is
    divided by sqrt(mean(e^2) + rms_eps) (RMSNorm with unit gain) before the
    rotation. The rotation keeps each pair's norm, so the order of the two
    steps does not change the exact result.
"""
import numpy as np

from . import formats, rope


def pool(x, z, m):
    """x [n_tok, D] fp64, z [n_tok] fp64 -> pooled [n_tok/m, D] fp64 (no RoPE)."""
    n_tok, D = x.shape
    assert n_tok % m == 0
    xb = x.reshape(n_tok // m, m, D)
    zb = z.reshape(n_tok // m, m)
    zmax = zb.max(axis=1, keepdims=True)
    w = np.exp(zb - zmax)
    alpha = w / w.sum(axis=1, keepdims=True)
    return np.einsum("jm,jmd->jd", alpha, xb)


def rms_norm(e, eps):
    """Unit-gain RMSNorm of each row: e / sqrt(mean(e^2) + eps)."""
    e = np.asarray(e, dtype=np.float64)
    return e / np.sqrt(np.mean(e * e, axis=-1, keepdims=True) + eps)


def compress(x_bits, z, pos0, m, d_rope, rope_base, out_dtype, entry_pos_offset=0, rms_eps=0.0):
    """One sequence.

    x_bits [n_tok, D] bf16 bits; z [n_tok] fp32; pos0 = position of x[0].
    Returns (exact fp64 rotated entries [n, D], stored, scale) where stored is
    bf16 bits [n, D] (scale None), e4m3 codes [n, D] with fp32 scales [n], or MXFP4
    codes [n, D/2] with E8M0 scales [n, D/32].
    """
    x = formats.bf16_to_f64(x_bits)
    zz = np.asarray(z, dtype=np.float64)
    e = pool(x, zz, m)
    if rms_eps > 0:
        e = rms_norm(e, rms_eps)
    n = e.shape[0]
    p = pos0 + np.arange(n, dtype=np.int64) * m + entry_pos_offset
    e = rope.apply(e, p, d_rope, rope_base)
    if out_dtype == "bf16":
        return e, formats.f64_to_bf16(e), None
    if out_dtype == "mxfp4":
        codes, scales = formats.f64_to_mxfp4(e, formats.MX_KV_E_MIN, formats.MX_KV_E_MAX)
        return e, codes, scales
    assert out_dtype == "fp8"
    amax = np.abs(e).max(axis=1)
    s = np.where(amax == 0, 1.0, amax / formats.E4M3_MAX).astype(np.float32)
    codes = formats.f64_to_e4m3(e / s.astype(np.float64)[:, None])
    return e, codes, s


def magnitude(x_bits, z, m, d_rope):
    """sum_i a_i |x_i| per pooled element (rotated dims: the pair's two sums added).

    The scale of the rounding error of any finite-precision evaluation of the
    pooled entry; parity bounds are stated in multiples of it.
    """
    mag = pool(np.abs(formats.bf16_to_f64(x_bits)), np.asarray(z, dtype=np.float64), m)
    if d_rope:
        D = mag.shape[1]
        pair = mag[:, D - d_rope::2] + mag[:, D - d_rope + 1::2]
        mag[:, D - d_rope::2] = pair
        mag[:, D - d_rope + 1::2] = pair
    return mag


def index_keys(xk_bits, z, m):
    """Indexer keys of the entries of one sequence: the per-token keys xk_bits [n_tok, D_I] (bf16
    bits) pooled with the same softmax weights as the entries (z [n_tok]), then MXFP4-encoded.
    Reading (the pages give the indexer keys no source of their own): an entry's key is the pooled
    key of its tokens, stored like the other indexer inputs ([P5] section "두 가지 압축 전략: CSA
    및 HCA": the indexer runs in FP4). No RoPE.
    Returns (exact fp64 pooled keys [n, D_I], packed codes [n, D_I/2], E8M0 scales [n, D_I/32])."""
    k = pool(formats.bf16_to_f64(xk_bits), np.asarray(z, dtype=np.float64), m)
    packed, scales = formats.f64_to_mxfp4(k)
    return k, packed, scales

