"""Parity checks between the HIP path's outputs and the oracle's (test helpers)."""
import numpy as np

from oracle import formats

REL_L2 = 5e-3       # attention outputs (bf16 out, fp32 accumulate)
MAX_ABS = 2e-2


class ParityError(AssertionError):
    pass


def topk_exact(got, want, what="top-k"):
    """Index lists must be bit-identical, order and -1 padding included."""
    got = np.asarray(got)
    want = np.asarray(want)
    if got.shape != want.shape:
        raise ParityError(f"{what}: shape {got.shape} != {want.shape}")
    bad = np.argwhere(got != want)
    if bad.size:
        r = tuple(bad[0][:-1])
        raise ParityError(f"{what}: {len(bad)} mismatching slots; first at {tuple(bad[0])}: "
                          f"got {got[r][:8]} want {want[r][:8]}")


def attn_close(got_bits, want, what="attention", rel_l2=REL_L2, max_abs=MAX_ABS):
    """bf16 output vs fp64 oracle: rel-L2 <= 5e-3 and max-abs <= 2e-2 over the whole tensor."""
    g = formats.bf16_to_f64(np.asarray(got_bits).view(np.uint16))
    w = np.asarray(want, dtype=np.float64)
    if g.shape != w.shape:
        raise ParityError(f"{what}: shape {g.shape} != {w.shape}")
    if not np.all(np.isfinite(g)):
        raise ParityError(f"{what}: non-finite output")
    err = np.linalg.norm((g - w).ravel())
    ref = np.linalg.norm(w.ravel())
    rel = err / max(ref, 1e-300)
    mab = np.abs(g - w).max() if g.size else 0.0
    if rel > rel_l2 or mab > max_abs:
        raise ParityError(f"{what}: rel-L2 {rel:.3e} (<= {rel_l2}) max-abs {mab:.3e} (<= {max_abs})")
    return rel, mab


def lse_close(got, want, bound=None, what="lse"):
    """|lse_gpu - lse_oracle| <= bound + 1e-5 * (1 + |lse|) per element.

    lse = ln sum_j exp(l_j) moves by at most max_j |dl_j|, so `bound` is a bound on the
    logit error (see rope_logit_bound); without one, 1e-3 is used.
    """
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    b = 1e-3 if bound is None else np.asarray(bound, dtype=np.float64)
    tol = b + 1e-5 * (1 + np.abs(w))
    d = np.abs(g - w)
    if g.size and not np.all(d <= tol):
        i = np.unravel_index(np.argmax(d - tol), d.shape)
        raise ParityError(f"{what}: |dlse| {d[i]:.3e} > {np.broadcast_to(tol, d.shape)[i]:.3e} at {i}")


def rope_logit_bound(q_rot, K, d_rope, scale, window_rows):
    """Logit error of a bf16 MFMA evaluation: q_rot's rotated dims and the rotated window keys
    are rounded to bf16 (relative error <= 2^-9 each) before the fp32-accumulated product.

    q_rot [H, D] and K [S, D] in fp64 (oracle); window_rows: boolean [S], keys rotated on the fly.
    Returns [H]: scale * max_j sum_{rotated i} |q_i| |k_ji| * (2^-9 (q) + 2^-9 (window key) + 2^-18)
    plus an fp32 accumulation allowance of D * 2^-24 * scale * max_j sum_i |q_i||k_ji|.
    """
    D = q_rot.shape[1]
    if K.shape[0] == 0:
        return np.zeros(q_rot.shape[0])
    aq, ak = np.abs(q_rot), np.abs(K)
    rot = slice(D - d_rope, D)
    per_key = 2.0 ** -9 + np.where(np.asarray(window_rows), 2.0 ** -9 + 2.0 ** -18, 0.0)
    rope_part = (aq[:, rot] @ ak[:, rot].T) * per_key[None, :]
    full = aq @ ak.T
    return scale * (rope_part.max(axis=1) + D * 2.0 ** -24 * full.max(axis=1))


def _ulp(v, p, emin):
    """Spacing of a p-bit-significand float grid at |v| (subnormal spacing below 2^emin)."""
    v = np.maximum(np.abs(v), 2.0 ** emin)
    return 2.0 ** (np.floor(np.log2(v)) - (p - 1))


# Relative rounding unit of the GPU's compression arithmetic. The kernels evaluate the pooling
# weights, the pooled sums, the RMSNorm factor and the rotation in fp64 (unit 2^-53); 2^-50
# leaves room for the few roundings of the library functions (exp, sin, cos, sqrt).
EVAL_UNIT = 2.0 ** -50


def pool_error_bound(mag, m, unit=EVAL_UNIT):
    """Bound on |evaluated pooled value - exact|: (m + 10) * unit * sum_i a_i |x_i| (RoPE pairs
    summed).

    A sum of m products a_i*x_i carries at most about m units of sum|a_i x_i|; the a_i (exp and
    divide) and the rotation add a few more units; 10 covers them.
    """
    return (m + 10) * unit * mag


def rms_error_bound(pooled, mag, e_exact, m, d_rope, eps, unit=EVAL_UNIT):
    """Bound on |evaluation - exact| of RMS-normalised, rotated entries.

    pooled: the oracle's exact unrotated pooled rows [n, D]; mag as for pool_error_bound;
    e_exact: the normalised rotated rows. With d the pooling bound and r = 1/sqrt(mean(v^2)
    + eps), the evaluated factor is within r * delta of r, delta = sum|v| d / sum v^2 + (D + 8)
    unit (sum of squares, square root, division), so an element is off by at most
    r d + delta |e| (rotated dims: the pair's |e| summed).
    """
    v = np.asarray(pooled, dtype=np.float64)
    D = v.shape[-1]
    d = pool_error_bound(np.asarray(mag, dtype=np.float64), m, unit)
    r = 1.0 / np.sqrt(np.mean(v * v, axis=-1, keepdims=True) + eps)
    delta = (np.abs(v) * d).sum(axis=-1, keepdims=True) / np.maximum((v * v).sum(axis=-1, keepdims=True), 1e-300) \
        + (D + 8) * unit
    ae = np.abs(np.asarray(e_exact, dtype=np.float64))
    if d_rope:
        rot = ae[..., D - d_rope:].reshape(ae.shape[:-1] + (d_rope // 2, 2)).sum(axis=-1)
        ae = ae.copy()
        ae[..., D - d_rope:] = np.repeat(rot, 2, axis=-1)
    return r * d + delta * ae


def compress_bf16_close(got_bits, e_exact, mag, m, what="compress bf16", max_frac=1e-3, d=None):
    """bf16 entries: |got - e| <= half a bf16 ulp of (|e| + d) + d, d = pool_error_bound.

    e_exact: the oracle's unrounded fp64 entries; mag: the oracle's pooling of |x|
    with the same weights (rotated dims: pair sums). At most max_frac of the
    elements may round differently from the oracle's own bf16 value. d: an explicit
    per-element bound instead (normalised entries: rms_error_bound).
    """
    g = formats.bf16_to_f64(np.asarray(got_bits).view(np.uint16))
    e = np.asarray(e_exact, dtype=np.float64)
    d = pool_error_bound(np.asarray(mag, dtype=np.float64), m) if d is None else np.asarray(d, np.float64)
    allowed = _ulp(np.abs(e) + d, 8, -126) / 2 + d
    err = np.abs(g - e)
    if not np.all(err <= allowed * (1 + 1e-9)):
        i = np.unravel_index(np.argmax(err - allowed), err.shape)
        raise ParityError(f"{what}: element {i} got {g[i]!r} exact {e[i]!r} (allowed {allowed[i]:.3e})")
    frac = np.count_nonzero(np.asarray(got_bits).view(np.uint16) != formats.f64_to_bf16(e)) / max(e.size, 1)
    if frac > max_frac:
        raise ParityError(f"{what}: {frac:.2e} of elements round differently from the oracle (> {max_frac})")


def compress_fp8_close(got_codes, got_scale, e_exact, mag, m, what="compress fp8", max_frac=1e-3, d=None):
    """fp8 entries with per-entry scale s = max|e|/448.

    Scale: relative error <= d(amax)/amax + 2^-22. Elements: |code*s - e| <= half an
    e4m3 step of |e|/s times s, plus d, plus |e| times the scale's relative error.
    """
    gs = np.asarray(got_scale, dtype=np.float64)
    e = np.asarray(e_exact, dtype=np.float64)
    d = pool_error_bound(np.asarray(mag, dtype=np.float64), m) if d is None else np.asarray(d, np.float64)
    amax = np.abs(e).max(axis=-1)
    s_ref = np.where(amax == 0, 1.0, amax / 448.0)
    i_max = np.argmax(np.abs(e), axis=-1)
    d_amax = np.take_along_axis(d, i_max[..., None], axis=-1)[..., 0]
    rs_allowed = np.where(amax == 0, 0.0, d_amax / np.maximum(amax, 1e-300)) + 2.0 ** -22
    rs = np.abs(gs - s_ref) / s_ref
    if not np.all(rs <= rs_allowed):
        i = np.unravel_index(np.argmax(rs - rs_allowed), rs.shape)
        raise ParityError(f"{what}: scale {i} rel diff {rs[i]:.2e} > {rs_allowed[i]:.2e}")
    g = formats.e4m3_to_f64(np.asarray(got_codes)) * gs[..., None]
    allowed = _ulp(np.abs(e) / s_ref[..., None] + d / s_ref[..., None], 4, -6) / 2 * gs[..., None] \
        + d + np.abs(e) * rs_allowed[..., None]
    err = np.abs(g - e)
    if not np.all(err <= allowed * (1 + 1e-9)):
        i = np.unravel_index(np.argmax(err - allowed), err.shape)
        raise ParityError(f"{what}: element {i} got {g[i]!r} exact {e[i]!r} (allowed {allowed[i]:.3e})")
    want_codes = formats.f64_to_e4m3(e / s_ref[..., None])
    frac = np.count_nonzero(np.asarray(got_codes) != want_codes) / max(e.size, 1)
    if frac > max_frac:
        raise ParityError(f"{what}: {frac:.2e} of codes differ from the oracle's (> {max_frac})")


def mxfp4_close(got_packed, got_scale, k_exact, mag, m, what="mxfp4 keys", max_frac=1e-3,
                e_range=(formats.MX_E_MIN, formats.MX_E_MAX), d=None):
    """MXFP4 values from the GPU's pooling vs the exact fp64 pooled values k_exact [..., D].

    With d = pool_error_bound(mag, m) the bound on |evaluated pooled - exact|: each block exponent is
    the one of some value within d of the block maximum, and each code lies between the codes of
    (v - d) and (v + d) under that exponent; at most max_frac of the codes differ from the
    oracle's own encoding (differences only where v is within d of a rounding midpoint).
    """
    k = np.asarray(k_exact, dtype=np.float64)
    d = pool_error_bound(np.asarray(mag, dtype=np.float64), m) if d is None else np.asarray(d, np.float64)
    D = k.shape[-1]
    gs = np.asarray(got_scale).astype(np.int64)
    kb = k.reshape(k.shape[:-1] + (D // 32, 32))
    db = d.reshape(kb.shape)
    amax_lo = np.maximum(np.abs(kb) - db, 0.0).max(axis=-1)   # the evaluated block maximum lies in [lo, hi]
    amax_hi = (np.abs(kb) + db).max(axis=-1)
    _, s_lo = formats.f64_to_mxfp4(np.repeat(amax_lo, 32, axis=-1).reshape(k.shape), *e_range)
    _, s_hi = formats.f64_to_mxfp4(np.repeat(amax_hi, 32, axis=-1).reshape(k.shape), *e_range)
    ok_s = (gs >= s_lo.astype(np.int64)) & (gs <= s_hi.astype(np.int64))
    if not np.all(ok_s):
        i = np.argwhere(~ok_s)[0]
        raise ParityError(f"{what}: block {tuple(i)} scale {gs[tuple(i)]} outside [{s_lo[tuple(i)]}, {s_hi[tuple(i)]}]")
    E = np.repeat(gs - 127, 32, axis=-1).reshape(k.shape)
    got = formats.unpack_fp4(got_packed)
    sval = lambda c: np.where(c & 8, -1, 1) * (c & 7)  # noqa: E731  (monotone in the value)
    lo = sval(formats.e2m1_round(np.abs(k - d) / 2.0 ** E) | np.where(k - d < 0, 8, 0))
    hi = sval(formats.e2m1_round(np.abs(k + d) / 2.0 ** E) | np.where(k + d < 0, 8, 0))
    g = sval(got.astype(np.int64))
    bad = (g < np.minimum(lo, hi)) | (g > np.maximum(lo, hi))
    if bad.any():
        i = tuple(np.argwhere(bad)[0])
        raise ParityError(f"{what}: element {i} code {got[i]} value {k[i]!r} (E={E[i]}, bound {d[i]:.2e})")
    want, _ = formats.f64_to_mxfp4(k, *e_range)
    frac = np.count_nonzero(got != formats.unpack_fp4(want)) / max(got.size, 1)
    if frac > max_frac:
        raise ParityError(f"{what}: {frac:.2e} of codes differ from the oracle's (> {max_frac})")
