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


def lse_close(got, want, what="lse", atol=1e-3):
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    d = np.abs(g - w).max() if g.size else 0.0
    if not d <= atol:
        raise ParityError(f"{what}: max |dlse| {d:.3e} > {atol}")


def compress_bf16_close(got_bits, want_bits, what="compress bf16", max_frac=1e-3):
    """Every element within 1 bf16 ulp of the oracle's stored value; at most 0.1% differ."""
    g = np.asarray(got_bits).view(np.int16).astype(np.int64)
    w = np.asarray(want_bits).view(np.int16).astype(np.int64)
    # ulp distance on the sign-magnitude encoding
    def ordered(v):
        return np.where(v < 0, -(v & 0x7FFF), v)
    d = np.abs(ordered(g) - ordered(w))
    if d.max(initial=0) > 1:
        raise ParityError(f"{what}: element {np.unravel_index(np.argmax(d), d.shape)} off by {d.max()} ulp")
    frac = np.count_nonzero(d) / max(d.size, 1)
    if frac > max_frac:
        raise ParityError(f"{what}: {frac:.2e} of elements differ by 1 ulp (> {max_frac})")


def compress_fp8_close(got_codes, got_scale, want_codes, want_scale, what="compress fp8", max_frac=1e-3):
    gs = np.asarray(got_scale, dtype=np.float64)
    ws = np.asarray(want_scale, dtype=np.float64)
    rs = np.abs(gs - ws) / np.abs(ws)
    if rs.max(initial=0) > 1e-6:
        raise ParityError(f"{what}: scale rel diff {rs.max():.2e} > 1e-6")
    g = np.asarray(got_codes).astype(np.int64)
    w = np.asarray(want_codes).astype(np.int64)
    def ordered(v):
        return np.where(v & 0x80, -(v & 0x7F), v & 0x7F)
    d = np.abs(ordered(g) - ordered(w))
    if d.max(initial=0) > 1:
        raise ParityError(f"{what}: a code differs by {d.max()} steps")
    frac = np.count_nonzero(d) / max(d.size, 1)
    if frac > max_frac:
        raise ParityError(f"{what}: {frac:.2e} of codes differ by one step (> {max_frac})")
