"""Shared-KV MQA attention over compressed entries plus a sliding window.

Test infrastructure: see the package docstring.

[P5] section "두 가지 압축 전략: CSA 및 HCA": CSA runs softmax attention only on
the top-k selected entries with a sliding-window branch in parallel; HCA runs
dense attention over all of its entries; both use MQA with one shared KV
projection and partial RoPE. [P3] section "쉽게 이해하기": the window branch
covers the latest 128 tokens.

Readings taken where the pages are silent:
  * one stored vector u per entry/token: K = u (all D dims), V = u[:d_v];
  * compressed entries are stored already rotated; window tokens are stored raw
    and rotated at their own position; the query is rotated at its position t;
  * the window is the tokens [max(lo, t-W+1), t]; entries visible to t are
    j < floor((t+1)/m); a token may appear both raw in the window and inside a
    pooled entry (no de-duplication);
  * the window and the entries share ONE softmax per head (no learned gate);
  * logits = softmax_scale * q.K; lse is the natural log of the softmax
    denominator; output rounded to bf16 by RNE.
"""
import numpy as np

from . import formats, rope


def decode_entries(ckv, ckv_scale, dtype):
    """Stored entries -> fp64 vectors. bf16 bits, e4m3 codes times per-entry fp32 scale, or
    MXFP4 codes with per-32 E8M0 scales."""
    if dtype == "bf16":
        return formats.bf16_to_f64(ckv)
    if dtype == "mxfp4":
        return formats.mxfp4_to_f64(ckv, ckv_scale)
    assert dtype == "fp8"
    return formats.e4m3_to_f64(ckv) * np.asarray(ckv_scale, dtype=np.float64)[..., None]


def attend(q_rot, K, V, scale):
    """q_rot [H, D], K [S, D], V [S, d_v] fp64 -> (o [H, d_v], lse [H]). Empty S -> zeros, -inf."""
    H = q_rot.shape[0]
    if K.shape[0] == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    logits = scale * (q_rot @ K.T)                     # [H, S]
    mx = logits.max(axis=1, keepdims=True)
    w = np.exp(logits - mx)
    den = w.sum(axis=1, keepdims=True)
    o = (w / den) @ V
    lse = (mx + np.log(den))[:, 0]
    return o, lse


class Entries:
    """Stored compressed cache of one sequence, decoded row by row on demand."""

    def __init__(self, ckv, ckv_scale, dtype):
        self.ckv, self.scale, self.dtype = ckv, ckv_scale, dtype
        self.D = ckv.shape[-1] * (2 if dtype == "mxfp4" else 1)

    def rows(self, sel):
        sel = np.asarray(sel, dtype=np.int64)
        if sel.size == 0:
            return np.zeros((0, self.D))
        sc = None if self.scale is None else self.scale[sel]
        return decode_entries(self.ckv[sel], sc, self.dtype)


def key_set(t, entries, sel, win_tokens, win_pos, d_rope, d_v, rope_base):
    """Build (K, V) for query position t.

    entries: Entries (stored rows, already rotated); sel: entry ids (-1 skipped);
    win_tokens: raw bf16 bits [W_t, D] at positions win_pos [W_t].
    """
    sel = [int(j) for j in sel if j >= 0]
    Ke = entries.rows(sel)
    xw = formats.bf16_to_f64(win_tokens) if len(win_pos) else np.zeros((0, entries.D))
    Kw = rope.apply(xw, np.asarray(win_pos), d_rope, rope_base) if len(win_pos) else xw
    K = np.concatenate([Ke, Kw], axis=0)
    return K, K[:, :d_v]


def query(q_bits, t, d_rope, rope_base, q_rms_eps=0.0):
    """Query heads [H, D] as used in the logits: optionally RMS-normalised (unit gain, over
    the raw D dims; [P5]'s query normalisation), then rotated at position t."""
    q = formats.bf16_to_f64(q_bits)
    if q_rms_eps > 0:
        q = q / np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + q_rms_eps)
    return rope.apply(q, np.full(q_bits.shape[0], t), d_rope, rope_base)


def decode_one(q_bits, t, entries, n_entries, topk_idx, ring, W, d_rope, d_v, rope_base, scale, q_rms_eps=0.0,
               ring_cap=None):
    """One decode query for one sequence.

    q_bits [H, D] bf16 (unrotated) at position t; entries: Entries;
    n_entries visible entries; topk_idx [k] (CSA) or None (HCA: all j < n_entries);
    ring [R, D] bf16 raw token ring (R = ring_cap, default W), token at position p held in
    slot p mod R; the window is positions [max(0, t-W+1), t].
    """
    R = W if ring_cap is None else ring_cap
    q = query(q_bits, t, d_rope, rope_base, q_rms_eps)
    sel = range(n_entries) if topk_idx is None else [j for j in topk_idx if 0 <= j]
    if topk_idx is not None:
        assert all(j < n_entries for j in sel), "selected entry not visible"
    wpos = np.arange(max(0, t - W + 1), t + 1)
    wtok = ring[wpos % R] if W > 0 else np.zeros((0, entries.D), np.uint16)
    K, V = key_set(t, entries, sel, wtok, wpos if W > 0 else [], d_rope, d_v, rope_base)
    return attend(q, K, V, scale)


def prefill_one(q_bits, t, pos0, entries, m, topk_idx, x_bits, W, d_rope, d_v, rope_base, scale, q_rms_eps=0.0):
    """One prefill row at position t of a prompt whose raw tokens x_bits start at pos0.

    Entries visible: j < floor((t+1)/m); topk_idx [k] or None (= all visible).
    Window: raw tokens at positions [max(pos0, t-W+1), t] taken from x_bits.
    """
    n_vis = (t + 1) // m
    q = query(q_bits, t, d_rope, rope_base, q_rms_eps)
    sel = range(n_vis) if topk_idx is None else [j for j in topk_idx if 0 <= j]
    if topk_idx is not None:
        assert all(j < n_vis for j in sel), "selected entry not visible"
    wpos = np.arange(max(pos0, t - W + 1), t + 1) if W > 0 else np.zeros(0, np.int64)
    K, V = key_set(t, entries, sel, x_bits[wpos - pos0], wpos, d_rope, d_v, rope_base)
    return attend(q, K, V, scale)
