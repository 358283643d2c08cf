"""Decode loop of one CSA layer and one HCA layer with ring buffers and re-compression.

Test infrastructure: see the package docstring.

[P3] section "주요 인사이트": CSA layers and HCA layers are interleaved 1:1.
[P3] section "쉽게 이해하기" and [P4]: each keeps a window of the latest 128
tokens. [P5] section "두 가지 압축 전략: CSA 및 HCA": CSA pools 4 tokens per
entry and selects top-k with the FP4 indexer; HCA pools 128 tokens per entry
and attends to all entries.

Readings taken where the pages are silent:
  * decode step at position t: the new raw token (bf16) and its pooling logit
    go into ring slot t mod W; when (t+1) is a multiple of m, the block of
    positions [t-m+1, t] (contiguous ring slots, since m divides W) is
    compressed into entry (t+1)/m - 1 at position t-m+1; then the layer
    attends with its query at t;
  * the indexer key of each CSA entry is an input (already present in the key
    buffer); only its visibility (j < n_entries) changes during the loop;
  * a draft step ([P4] section "DSpark 추측 디코딩": the model checks a block of
    drafted tokens at once) appends all T draft tokens (with their block
    compressions) and then answers the T queries, query j seeing what a
    one-token step at t0 + j would see (entries j < (t0+j+1)/m, window up to
    t0 + j). The ring has R >= W + T - 1 slots (slot = position mod R, R a
    multiple of m) so that no query's window is overwritten. When only the
    first a draft tokens are accepted the next step starts at t0 + a: its
    tokens overwrite the rejected ring slots, and a block that held a rejected
    token is compressed again when it completes again.
"""
import numpy as np

from . import attention, compress, indexer, topk as topk_mod


class Layer:
    """State of one layer for a batch of sequences (arrays are modified in place)."""

    def __init__(self, kind, m, W, d_rope, d_v, rope_base, scale, ckv, ckv_scale, dtype,
                 n_entries, ring_x, ring_z, k=None, ik=None, ik_scale=None, ring_xk=None, rms_eps=0.0):
        assert kind in ("csa", "hca")
        self.kind, self.m, self.W = kind, m, W
        self.d_rope, self.d_v, self.rope_base, self.scale = d_rope, d_v, rope_base, scale
        self.ckv, self.ckv_scale, self.dtype = ckv, ckv_scale, dtype
        self.n_entries = np.array(n_entries, dtype=np.int64)
        self.ring_x, self.ring_z = ring_x, ring_z
        self.R = ring_x.shape[1]   # ring slots (W for one-token steps)
        assert self.R >= W and self.R % m == 0
        self.k, self.ik, self.ik_scale = k, ik, ik_scale
        # per-token indexer keys of the window: when given, each new entry's key is derived from
        # its tokens' keys (compress.index_keys) instead of being an input
        self.ring_xk = ring_xk
        # > 0: unit-gain RMSNorm of new entries and of the queries (compress.compress, attention.query)
        self.rms_eps = rms_eps

    def step(self, t, x_new, z_new, q, iq=None, iq_scale=None, outputs=True, sel_from=None, update=True,
             xk_new=None):
        """Positions t [B]; x_new [B, D] bf16; z_new [B]; q [B, H, D] bf16; iq [B, H_I, D_I/2].

        Returns (o fp64 [B, H, d_v], lse [B, H], idx int32 [B, k] or None); with
        outputs=False only the state update (window, re-compression) runs.

        Cross-layer index sharing ([P1] section "주요 댓글" on the indexer that chooses what
        attention reads, and the reuse / re-index layer modes): sel_from [B, k] gives the
        top-k of another layer, used instead of this layer's own indexer ("reuse"); with
        update=False the layer only reads its (shared) window and entries, another layer
        having appended and compressed them ("re-index": its own query, shared KV and keys).
        """
        B = len(t)
        outs, lses, idxs = [], [], []
        for b in range(B):
            tb = int(t[b])
            if update:
                self._update(b, tb, x_new[b], z_new[b], None if xk_new is None else xk_new[b])
                n = int(self.n_entries[b])
                assert n == (tb + 1) // self.m
            else:
                n = (tb + 1) // self.m  # the sharing layer has brought the entries up to t
            if not outputs:
                continue
            sel = None
            if self.kind == "csa" and sel_from is not None:
                sel = np.asarray(sel_from[b])
            elif self.kind == "csa":
                sc = indexer.scores(iq[b][None], iq_scale[b][None], self.ik[b, :n], self.ik_scale[b, :n],
                                    np.array([n]))
                sel, _ = topk_mod.topk(sc, self.k)
                sel = sel[0]
                idxs.append(sel)
            ent = attention.Entries(self.ckv[b], None if self.ckv_scale is None else self.ckv_scale[b],
                                    self.dtype)
            o, lse = attention.decode_one(q[b], tb, ent, n, sel, self.ring_x[b], self.W,
                                          self.d_rope, self.d_v, self.rope_base, self.scale, self.rms_eps,
                                          ring_cap=self.R)
            outs.append(o)
            lses.append(lse)
        if not outputs:
            return None, None, None
        return np.stack(outs), np.stack(lses), (np.stack(idxs) if idxs else None)

    def step_draft(self, t0, x_new, z_new, q, iq=None, iq_scale=None, xk_new=None):
        """One step of T draft tokens per sequence at positions t0[b] .. t0[b] + T - 1.

        x_new [B, T, D], z_new [B, T], q [B, T, H, D], iq [B, T, H_I, D_I/2], iq_scale
        [B, T, H_I, D_I/32], xk_new [B, T, D_I] or None. Returns (o [B, T, H, d_v], lse [B, T, H],
        idx [B, T, k] or None).
        """
        B, T = x_new.shape[0], x_new.shape[1]
        for b in range(B):
            for j in range(T):
                self._update(b, int(t0[b]) + j, x_new[b, j], z_new[b, j], None if xk_new is None else xk_new[b, j])
        outs, lses, idxs = [], [], []
        for b in range(B):
            ob, lb, ib = [], [], []
            ent = attention.Entries(self.ckv[b], None if self.ckv_scale is None else self.ckv_scale[b], self.dtype)
            for j in range(T):
                tj = int(t0[b]) + j
                n = (tj + 1) // self.m
                sel = None
                if self.kind == "csa":
                    sc = indexer.scores(iq[b, j][None], iq_scale[b, j][None], self.ik[b, :n], self.ik_scale[b, :n],
                                        np.array([n]))
                    sel = topk_mod.topk(sc, self.k)[0][0]
                    ib.append(sel)
                o, lse = attention.decode_one(q[b, j], tj, ent, n, sel, self.ring_x[b], self.W, self.d_rope,
                                              self.d_v, self.rope_base, self.scale, self.rms_eps, ring_cap=self.R)
                ob.append(o)
                lb.append(lse)
            outs.append(np.stack(ob))
            lses.append(np.stack(lb))
            if ib:
                idxs.append(np.stack(ib))
        return np.stack(outs), np.stack(lses), (np.stack(idxs) if idxs else None)

    def _update(self, b, tb, x_new, z_new, xk_new=None):
        """Window append of position tb and, at a block end, its compression (sequence b)."""
        self.ring_x[b, tb % self.R] = x_new
        self.ring_z[b, tb % self.R] = z_new
        if self.ring_xk is not None:
            self.ring_xk[b, tb % self.R] = xk_new
        if (tb + 1) % self.m == 0:
            j = (tb + 1) // self.m - 1
            # j < n_entries: the block is compressed again after a rejected draft token
            assert j <= self.n_entries[b], "entry count out of step with position"
            p0 = tb - self.m + 1
            slots = np.arange(p0, tb + 1) % self.R
            _, stored, s = compress.compress(self.ring_x[b, slots], self.ring_z[b, slots], p0,
                                             self.m, self.d_rope, self.rope_base, self.dtype, rms_eps=self.rms_eps)
            self.ckv[b, j] = stored[0]
            if s is not None:
                self.ckv_scale[b, j] = s[0]
            if self.ring_xk is not None:
                _, kp, ks = compress.index_keys(self.ring_xk[b, slots], self.ring_z[b, slots], self.m)
                self.ik[b, j] = kp[0]
                self.ik_scale[b, j] = ks[0]
            self.n_entries[b] = j + 1
