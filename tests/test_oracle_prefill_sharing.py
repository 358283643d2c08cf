"""Pins of oracle.attention.prefill_one and of the cross-layer sharing branches of
oracle.hybrid.Layer.step (reuse: sel_from; re-index: update=False).

Page "DeepSeek-V4가 이차적 어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는 방법", section
"두 가지 압축 전략: CSA 및 HCA": every prompt position attends to its selected entries plus
its causal window; the blog post on DeepSeek V4.1 Flash (jjy0501.blogspot.com), paragraph on
CSA2's layer modes: a reuse layer takes another layer's top-k, a re-index layer shares the KV
but scores it with its own query.

Prefill rows are pinned against textbook causal attention (torch SDPA with a mask, fp64),
against the closed form of window duplicates (+ln 2 on their logits), and against the decode
oracle on a ring built from the prompt; the sharing branches against a from-scratch
recomputation over the token history (compression of every block, indexer, top-k, attention).
"""
import math

import numpy as np
import torch

from oracle import attention, compress, formats, hybrid, indexer, rope, topk


def _bf16(rng, shape, std=1.0):
    return formats.f64_to_bf16(rng.standard_normal(shape) * std)


def _sdpa_masked(q, k, v, scale, allowed, bias=None):
    """softmax(q k^T * scale + bias) v over the allowed keys, by torch (fp64, CPU).
    q [T, H, D], k [S, D], v [S, dv]; allowed [T, S] boolean; bias [T, S] or None."""
    T, H, D = q.shape
    qt = torch.from_numpy(np.ascontiguousarray(q.transpose(1, 0, 2))).double()[None]     # [1, H, T, D]
    kt = torch.from_numpy(np.ascontiguousarray(k)).double()[None, None].expand(1, H, -1, -1)
    vt = torch.from_numpy(np.ascontiguousarray(v)).double()[None, None].expand(1, H, -1, -1)
    b = np.where(allowed, 0.0, -np.inf) + (0.0 if bias is None else bias)
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=torch.from_numpy(b)[None, None],
                                                         scale=scale)
    return o[0].numpy().transpose(1, 0, 2)                                                # [T, H, dv]


def _rows(fn, T):
    o, l = zip(*[fn(r) for r in range(T)])
    return np.stack(o), np.stack(l)


def test_prefill_block_of_one_no_window_is_causal_attention():
    """m = 1, all visible entries selected (k = N and topk = None), W = 0: row t attends to the
    tokens at positions <= t, i.e. textbook causal attention (torch SDPA, causal mask)."""
    rng = np.random.default_rng(11)
    T, H, D, dr, dv, base, scale = 37, 3, 32, 16, 24, 10000.0, 0.3
    x = _bf16(rng, (T, D), 0.8)
    z = np.zeros(T, np.float32)                       # uniform pooling logits
    e, stored, _ = compress.compress(x, z, 0, 1, dr, base, "bf16")
    ent = attention.Entries(stored, None, "bf16")
    q = _bf16(rng, (T, H, D), 0.8)
    o_dense, l_dense = _rows(lambda r: attention.prefill_one(q[r], r, 0, ent, 1, None, x, 0, dr, dv, base, scale), T)
    sel_all = np.arange(T)
    o_sel, l_sel = _rows(lambda r: attention.prefill_one(q[r], r, 0, ent, 1, sel_all[:r + 1], x, 0, dr, dv, base,
                                                         scale), T)
    # keys: the stored entries (bf16 of the rotated tokens); queries rotated at their own row
    K = formats.bf16_to_f64(stored)
    qr = rope.apply(formats.bf16_to_f64(q), np.arange(T)[:, None].repeat(H, 1), dr, base)
    causal = np.tril(np.ones((T, T), bool))
    want = _sdpa_masked(qr, K, K[:, :dv], scale, causal)
    assert np.allclose(o_dense, want, rtol=1e-12, atol=1e-14)
    assert np.allclose(o_sel, want, rtol=1e-12, atol=1e-14)
    lg = scale * np.einsum("thd,sd->ths", qr, K)
    lse = np.log(np.where(causal[:, None, :], np.exp(lg), 0.0).sum(axis=-1))
    assert np.allclose(l_dense, lse, atol=1e-12) and np.allclose(l_sel, lse, atol=1e-12)


def test_prefill_window_starts_at_the_prompt_and_duplicates_add_ln2():
    """m = 1, no RoPE, every visible entry, W > 0, a prompt starting at pos0 > 0 whose entries
    cover the history before it: row t sees entries j <= t and raw tokens [max(pos0, t-W+1), t];
    each token present both ways gets +ln 2 on its logit. Rows near the prompt start have fewer
    than W window tokens (only those at or after pos0)."""
    rng = np.random.default_rng(12)
    pos0, T, H, D, dv, W, scale = 9, 30, 2, 16, 16, 7, 0.5
    hist = _bf16(rng, (pos0 + T, D), 0.7)             # tokens at positions 0 .. pos0 + T - 1
    _, stored, _ = compress.compress(hist, np.zeros(pos0 + T, np.float32), 0, 1, 0, 1.0, "bf16")
    assert np.array_equal(stored, hist)
    ent = attention.Entries(stored, None, "bf16")
    x = hist[pos0:]                                    # the prompt's raw tokens
    q = _bf16(rng, (T, H, D), 0.7)
    o, l = _rows(lambda r: attention.prefill_one(q[r], pos0 + r, pos0, ent, 1, None, x, W, 0, dv, 1.0, scale), T)
    K = formats.bf16_to_f64(hist)
    t = pos0 + np.arange(T)
    allowed = np.arange(pos0 + T)[None, :] <= t[:, None]
    in_win = (np.arange(pos0 + T)[None, :] >= np.maximum(pos0, t - W + 1)[:, None]) & allowed
    bias = np.where(in_win, math.log(2.0), 0.0)
    want = _sdpa_masked(formats.bf16_to_f64(q), K, K[:, :dv], scale, allowed, bias)
    assert np.allclose(o, want, rtol=1e-12, atol=1e-14)
    # rows whose window is clipped by the prompt start: duplicates = t - pos0 + 1 < W
    assert in_win[0].sum() == 1 and in_win[W - 2].sum() == W - 1 and in_win[W].sum() == W
    lg = scale * np.einsum("thd,sd->ths", formats.bf16_to_f64(q), K) + bias[:, None, :]
    lse = np.log(np.where(allowed[:, None, :], np.exp(lg), 0.0).sum(axis=-1))
    assert np.allclose(l, lse, atol=1e-12)


def test_prefill_rows_equal_decode_on_a_ring_built_from_the_prompt():
    """Every row of a prompt at pos0 > 0 (rows before the first block end included: window only)
    equals the decode oracle at that position with n_entries = floor((t+1)/m), a ring holding
    the prompt's tokens at slots position mod R and a window of the tokens since pos0."""
    rng = np.random.default_rng(13)
    pos0, T, m, H, D, dr, dv, W, k, base, scale = 6, 45, 4, 2, 24, 8, 16, 12, 5, 10000.0, 0.35
    n_tok = (pos0 + T) // m * m
    hist = _bf16(rng, (n_tok, D), 0.6)
    z = rng.standard_normal(n_tok).astype(np.float32)
    _, codes, sc = compress.compress(hist, z, 0, m, dr, base, "fp8")
    ent = attention.Entries(codes, sc, "fp8")
    N = n_tok // m
    x = _bf16(rng, (T, D), 0.6)                        # the prompt (its own raw tokens)
    q = _bf16(rng, (T, H, D), 0.6)
    tk = np.full((T, k), -1, np.int32)
    for r in range(T):
        vis = (pos0 + r + 1) // m
        s = rng.permutation(min(vis, N))[:k]
        tk[r, :len(s)] = s
    R = 16                                             # ring of R >= W slots
    for r in range(T):
        t = pos0 + r
        n = min(N, (t + 1) // m)
        for sel in (None, tk[r]):
            if sel is None and n < (t + 1) // m:
                continue
            o_p, l_p = attention.prefill_one(q[r], t, pos0, ent, m, sel, x, W, dr, dv, base, scale)
            w_eff = min(W, t - pos0 + 1)               # window tokens available in the prompt
            ring = np.zeros((R, D), np.uint16)
            for p in range(t - w_eff + 1, t + 1):
                ring[p % R] = x[p - pos0]
            o_d, l_d = attention.decode_one(q[r], t, ent, n, sel, ring, w_eff, dr, dv, base, scale, ring_cap=R)
            assert np.array_equal(o_p, o_d) and np.array_equal(l_p, l_d), (r, sel is None)
    # the first rows (t < m - 1 relative to the start of the entries) see no entries when pos0 = 0
    o0, _ = attention.prefill_one(q[0], 0, 0, ent, m, None, x, W, dr, dv, base, scale)
    xr = rope.apply(formats.bf16_to_f64(x[:1]), np.array([0]), dr, base)
    assert np.allclose(o0, np.repeat(xr[:, :dv], H, axis=0), rtol=1e-12, atol=1e-15)   # one key: weight 1


def _history(rng, B, L, steps, D, DI, cap):
    tokens = _bf16(rng, (B, L + steps, D), 0.5)
    logits = rng.standard_normal((B, L + steps)).astype(np.float32)
    ik = rng.integers(0, 256, (B, cap, DI // 2), dtype=np.uint8)
    iks = rng.integers(126, 128, (B, cap, DI // 32), dtype=np.uint8)
    return tokens, logits, ik, iks


def _csa_layer(tokens, logits, ik, iks, B, L, W, m, D, dr, dv, k, cap):
    ckv = np.zeros((B, cap, D), np.uint8)
    scl = np.ones((B, cap), np.float32)
    for b in range(B):
        _, c, s = compress.compress(tokens[b, :L], logits[b, :L], 0, m, dr, 10000.0, "fp8")
        ckv[b, :L // m], scl[b, :L // m] = c, s
    ring_x = np.zeros((B, W, D), np.uint16)
    ring_z = np.zeros((B, W), np.float32)
    for p in range(L - W, L):
        ring_x[:, p % W], ring_z[:, p % W] = tokens[:, p], logits[:, p]
    return hybrid.Layer("csa", m, W, dr, dv, 10000.0, 0.3, ckv, scl, "fp8", np.full(B, L // m), ring_x, ring_z,
                        k=k, ik=ik.copy(), ik_scale=iks.copy())


def _from_scratch(tokens, logits, ik, iks, b, t, m, W, dr, dv, q, sel=None, iq=None, iqs=None, k=None):
    """Output at position t recomputed from the whole token history of sequence b: every block
    compressed anew, the indexer and top-k (unless sel is given), the ring rebuilt."""
    n = (t + 1) // m
    _, c, sc = compress.compress(tokens[b, :n * m], logits[b, :n * m], 0, m, dr, 10000.0, "fp8")
    if sel is None:
        s = indexer.scores(iq[None], iqs[None], ik[b, :n], iks[b, :n], np.array([n]))
        sel = topk.topk(s, k)[0][0]
    ring = np.zeros((W, tokens.shape[-1]), np.uint16)
    for p in range(t - W + 1, t + 1):
        ring[p % W] = tokens[b, p]
    o, l = attention.decode_one(q, t, attention.Entries(c, sc, "fp8"), n, sel, ring, W, dr, dv, 10000.0, 0.3)
    return o, l, sel


def test_reuse_layer_attends_its_own_kv_over_the_source_top_k():
    """Reuse (sel_from): layer 1 keeps its own KV and window but takes layer 0's top-k; every
    step equals a from-scratch recomputation over layer 1's history with layer 0's selection,
    and layer 0's selection equals its own from-scratch indexer + top-k."""
    rng = np.random.default_rng(14)
    B, H, D, dv, dr, W, L, steps, m, HI, DI, k = 2, 2, 16, 8, 8, 16, 64, 23, 4, 2, 32, 6
    cap = (L + steps) // m + 1
    h0 = _history(rng, B, L, steps, D, DI, cap)
    h1 = _history(rng, B, L, steps, D, DI, cap)
    l0 = _csa_layer(*h0, B, L, W, m, D, dr, dv, k, cap)
    l1 = _csa_layer(*h1, B, L, W, m, D, dr, dv, k, cap)
    for s in range(steps):
        t = L + s
        tv = np.full(B, t)
        q0, q1 = _bf16(rng, (B, H, D), 0.5), _bf16(rng, (B, H, D), 0.5)
        iq = rng.integers(0, 256, (B, HI, DI // 2), dtype=np.uint8)
        iqs = np.full((B, HI, 1), 127, np.uint8)
        _, _, idx0 = l0.step(tv, h0[0][:, t], h0[1][:, t], q0, iq, iqs)
        o1, lse1, idx1 = l1.step(tv, h1[0][:, t], h1[1][:, t], q1, sel_from=idx0)
        assert idx1 is None                             # a reuse layer runs no indexer
        for b in range(B):
            _, _, sel0 = _from_scratch(*h0, b, t, m, W, dr, dv, q0[b], iq=iq[b], iqs=iqs[b], k=k)
            assert np.array_equal(idx0[b], sel0)
            o, l, _ = _from_scratch(*h1, b, t, m, W, dr, dv, q1[b], sel=sel0)
            assert np.array_equal(o1[b], o) and np.array_equal(lse1[b], l), (s, b)


def test_reindex_layer_scores_the_shared_kv_with_its_own_query():
    """Re-index (update=False): layer 1 shares layer 0's entries, window and indexer keys (layer 0
    appends and compresses), and scores them with its own indexer query; every step equals a
    from-scratch recomputation over layer 0's history with layer 1's query and top-k, and differs
    from layer 0's own selection somewhere."""
    rng = np.random.default_rng(15)
    B, H, D, dv, dr, W, L, steps, m, HI, DI, k = 2, 2, 16, 8, 8, 16, 64, 23, 4, 2, 32, 6
    cap = (L + steps) // m + 1
    h0 = _history(rng, B, L, steps, D, DI, cap)
    l0 = _csa_layer(*h0, B, L, W, m, D, dr, dv, k, cap)
    l1 = hybrid.Layer("csa", m, W, dr, dv, 10000.0, 0.3, l0.ckv, l0.ckv_scale, "fp8", l0.n_entries, l0.ring_x,
                      l0.ring_z, k=k, ik=l0.ik, ik_scale=l0.ik_scale)
    differ = 0
    for s in range(steps):
        t = L + s
        tv = np.full(B, t)
        q0, q1 = _bf16(rng, (B, H, D), 0.5), _bf16(rng, (B, H, D), 0.5)
        iq0 = rng.integers(0, 256, (B, HI, DI // 2), dtype=np.uint8)
        iq1 = rng.integers(0, 256, (B, HI, DI // 2), dtype=np.uint8)
        iqs = np.full((B, HI, 1), 127, np.uint8)
        _, _, idx0 = l0.step(tv, h0[0][:, t], h0[1][:, t], q0, iq0, iqs)
        o1, lse1, idx1 = l1.step(tv, None, None, q1, iq1, iqs, update=False)
        for b in range(B):
            o, l, sel = _from_scratch(*h0, b, t, m, W, dr, dv, q1[b], iq=iq1[b], iqs=iqs[b], k=k)
            assert np.array_equal(idx1[b], sel) and np.array_equal(o1[b], o) and np.array_equal(lse1[b], l), (s, b)
            differ += not np.array_equal(idx1[b], idx0[b])
    assert differ > 0
