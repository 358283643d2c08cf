"""Pins of oracle.attention and oracle.hybrid: textbook attention, closed forms, brute force."""
import math

import numpy as np
import torch

from oracle import attention, compress, formats, hybrid, indexer, rope, topk


def _bf16(rng, shape, std=1.0):
    return formats.f64_to_bf16(rng.standard_normal(shape) * std)


def sdpa(q, k, v, scale, bias=None):
    """Textbook attention from torch (fp64, CPU): softmax(q k^T * scale + bias) v."""
    qt, kt, vt = (torch.from_numpy(np.ascontiguousarray(a)).double()[None, None] for a in (q, k, v))
    mask = None if bias is None else torch.from_numpy(bias).double()[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale)
    return o[0, 0].numpy()


def test_block_of_one_full_selection_no_window_is_plain_attention():
    """m=1, uniform logits, k=N, W=0, no RoPE: CSA reduces to textbook softmax attention."""
    rng = np.random.default_rng(0)
    L, H, D = 40, 4, 16
    x = _bf16(rng, (L, D), 0.7)
    _, stored, _ = compress.compress(x, np.zeros(L, np.float32), 0, 1, 0, 10000.0, "bf16")
    assert np.array_equal(stored, x)
    ent = attention.Entries(stored, None, "bf16")
    q = _bf16(rng, (H, D), 0.7)
    t = L - 1
    iq = rng.integers(0, 256, (1, 2, 16), dtype=np.uint8)
    ik = rng.integers(0, 256, (L, 16), dtype=np.uint8)
    sc = indexer.scores(iq, np.full((1, 2, 1), 127, np.uint8), ik, np.full((L, 1), 127, np.uint8), np.array([L]))
    sel = topk.topk(sc, L)[0][0]
    o, lse = attention.decode_one(q, t, ent, L, sel, np.zeros((1, D), np.uint16), 0, 0, D, 10000.0, 0.3)
    xf = formats.bf16_to_f64(x)
    want = sdpa(formats.bf16_to_f64(q), xf, xf, 0.3)
    assert np.allclose(o, want, rtol=1e-12, atol=1e-14)
    logits = 0.3 * formats.bf16_to_f64(q) @ xf.T
    assert np.allclose(lse, np.log(np.exp(logits).sum(axis=1)), atol=1e-12)


def test_topk_of_all_entries_equals_dense_hca_path():
    rng = np.random.default_rng(1)
    N, H, D, dv, W = 30, 3, 24, 16, 8
    ckv = rng.integers(0, 0x7E, (N, D), dtype=np.uint8)
    sc = rng.uniform(0.001, 0.01, N).astype(np.float32)
    ent = attention.Entries(ckv, sc, "fp8")
    ring = _bf16(rng, (W, D), 0.3)
    q = _bf16(rng, (H, D), 0.3)
    t = 4 * N + 2
    perm = rng.permutation(N)
    a = attention.decode_one(q, t, ent, N, perm, ring, W, 8, dv, 10000.0, 0.2)
    b = attention.decode_one(q, t, ent, N, None, ring, W, 8, dv, 10000.0, 0.2)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-15) and np.allclose(a[1], b[1], atol=1e-12)


def test_window_duplicates_add_ln2_to_their_logits():
    """m=1, k=N, W>0, no RoPE: the last W tokens appear twice -> +ln 2 on their logits."""
    rng = np.random.default_rng(2)
    L, H, D, W = 50, 2, 8, 6
    x = _bf16(rng, (L, D))
    ent = attention.Entries(x, None, "bf16")
    ring = np.zeros((W, D), np.uint16)
    t = L - 1
    for p in range(L - W, L):
        ring[p % W] = x[p]
    q = _bf16(rng, (H, D))
    o, lse = attention.decode_one(q, t, ent, L, np.arange(L), ring, W, 0, D, 1.0, 0.5)
    bias = np.zeros((H, L))
    bias[:, L - W:] = math.log(2.0)
    xf = formats.bf16_to_f64(x)
    assert np.allclose(o, sdpa(formats.bf16_to_f64(q), xf, xf, 0.5, bias), rtol=1e-12, atol=1e-14)


def test_no_entries_is_sliding_window_attention_and_union_is_lse_merge():
    rng = np.random.default_rng(3)
    H, D, dv, W, dr = 4, 16, 12, 8, 8
    t = 5                                      # fewer than W tokens so far, no entries
    ring = _bf16(rng, (W, D))
    q = _bf16(rng, (H, D))
    ent = attention.Entries(rng.integers(0, 0x7E, (4, D), dtype=np.uint8), np.ones(4, np.float32) / 64, "fp8")
    o, lse = attention.decode_one(q, t, ent, 0, None, ring, W, dr, dv, 10000.0, 0.25)
    pos = np.arange(0, t + 1)
    kw = rope.apply(formats.bf16_to_f64(ring[pos % W]), pos, dr, 10000.0)
    qr = rope.apply(formats.bf16_to_f64(q), np.full(H, t), dr, 10000.0)
    assert np.allclose(o, sdpa(qr, kw, kw[:, :dv], 0.25), rtol=1e-12, atol=1e-14)
    # union of entries and window = LSE-merge of the two partial attentions
    t2 = 23
    ring2 = _bf16(rng, (W, D))
    ou, lu = attention.decode_one(q, t2, ent, 4, None, ring2, W, dr, dv, 10000.0, 0.25)
    oe, le = attention.decode_one(q, t2, ent, 4, None, ring2, 0, dr, dv, 10000.0, 0.25)
    pos2 = np.arange(t2 - W + 1, t2 + 1)
    qr2 = rope.apply(formats.bf16_to_f64(q), np.full(H, t2), dr, 10000.0)
    kw2 = rope.apply(formats.bf16_to_f64(ring2[pos2 % W]), pos2, dr, 10000.0)
    ow, lw = attention.attend(qr2, kw2, kw2[:, :dv], 0.25)
    mx = np.maximum(le, lw)
    lm = mx + np.log(np.exp(le - mx) + np.exp(lw - mx))
    om = (np.exp(le - lm)[:, None] * oe + np.exp(lw - lm)[:, None] * ow)
    assert np.allclose(ou, om, rtol=1e-12, atol=1e-14) and np.allclose(lu, lm, atol=1e-12)


def test_decode_matches_loop_brute_force():
    rng = np.random.default_rng(4)
    N, H, D, dv, W, dr, base, scale = 6, 2, 8, 6, 4, 4, 100.0, 0.4
    ckv = _bf16(rng, (N, D))
    ring = _bf16(rng, (W, D))
    q = _bf16(rng, (H, D))
    t, sel = 29, [4, -1, 1, 5]
    o, lse = attention.decode_one(q, t, attention.Entries(ckv, None, "bf16"), 7, sel, ring, W, dr, dv, base, scale)

    def rot(v, p):
        v = list(v)
        for i in range(dr // 2):
            a = p * base ** (-2.0 * i / dr)
            x0, x1 = v[D - dr + 2 * i], v[D - dr + 2 * i + 1]
            v[D - dr + 2 * i], v[D - dr + 2 * i + 1] = x0 * math.cos(a) - x1 * math.sin(a), x0 * math.sin(a) + x1 * math.cos(a)
        return v
    keys = [list(formats.bf16_to_f64(ckv[j])) for j in (4, 1, 5)]
    keys += [rot(formats.bf16_to_f64(ring[p % W]), p) for p in range(t - W + 1, t + 1)]
    for h in range(H):
        qh = rot(formats.bf16_to_f64(q[h]), t)
        lg = [scale * sum(a * b for a, b in zip(qh, kk)) for kk in keys]
        mx = max(lg)
        ws = [math.exp(v - mx) for v in lg]
        den = sum(ws)
        for d in range(dv):
            assert abs(o[h, d] - sum(w * kk[d] for w, kk in zip(ws, keys)) / den) < 1e-12
        assert abs(lse[h] - (mx + math.log(den))) < 1e-12


def test_shifting_every_position_leaves_the_output_unchanged():
    rng = np.random.default_rng(5)
    m, nblk, H, D, dv, W, dr = 4, 8, 2, 16, 8, 8, 8
    x = _bf16(rng, (m * nblk, D))
    z = rng.standard_normal(m * nblk).astype(np.float32)
    q = _bf16(rng, (H, D))
    outs = []
    for shift in (0, 4 * 1000):
        e, _, _ = compress.compress(x, z, shift, m, dr, 10000.0, "bf16")
        # use the exact fp64 entries so only position arithmetic is tested
        class Exact:
            D = e.shape[1]

            def rows(self, sel, e=e):
                return e[np.asarray(sel, dtype=np.int64)] if len(sel) else np.zeros((0, self.D))
        t = shift + m * nblk - 1
        ring = np.zeros((W, D), np.uint16)
        for p in range(t - W + 1, t + 1):
            ring[p % W] = x[p - shift]
        outs.append(attention.decode_one(q, t, Exact(), nblk, None, ring, W, dr, dv, 10000.0, 0.3)[0])
    assert np.allclose(outs[0], outs[1], rtol=1e-9, atol=1e-12)


def test_hybrid_loop_equals_one_shot_recomputation():
    """The ring buffer and periodic re-compression agree with compressing the full token history."""
    rng = np.random.default_rng(6)
    B, H, D, dv, dr, W, L, steps = 2, 2, 16, 8, 8, 16, 64, 40
    HI, DI, k = 2, 32, 8
    tokens = _bf16(rng, (B, L + steps, D), 0.5)
    logits = rng.standard_normal((B, L + steps)).astype(np.float32)
    layers = {}
    for kind, m in (("csa", 4), ("hca", 16)):
        n0 = L // m
        cap = (L + steps) // m
        ckv = np.zeros((B, cap, D), np.uint8)
        scl = np.ones((B, cap), np.float32)
        for b in range(B):   # initial entries: compression of the history (so one-shot can rebuild them)
            _, c, s = compress.compress(tokens[b, :L], logits[b, :L], 0, m, dr, 10000.0, "fp8")
            ckv[b, :n0], scl[b, :n0] = c, s
        ring_x = np.zeros((B, W, D), np.uint16)
        ring_z = np.zeros((B, W), np.float32)
        for p in range(L - W, L):
            ring_x[:, p % W] = tokens[:, p]
            ring_z[:, p % W] = logits[:, p]
        ik = rng.integers(0, 256, (B, cap, DI // 2), dtype=np.uint8)
        iks = rng.integers(126, 128, (B, cap, DI // 32), dtype=np.uint8)
        layers[kind] = hybrid.Layer(kind, m, W, dr, dv, 10000.0, 0.3, ckv, scl, "fp8", np.full(B, n0),
                                    ring_x, ring_z, k=k, ik=ik, ik_scale=iks)
    for s in range(steps):
        t = np.full(B, L + s)
        q = _bf16(rng, (B, H, D), 0.5)
        iq = rng.integers(0, 256, (B, HI, DI // 2), dtype=np.uint8)
        iqs = np.full((B, HI, 1), 127, np.uint8)
        for kind, lay in layers.items():
            o, lse, idx = lay.step(t, tokens[:, L + s], logits[:, L + s], q, iq, iqs)
            m = lay.m
            n = (L + s + 1) // m
            for b in range(B):   # one-shot: compress the whole history, attend from scratch
                _, c, sc = compress.compress(tokens[b, :n * m], logits[b, :n * m], 0, m, dr, 10000.0, "fp8")
                assert np.array_equal(lay.ckv[b, :n], c) and np.array_equal(lay.ckv_scale[b, :n], sc)
                ent = attention.Entries(c, sc, "fp8")
                sel = None
                if kind == "csa":
                    scs = indexer.scores(iq[b][None], iqs[b][None], lay.ik[b, :n], lay.ik_scale[b, :n], np.array([n]))
                    sel = topk.topk(scs, k)[0][0]
                    assert np.array_equal(sel, idx[b])
                full_ring = np.zeros((W, D), np.uint16)
                for p in range(L + s - W + 1, L + s + 1):
                    full_ring[p % W] = tokens[b, p]
                o1, l1 = attention.decode_one(q[b], L + s, ent, n, sel, full_ring, W, dr, dv, 10000.0, 0.3)
                assert np.allclose(o[b], o1, rtol=0, atol=0) and np.allclose(lse[b], l1, rtol=0, atol=0)


def test_hybrid_loop_derived_keys_equal_one_shot_pooling():
    """Keys derived in the loop (ring of per-token keys) equal pooling the full key history."""
    rng = np.random.default_rng(7)
    B, D, dv, dr, W, L, steps, m, DI = 2, 16, 8, 8, 16, 32, 37, 4, 64
    tokens = _bf16(rng, (B, L + steps, D), 0.5)
    keys = _bf16(rng, (B, L + steps, DI), 1.0)
    logits = rng.standard_normal((B, L + steps)).astype(np.float32)
    cap = (L + steps) // m
    ring_x = np.zeros((B, W, D), np.uint16)
    ring_xk = np.zeros((B, W, DI), np.uint16)
    ring_z = np.zeros((B, W), np.float32)
    for p in range(L - W, L):
        ring_x[:, p % W], ring_xk[:, p % W], ring_z[:, p % W] = tokens[:, p], keys[:, p], logits[:, p]
    ik = np.zeros((B, cap, DI // 2), np.uint8)
    iks = np.zeros((B, cap, DI // 32), np.uint8)
    lay = hybrid.Layer("csa", m, W, dr, dv, 10000.0, 0.3, np.zeros((B, cap, D), np.uint8), np.ones((B, cap), np.float32),
                       "fp8", np.full(B, L // m), ring_x, ring_z, k=4, ik=ik, ik_scale=iks, ring_xk=ring_xk)
    for s in range(steps):
        lay.step(np.full(B, L + s), tokens[:, L + s], logits[:, L + s], None, outputs=False, xk_new=keys[:, L + s])
    n = (L + steps) // m
    for b in range(B):
        _, kp, ks = compress.index_keys(keys[b, L:n * m], logits[b, L:n * m], m)
        assert np.array_equal(ik[b, L // m:n], kp) and np.array_equal(iks[b, L // m:n], ks)
    assert not ik[:, n:].any()


def test_query_rms_norm_is_plain_attention_on_normalised_queries():
    """m=1, k=N, W=0, no RoPE, q_rms_eps > 0: textbook attention of torch-rms_norm'ed queries;
    with eps -> 0 the output does not depend on the query's scale."""
    rng = np.random.default_rng(23)
    L, H, D = 24, 3, 32
    x = _bf16(rng, (L, D), 0.5)
    ent = attention.Entries(x, None, "bf16")
    q = _bf16(rng, (H, D), 0.5)
    eps = 1e-5
    o, lse = attention.decode_one(q, L - 1, ent, L, None, np.zeros((1, D), np.uint16), 0, 0, D, 10000.0, 0.4,
                                  q_rms_eps=eps)
    qn = torch.nn.functional.rms_norm(torch.from_numpy(formats.bf16_to_f64(q)), (D,), eps=eps).numpy()
    xf = formats.bf16_to_f64(x)
    assert np.allclose(o, sdpa(qn, xf, xf, 0.4), rtol=1e-12, atol=1e-14)
    assert np.allclose(lse, np.log(np.exp(0.4 * qn @ xf.T).sum(axis=1)), atol=1e-12)
    q4 = formats.f64_to_bf16(4.0 * formats.bf16_to_f64(q))   # exact power-of-two scaling
    a = attention.decode_one(q, L - 1, ent, L, None, np.zeros((1, D), np.uint16), 0, 0, D, 10000.0, 0.4,
                             q_rms_eps=1e-30)
    b = attention.decode_one(q4, L - 1, ent, L, None, np.zeros((1, D), np.uint16), 0, 0, D, 10000.0, 0.4,
                             q_rms_eps=1e-30)
    assert np.allclose(a[0], b[0], rtol=1e-12, atol=1e-14)
    c = attention.decode_one(q4, L - 1, ent, L, None, np.zeros((1, D), np.uint16), 0, 0, D, 10000.0, 0.4)
    assert not np.allclose(a[0], c[0], rtol=1e-6)


def _layer(kind, m, W, R, B, L, D, dr, dv, cap, rng, tokens, logits, ik, iks, k):
    ckv = np.zeros((B, cap, D), np.uint8)
    scl = np.ones((B, cap), np.float32)
    n0 = L // m
    for b in range(B):
        _, c, s = compress.compress(tokens[b, :L], logits[b, :L], 0, m, dr, 10000.0, "fp8")
        ckv[b, :n0], scl[b, :n0] = c, s
    ring_x = np.zeros((B, R, D), np.uint16)
    ring_z = np.zeros((B, R), np.float32)
    for p in range(L - W, L):
        ring_x[:, p % R] = tokens[:, p]
        ring_z[:, p % R] = logits[:, p]
    return hybrid.Layer(kind, m, W, dr, dv, 10000.0, 0.3, ckv, scl, "fp8", np.full(B, n0), ring_x, ring_z, k=k,
                        ik=ik.copy(), ik_scale=iks.copy())


def test_draft_steps_equal_single_steps_and_rejected_tokens_leave_no_trace():
    """A draft step answers query j exactly as a one-token step at t0 + j; after only the first
    draft token is accepted, the next draft (re-drafted tokens) matches one-token steps over the
    accepted history: rejected tokens leave no trace in the ring or the entries."""
    rng = np.random.default_rng(8)
    B, H, D, dv, dr, W, L, T, m = 2, 2, 16, 8, 8, 8, 32, 3, 4
    HI, DI, k = 2, 32, 4
    n_tok = L + 16
    tokens = _bf16(rng, (B, n_tok, D), 0.5)
    logits = rng.standard_normal((B, n_tok)).astype(np.float32)
    cap = n_tok // m + 1
    ik = rng.integers(0, 256, (B, cap, DI // 2), dtype=np.uint8)
    iks = rng.integers(126, 128, (B, cap, DI // 32), dtype=np.uint8)
    q = _bf16(rng, (B, 8, H, D), 0.5)
    iq = rng.integers(0, 256, (B, 8, HI, DI // 2), dtype=np.uint8)
    iqs = np.full((B, 8, HI, 1), 127, np.uint8)
    rejected = _bf16(rng, (B, 2, D), 0.5)       # draft tokens 1 and 2 of the first step
    for kind, mm in (("csa", m), ("hca", 8)):
        R = -(-(W + T - 1) // mm) * mm           # >= W + T - 1, a multiple of m
        a = _layer(kind, mm, W, R, B, L, D, dr, dv, cap, rng, tokens, logits, ik, iks, k)
        s1 = _layer(kind, mm, W, W, B, L, D, dr, dv, cap, rng, tokens, logits, ik, iks, k)
        # step 1: draft of 3 at L (tokens L, rejected, rejected); only token L is accepted
        x1 = np.concatenate([tokens[:, L:L + 1], rejected], axis=1)
        z1 = np.concatenate([logits[:, L:L + 1], rng.standard_normal((B, 2)).astype(np.float32)], axis=1)
        o1, l1, _ = a.step_draft(np.full(B, L), x1, z1, q[:, 0:3], iq[:, 0:3], iqs[:, 0:3])
        # step 2: draft of 3 at L + 1 (the real tokens L+1 .. L+3)
        o2, l2, i2 = a.step_draft(np.full(B, L + 1), tokens[:, L + 1:L + 4], logits[:, L + 1:L + 4], q[:, 3:6],
                                  iq[:, 3:6], iqs[:, 3:6])
        # the same history one token at a time: L (query 0), then L+1 .. L+3 (queries 3..5)
        for j, (tq, qi) in enumerate([(L, 0), (L + 1, 3), (L + 2, 4), (L + 3, 5)]):
            o, lse, idx = s1.step(np.full(B, tq), tokens[:, tq], logits[:, tq], q[:, qi], iq[:, qi], iqs[:, qi])
            got_o, got_l = (o1[:, 0], l1[:, 0]) if j == 0 else (o2[:, j - 1], l2[:, j - 1])
            assert np.allclose(got_o, o, rtol=0, atol=0) and np.allclose(got_l, lse, rtol=0, atol=0), (kind, j)
            if kind == "csa" and j > 0:
                assert np.array_equal(i2[:, j - 1], idx)
        n = (L + 4) // mm
        assert np.array_equal(a.ckv[:, :n], s1.ckv[:, :n]) and np.array_equal(a.ckv_scale[:, :n], s1.ckv_scale[:, :n])
