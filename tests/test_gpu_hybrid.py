"""GPU parity of the CSA+HCA decode loop (ring append, periodic re-compression, index, attention)."""
import numpy as np
import pytest
import torch

from compressed_sparse_kv_03_amd import hybrid, native
from oracle import attention as oatt
from oracle import hybrid as ohyb
from tests import parity
from tests.gpu_util import say
from tests.test_gpu_attention import logit_bound

pytestmark = pytest.mark.gpu


def oracle_layers(spec, st):
    layers = {}
    for name, m in (("csa", spec.m_csa), ("hca", spec.m_hca)):
        h = st[name]
        csa = name == "csa"
        layers[name] = ohyb.Layer(name, m, spec.W, spec.d_rope, spec.d_v, spec.rope_base, spec.scale,
                                  h["ckv"].copy(), h["scl"].copy(), spec.kv_dtype, np.full(spec.B, spec.L // m),
                                  h["ring"].copy(), h["ringz"].copy(), k=spec.k,
                                  ik=st["ik"].copy() if csa else None, ik_scale=st["iks"].copy() if csa else None,
                                  ring_xk=st["ring_xk"].copy() if (csa and spec.derive_keys) else None,
                                  rms_eps=spec.rms_eps)
    return layers


def lse_bounds(spec, lay, t, q, idx):
    """Per-head logit error bounds of one step (after the oracle layer's update), for runs whose
    logits are large enough that the default lse tolerance does not cover the bf16 evaluation."""
    out = []
    for b in range(len(t)):
        tb = int(t[b])
        n = int(lay.n_entries[b])
        ent = oatt.Entries(lay.ckv[b], lay.ckv_scale[b], spec.kv_dtype)
        sel = range(n) if idx is None else [j for j in idx[b] if j >= 0]
        wpos = np.arange(max(0, tb - spec.W + 1), tb + 1)
        out.append(logit_bound(q[b], tb, ent, sel, lay.ring_x[b][wpos % spec.W], wpos, spec.d_rope, spec.d_v,
                               spec.scale, spec.rms_eps))
    return np.stack(out)


def check_mxfp4_entries(g_codes, g_scales, o_codes, o_scales, what):
    """MXFP4 entries of the loop against the oracle's: exponents within one (rarely different),
    codes within one e2m1 step, at most 1e-3 of either different."""
    from oracle import formats
    ordered = lambda c: np.where(c & 8, -(c & 7), c & 7).astype(np.int64)  # noqa: E731
    d = np.abs(ordered(formats.unpack_fp4(g_codes)) - ordered(formats.unpack_fp4(o_codes)))
    ds = np.abs(g_scales.astype(np.int64) - o_scales.astype(np.int64))
    assert d.max(initial=0) <= 1 and np.count_nonzero(d) <= 1e-3 * max(d.size, 1), f"{what}: mxfp4 codes"
    assert ds.max(initial=0) <= 1 and np.count_nonzero(ds) <= 1e-3 * max(ds.size, 1), f"{what}: mxfp4 exponents"


def check_loop(pair, sample_steps):
    spec = pair.s
    st = pair.host_state()
    layers = oracle_layers(spec, st)
    out = {n: pair.out[n].cpu().numpy() for n in ("csa", "hca")}
    lse = {n: pair.lse[n].cpu().numpy() for n in ("csa", "hca")}
    tk = pair.topk.cpu().numpy()
    checked = 0
    for i in range(spec.steps):
        want = i in sample_steps
        t = np.full(spec.B, spec.L + i)
        for name, lay in layers.items():
            h = st[name]
            iq = st["iq"][i][:, 0] if name == "csa" else None
            iqs = st["iqs"][i][:, 0] if name == "csa" else None
            xk = st["xkn"][i] if (name == "csa" and spec.derive_keys) else None
            o, l, idx = lay.step(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs, outputs=want, xk_new=xk)
            if want:
                if idx is not None:
                    parity.topk_exact(tk[i][:, 0], idx, f"{name} top-k step {i}")
                parity.attn_close(out[name][i], o, f"{name} step {i}")
                bnd = lse_bounds(spec, lay, t, h["q"][i], idx) if spec.rms_eps > 0 else None
                parity.lse_close(lse[name][i], l, bnd, f"{name} lse step {i}")
                checked += 1
    # the re-compressed entries written by the loop match the oracle's (codes within one step)
    for name in ("csa", "hca"):
        n_end = (spec.L + spec.steps) // pair.m[name]
        n0 = spec.L // pair.m[name]
        if spec.kv_dtype == "mxfp4":
            check_mxfp4_entries(pair.ckv[name][:, n0:n_end].cpu().numpy(), pair.scl[name][:, n0:n_end].cpu().numpy(),
                                layers[name].ckv[:, n0:n_end], layers[name].ckv_scale[:, n0:n_end], name)
            continue
        g_codes = pair.ckv[name][:, n0:n_end].cpu().numpy().astype(np.int64)
        o_codes = layers[name].ckv[:, n0:n_end].astype(np.int64)
        ordered = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)  # noqa: E731
        d = np.abs(ordered(g_codes) - ordered(o_codes))
        assert d.max(initial=0) <= 1, f"{name}: a new fp8 code differs by {d.max()} steps"
        assert np.count_nonzero(d) <= 1e-3 * d.size, f"{name}: {np.count_nonzero(d) / d.size:.2e} of codes differ"
        gs = pair.scl[name][:, n0:n_end].cpu().numpy().astype(np.float64)
        os_ = layers[name].ckv_scale[:, n0:n_end].astype(np.float64)
        # both sides round the same fp64 value amax / 448 to fp32
        assert np.all(np.abs(gs - os_) <= 2.0 ** -22 * os_), f"{name}: new entry scales differ"
    if spec.derive_keys:  # derived indexer keys of the new entries (fp64 pooling: identical bytes)
        n0, n_end = spec.L // spec.m_csa, (spec.L + spec.steps) // spec.m_csa
        assert np.array_equal(pair.ik[:, n0:n_end].cpu().numpy(), layers["csa"].ik[:, n0:n_end]), "derived keys"
        assert np.array_equal(pair.iks[:, n0:n_end].cpu().numpy(), layers["csa"].ik_scale[:, n0:n_end]), \
            "derived key scales"
    return checked


def test_hybrid_loop_small_every_step():
    spec = hybrid.LayerPairSpec(B=2, L=2048, steps=300, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=64,
                                wid=55)
    say("hybrid small", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    assert check_loop(pair, set(range(spec.steps))) == 2 * spec.steps


@pytest.mark.parametrize("dyadic", [True, False])
def test_hybrid_loop_derived_keys_every_step(dyadic):
    """New entries' indexer keys pooled from per-token keys on the GPU, keys and top-k against the
    oracle's bit for bit. dyadic: keys on a 1/16 grid with uniform weights (the pooling is exact,
    ties at e2m1 midpoints included); otherwise N(0,1) keys and logits (the GPU pools in fp64 and
    encodes from fp64, so its codes are the oracle's)."""
    spec = hybrid.LayerPairSpec(B=2, L=2048, steps=300, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=128,
                                wid=57, derive_keys=True, dyadic_keys=dyadic)
    say("hybrid derived keys", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    assert check_loop(pair, set(range(spec.steps))) == 2 * spec.steps


@pytest.mark.parametrize("eps", [1e-6, 0.01])
def test_hybrid_loop_rms_norm_every_step(eps):
    """Entries and queries RMS-normalised (unit gain) in the loop: new entries' fp8 codes within one
    step of the oracle's and every step's top-k and attention within the parity bounds. eps = 1e-6
    is the operating value (every entry and query becomes unit-RMS: the sharpest softmax of the
    loop tests); eps = 0.01 is of the order of the inputs' mean square (1/D), so the factor still
    varies per vector. The GPU pools and normalises in fp64 and rounds to fp8 from fp64, so its new
    entries carry the oracle's codes; an independently rounded cache (one e4m3 step apart in a
    dominant entry) can move this softmax's output by more than the tolerance."""
    spec = hybrid.LayerPairSpec(B=2, L=2048, steps=260, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=64,
                                wid=58, rms_eps=eps)
    say("hybrid rms", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    assert check_loop(pair, set(range(spec.steps))) == 2 * spec.steps


@pytest.mark.parametrize("qk_fp4", [False, True], ids=["widened", "qk_fp4"])
def test_hybrid_loop_mxfp4_entries_every_step(qk_fp4):
    """MXFP4 compressed KV (OCP MX: e2m1 codes, per-32 E8M0 exponents) written by the loop and read
    by both attention layers; every step against the oracle loop storing its own MXFP4 entries.
    qk_fp4: the entry logits on the scaled FP4 MFMA (CSKV_QK_FP4), on the 64-head kernel (forced:
    these key sets are short enough for the 16-head kernel, which widens either way)."""
    spec = hybrid.LayerPairSpec(B=2, L=2048, steps=260, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=64,
                                wid=60, kv_dtype="mxfp4", qk_fp4=qk_fp4)
    say("hybrid mxfp4", spec)
    if qk_fp4:
        native.cskv_attn_path(native.ATTN_G64)  # before the workspaces are sized
    try:
        pair = hybrid.LayerPair(spec)
        pair.run(0, spec.steps)
        torch.cuda.synchronize()
    finally:
        native.cskv_attn_path(native.ATTN_AUTO)
    assert check_loop(pair, set(range(spec.steps))) == 2 * spec.steps


def test_hybrid_loop_graph_replays_match_eager():
    spec = hybrid.LayerPairSpec(B=2, L=4096, steps=140, H=64, D=576, d_rope=64, d_v=512, wid=56)
    say("hybrid graph", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    ref = {n: pair.out[n].clone() for n in ("csa", "hca")}
    ref_tk = pair.topk.clone()
    g = torch.cuda.CUDAGraph()
    pair.restore()
    with torch.cuda.graph(g):
        pair.run(0, spec.steps)
    for rep in range(3):
        pair.restore()
        for n in ("csa", "hca"):
            pair.out[n].zero_()
        pair.topk.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()    # eager work between replays
        for n in ("csa", "hca"):
            assert torch.equal(pair.out[n], ref[n]), f"replay {rep}: {n} output differs from eager"
        assert torch.equal(pair.topk, ref_tk), f"replay {rep}: top-k differs from eager"


@pytest.mark.parametrize("draft,accept_seed,H,D,d_v,k", [(1, -1, 64, 576, 512, 128), (4, 3, 64, 576, 512, 128),
                                                         (1, -1, 16, 128, 128, 32)])
def test_hybrid_loop_fused_append_matches_separate(draft, accept_seed, H, D, d_v, k):
    """The loop with each layer's state update inside its attention call (hybrid_attn_decode_append,
    on steps that complete no block) equals the loop with separate cskv_ring_append launches bit
    for bit: outputs, lse and top-k of every step, and the final rings."""
    spec = dict(B=2, L=4096, steps=140, H=H, D=D, d_rope=64, d_v=d_v, k=k, wid=58, draft=draft,
                accept_seed=accept_seed)
    say("hybrid fused append", spec)
    res = []
    for fuse in (False, True):
        pair = hybrid.LayerPair(hybrid.LayerPairSpec(fuse_append=fuse, **spec))
        pair.run(0, spec["steps"])
        torch.cuda.synchronize()
        res.append(pair)
    a, b = res
    for n in ("csa", "hca"):
        assert torch.equal(a.out[n], b.out[n]), f"{n} outputs differ"
        assert torch.equal(a.lse[n], b.lse[n]), f"{n} lse differs"
        assert torch.equal(a.ring[n], b.ring[n]) and torch.equal(a.ringz[n], b.ringz[n]), f"{n} rings differ"
        assert torch.equal(a.ckv[n], b.ckv[n]), f"{n} compressed entries differ"
    assert torch.equal(a.topk, b.topk), "top-k differs"


@pytest.mark.parametrize("split,nside,share", [("layers", 1, None), ("chains", 1, None), ("chains", 2, "reuse"),
                                               ("chains", 1, "reindex")])
def test_hybrid_stack_streams_graph_matches_serial(split, nside, share):
    """A stack of three pairs stepped on several streams (parallel branches per step), captured in
    one graph and replayed three times: every replay equals the serial eager run bit for bit
    (outputs, lse and top-k of every step)."""
    spec = dict(B=2, L=4096, steps=132, H=64, D=576, d_rope=64, d_v=512, wid=57)
    say("hybrid stack streams", spec, split, nside, share)
    pairs = [hybrid.LayerPair(hybrid.LayerPairSpec(seed=p, **spec)) for p in range(3)]
    for i in range(spec["steps"]):
        hybrid.step_stack(pairs, i, share=share)
    torch.cuda.synchronize()
    ref = [({n: (pr.out[n].clone(), pr.lse[n].clone()) for n in ("csa", "hca")}, pr.topk.clone()) for pr in pairs]
    side = [torch.cuda.Stream() for _ in range(nside)]
    for pr in pairs:
        pr.restore()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(spec["steps"]):
            hybrid.step_stack(pairs, i, share=share, side=side, split=split)
    for rep in range(3):
        for pr in pairs:
            pr.restore()
            for n in ("csa", "hca"):
                pr.out[n].zero_()
                pr.lse[n].zero_()
            pr.topk.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _ = torch.randn(1000, device="cuda").sum().item()    # eager work between replays
        for p, pr in enumerate(pairs):
            for n in ("csa", "hca"):
                assert torch.equal(pr.out[n], ref[p][0][n][0]), f"replay {rep}: pair {p} {n} output"
                assert torch.equal(pr.lse[n], ref[p][0][n][1]), f"replay {rep}: pair {p} {n} lse"
            if share is None or p == 0:
                assert torch.equal(pr.topk, ref[p][1]), f"replay {rep}: pair {p} top-k"


def test_hybrid_loop_1m():
    """The 1M-context pair (B=8, 256 steps): the top-k of every step and sequence bit-exact against
    the oracle's indexer over the same keys, and both layers' attention on sampled steps (block
    ends of the CSA and HCA layers among them) against the oracle loop."""
    from oracle import formats
    from oracle import indexer as oidx
    from oracle import topk as otopk

    spec = hybrid.LayerPairSpec()
    say("hybrid 1M", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    tk = pair.topk.cpu().numpy()
    ik, iks = pair.ik.cpu().numpy(), pair.iks.cpu().numpy()
    iq, iqs = pair.iq.cpu().numpy(), pair.iqs.cpu().numpy()
    nv = pair.nvalid.cpu().numpy()
    blk = 8
    for b in range(spec.B):
        kdec = formats.mxfp4_to_f64(ik[b], iks[b])
        for s0 in range(0, spec.steps, blk):
            q = formats.mxfp4_to_f64(iq[s0:s0 + blk, b, 0], iqs[s0:s0 + blk, b, 0])
            want = otopk.topk(oidx.scores_decoded(q, kdec, nv[s0:s0 + blk, b, 0]), spec.k)[0]
            parity.topk_exact(tk[s0:s0 + blk, b, 0], want, f"1M top-k sequence {b} steps {s0}..{s0 + blk - 1}")
        say("hybrid 1M top-k of every step, sequence", b)
    steps = {0, 1, 3, 4, 5, 126, 127, 128, 129, 252, 255}
    assert check_loop(pair, steps) == 2 * len(steps)


@pytest.mark.parametrize("share", ["reuse", "reindex"])
def test_hybrid_loop_cross_layer_index_sharing(share):
    """A second CSA layer that reuses the first layer's top-k (its own KV), or re-indexes the first
    layer's KV and keys with its own query; checked every step against the oracle run the same way."""
    from dataclasses import replace

    spec0 = hybrid.LayerPairSpec(B=2, L=2048, steps=40, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=64,
                                 wid=57)
    spec1 = replace(spec0, wid=58)
    say("hybrid sharing", share, spec1)
    p0, p1 = hybrid.LayerPair(spec0), hybrid.LayerPair(spec1)
    for i in range(spec0.steps):
        p0.step(i)
        p1.step(i, share=share, src=p0)
    torch.cuda.synchronize()
    st0, st1 = p0.host_state(), p1.host_state()
    l0, l1 = oracle_layers(spec0, st0), oracle_layers(spec1, st1)
    if share == "reindex":  # the second CSA layer reads the first one's entries, window and keys
        a = l0["csa"]
        l1["csa"] = ohyb.Layer("csa", spec1.m_csa, spec1.W, spec1.d_rope, spec1.d_v, spec1.rope_base, spec1.scale,
                               a.ckv, a.ckv_scale, "fp8", a.n_entries, a.ring_x, a.ring_z, k=spec1.k,
                               ik=st0["ik"], ik_scale=st0["iks"])
    out = {n: p1.out[n].cpu().numpy() for n in ("csa", "hca")}
    lse = {n: p1.lse[n].cpu().numpy() for n in ("csa", "hca")}
    tk1 = p1.topk.cpu().numpy()
    for i in range(spec0.steps):
        t = np.full(spec0.B, spec0.L + i)
        idx0 = None
        for name, lay in l0.items():
            h = st0[name]
            iq = st0["iq"][i][:, 0] if name == "csa" else None
            iqs = st0["iqs"][i][:, 0] if name == "csa" else None
            _, _, idx = lay.step(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs)
            if name == "csa":
                idx0 = idx
        for name, lay in l1.items():
            h = st1[name]
            csa = name == "csa"
            iq = st1["iq"][i][:, 0] if csa else None
            iqs = st1["iqs"][i][:, 0] if csa else None
            o, l, idx = lay.step(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs,
                                 sel_from=idx0 if (csa and share == "reuse") else None,
                                 update=not (csa and share == "reindex"))
            if csa and share == "reindex":
                parity.topk_exact(tk1[i][:, 0], idx, f"re-index top-k step {i}")
            parity.attn_close(out[name][i], o, f"{share} {name} step {i}")
            parity.lse_close(lse[name][i], l, None, f"{share} {name} lse step {i}")


@pytest.mark.parametrize("draft,accept_seed", [(4, 3), (6, -1)])
def test_hybrid_loop_draft_steps(draft, accept_seed):
    """Multi-token decode: draft tokens checked per step, causal inside the draft, with a seeded
    number of accepted tokens per step (rejected ones overwritten by the next draft). Every query of
    every step against the oracle's draft step: top-k bit-exact, attention within the parity bounds,
    and the entries written by the loop (recompressed after rejections) within one fp8 step."""
    spec = hybrid.LayerPairSpec(B=2, L=2048, steps=70, H=16, D=128, d_rope=64, d_v=128, k=32, H_I=4, D_I=64,
                                wid=59, draft=draft, accept_seed=accept_seed)
    say("hybrid draft", spec)
    pair = hybrid.LayerPair(spec)
    pair.run(0, spec.steps)
    torch.cuda.synchronize()
    st = pair.host_state()
    layers = {}
    for name, m in (("csa", spec.m_csa), ("hca", spec.m_hca)):
        h = st[name]
        layers[name] = ohyb.Layer(name, m, spec.W, spec.d_rope, spec.d_v, spec.rope_base, spec.scale,
                                  h["ckv"].copy(), h["scl"].copy(), "fp8", np.full(spec.B, spec.L // m),
                                  h["ring"].copy(), h["ringz"].copy(), k=spec.k,
                                  ik=st["ik"].copy() if name == "csa" else None,
                                  ik_scale=st["iks"].copy() if name == "csa" else None)
    out = {n: pair.out[n].cpu().numpy() for n in ("csa", "hca")}
    lse = {n: pair.lse[n].cpu().numpy() for n in ("csa", "hca")}
    tk = pair.topk.cpu().numpy()
    B, T = spec.B, draft
    for i in range(spec.steps):
        t0 = np.full(B, st["t0"][i])
        for name, lay in layers.items():
            h = st[name]
            csa = name == "csa"
            o, l, idx = lay.step_draft(t0, h["xn"][i], h["zn"][i], h["q"][i], st["iq"][i] if csa else None,
                                       st["iqs"][i] if csa else None)
            if idx is not None:
                parity.topk_exact(tk[i], idx, f"draft top-k step {i}")
            parity.attn_close(out[name][i], o.reshape(B * T, spec.H, spec.d_v), f"draft {name} step {i}")
            parity.lse_close(lse[name][i], l.reshape(B * T, spec.H), None, f"draft {name} lse step {i}")
    last = int(st["t0"][-1]) + draft          # entries of complete blocks up to the last position
    for name in ("csa", "hca"):
        n0, n_end = spec.L // pair.m[name], last // pair.m[name]
        g = pair.ckv[name][:, n0:n_end].cpu().numpy().astype(np.int64)
        o_ = layers[name].ckv[:, n0:n_end].astype(np.int64)
        ordered = lambda c: np.where(c & 0x80, -(c & 0x7F), c & 0x7F)  # noqa: E731
        d = np.abs(ordered(g) - ordered(o_))
        assert d.max(initial=0) <= 1 and np.count_nonzero(d) <= 1e-3 * max(d.size, 1), f"{name} entries"
