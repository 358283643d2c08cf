"""Decode loop of one CSA layer and one HCA layer (interleaved 1:1) on the GPU.

Page "딥시크 V4 분석: CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한 방법",
section "주요 인사이트": CSA and HCA layers alternate 1:1; section "쉽게 이해하기":
every layer keeps a window of the latest 128 tokens. Page "DeepSeek-V4가 이차적
어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는 방법", section "두 가지 압축 전략:
CSA 및 HCA": CSA pools 4 tokens per entry and selects top-k with the FP4 indexer,
HCA pools 128 per entry and attends densely.

One decode step at position t (the same t for every sequence of the batch):
  1. each layer writes its new raw token and pooling logit to ring slot t mod R (inside the
     layer's attention call when step 2 has nothing to compress, hybrid_attn_decode_append);
  2. if (t+1) % m == 0 the layer compresses ring slots of positions [t-m+1, t]
     (contiguous because m divides R) into entry (t+1)/m - 1;
  3. CSA: csa_index_topk over the visible entries, then hybrid_attn_decode on
     the selected entries + window; HCA: hybrid_attn_decode over all entries +
     window.
A draft step (draft = T > 1; the blog post on DeepSeek V4.1 Flash at jjy0501.blogspot.com,
section "DSpark 추측 디코딩":
the model checks a block of drafted tokens at once) appends T tokens at t0..t0+T-1
(with every block that completes) and answers T queries per sequence, query j
seeing entries j < (t0+j+1)/m and the window up to t0+j; the rings have
R >= W + T - 1 slots. With accept_seed >= 0 each step accepts a seeded number
of its draft tokens (1..T) and the next step starts after them: its tokens
overwrite the rejected ring slots and blocks holding rejected tokens are
compressed again when they complete again.
Every step is a call of libcskv.so on the current stream; the host only picks
pointers. All per-step inputs are generated up front and the per-step counts
live in device arrays, so a run of steps can be captured in one HIP graph.
"""
from dataclasses import dataclass

import numpy as np
import torch

from . import native, synth


@dataclass
class LayerPairSpec:
    B: int = 8
    L: int = 1 << 20          # position of the first decode token
    steps: int = 256
    H: int = 64
    D: int = 576
    d_rope: int = 64
    d_v: int = 512
    W: int = 128
    m_csa: int = 4
    m_hca: int = 128
    k: int = 128
    H_I: int = 8
    D_I: int = 128
    rope_base: float = 10000.0
    seed: int = 0
    wid: int = 5
    # the CSA layer derives each new entry's indexer key from per-token keys pooled with the
    # entry's weights (csa_index_key_pool) instead of taking it from the generator
    derive_keys: bool = False
    # per-token keys on a 1/16 grid and zero CSA pooling logits: the pooling is exact in fp32
    # (used by the loop parity test, where the derived keys must equal the oracle's)
    dyadic_keys: bool = False
    # > 0: unit-gain RMSNorm (this epsilon) of the new compressed entries and of the queries
    rms_eps: float = 0.0
    # draft tokens checked per step (1: plain decode) and the acceptance schedule (-1: every
    # draft token accepted; else the seed of the accepted counts, uniform in 1..draft)
    draft: int = 1
    accept_seed: int = -1
    # storage of the compressed entries: "fp8" (e4m3fn + fp32 scale per entry) or "mxfp4"
    kv_dtype: str = "fp8"
    # mxfp4 entries: attention logits on the scaled FP4 MFMA from the stored codes (CSKV_QK_FP4)
    qk_fp4: bool = False
    # a step that completes no block of a layer appends that layer's new tokens inside its attention
    # call (hybrid_attn_decode_append) instead of a cskv_ring_append launch of its own
    fuse_append: bool = True

    @property
    def sigma(self):
        return self.D ** -0.5

    @property
    def scale(self):
        return self.D ** -0.5


class LayerPair:
    """Device state and inputs of the CSA+HCA decode loop."""

    def __init__(self, spec: LayerPairSpec, device="cuda"):
        s = spec
        self.s = s
        self.dev = device
        assert s.W % s.m_csa == 0 and s.W % s.m_hca == 0 and s.L % s.m_hca == 0 and s.L % s.m_csa == 0
        assert s.L >= s.W and s.draft >= 1 and s.kv_dtype in ("fp8", "mxfp4")
        assert not s.qk_fp4 or s.kv_dtype == "mxfp4"
        self.kv_code = native.CSKV_MXFP4 if s.kv_dtype == "mxfp4" else native.CSKV_FP8_E4M3
        self.attn_code = self.kv_code | (native.CSKV_QK_FP4 if s.qk_fp4 else 0)
        sd = lambda t: synth.seed_of(s.seed, s.wid, t)  # noqa: E731
        B, D, T, Td = s.B, s.D, s.steps, s.draft
        self.m = {"csa": s.m_csa, "hca": s.m_hca}
        # rings of R >= W + Td - 1 slots, a multiple of m (R = W for one-token steps)
        self.R = {n: -(-(s.W + Td - 1) // m) * m for n, m in self.m.items()}
        # first draft position of every step
        if s.accept_seed < 0:
            acc = np.full(T, Td, np.int64)
        else:
            acc = np.random.default_rng(s.accept_seed).integers(1, Td + 1, T).astype(np.int64)
        t0 = s.L + np.concatenate([[0], np.cumsum(acc)[:-1]]).astype(np.int64)
        self.t_host, self.accepted = t0, acc
        last = int(t0[-1]) + Td - 1
        self.n0 = {"csa": s.L // s.m_csa, "hca": s.L // s.m_hca}
        self.cap = {n: (last + 1) // m + 1 for n, m in self.m.items()}
        self.ckv, self.scl, self.ring, self.ringz, self.q, self.xn, self.zn = {}, {}, {}, {}, {}, {}, {}
        for li, name in enumerate(("csa", "hca")):
            base = 100 * li
            R = self.R[name]
            gen = synth.mxfp4_rows_normal if s.kv_dtype == "mxfp4" else synth.fp8_rows_normal
            c, sc = gen((B, self.cap[name], D), s.sigma, sd(base + 0), device)
            self.ckv[name], self.scl[name] = c, sc
            # window tokens at positions L-W .. L-1, in ring slots (position mod R)
            self.ring[name] = self._to_ring(synth.normal_bf16_bits((B, s.W, D), s.sigma, sd(base + 1), device), R)
            self.ringz[name] = self._to_ring(synth.normal((B, s.W), 1.0, sd(base + 2), device), R)
            self.q[name] = synth.normal_bf16_bits((T, B, Td, s.H, D), s.sigma, sd(base + 3), device)
            self.xn[name] = synth.normal_bf16_bits((T, B, Td, D), s.sigma, sd(base + 4), device)
            self.zn[name] = synth.normal((T, B, Td), 1.0, sd(base + 5), device)
        # indexer keys of every entry (without derive_keys, future entries' keys are inputs too)
        # and queries
        self.ik, self.iks = synth.mxfp4_normal((B, self.cap["csa"], s.D_I), sd(10), device)
        self.iq, self.iqs = synth.mxfp4_normal((T, B, Td, s.H_I, s.D_I), sd(11), device)
        if s.derive_keys:  # per-token indexer keys: the window's and each new token's
            if s.dyadic_keys:
                g = synth.generator(sd(12), device)
                grid = lambda shape: synth.bf16_bits(  # noqa: E731
                    torch.randint(-64, 65, shape, generator=g, device=device).to(torch.float32) / 16)
                ring_xk, self.xkn = grid((B, s.W, s.D_I)), grid((T, B, Td, s.D_I))
                self.ringz["csa"].zero_()
                self.zn["csa"].zero_()
            else:
                ring_xk = synth.normal_bf16_bits((B, s.W, s.D_I), 1.0, sd(12), device)
                self.xkn = synth.normal_bf16_bits((T, B, Td, s.D_I), 1.0, sd(13), device)
            self.ring_xk = self._to_ring(ring_xk, self.R["csa"])
        # per-step device scalars: the first draft position, every query's position and the
        # entries it sees, and the blocks each step completes (start position, entry index)
        rep = lambda a, dt: torch.from_numpy(np.ascontiguousarray(  # noqa: E731
            np.repeat(np.asarray(a)[:, None], B, 1).astype(dt))).to(device)
        self.pos = rep(t0, np.int64)                                          # [T, B]
        tq = t0[:, None] + np.arange(Td)[None, :]                             # [T, Td]
        self.qpos = torch.from_numpy(np.ascontiguousarray(
            np.repeat(tq[:, None, :], B, 1).astype(np.int64))).to(device)   # [T, B, Td]
        self.nent, self.blocks = {}, {}
        for name in ("csa", "hca"):
            m = self.m[name]
            self.nent[name] = torch.from_numpy(np.ascontiguousarray(
                np.repeat(((tq + 1) // m)[:, None, :], B, 1).astype(np.int32))).to(device)
            ends = [[int(e) for e in range(int(t0[i]), int(t0[i]) + Td) if (e + 1) % m == 0] for i in range(T)]
            flat = [e for es in ends for e in es]
            p0 = rep(np.array([e - m + 1 for e in flat], np.int64).reshape(-1), np.int64) if flat else None
            e0 = rep(np.array([(e + 1) // m - 1 for e in flat], np.int64), np.int32) if flat else None
            blocks, n = [], 0
            for i in range(T):
                blocks.append([((e - m + 1) % self.R[name], p0[n + u], e0[n + u]) for u, e in enumerate(ends[i])])
                n += len(ends[i])
            self.blocks[name] = blocks
        self.nvalid = self.nent["csa"]                                        # [T, B, Td]
        # outputs of every step (query rows b * Td + j)
        self.out = {n: torch.empty((T, B * Td, s.H, s.d_v), dtype=torch.int16, device=device) for n in ("csa", "hca")}
        self.lse = {n: torch.empty((T, B * Td, s.H), dtype=torch.float32, device=device) for n in ("csa", "hca")}
        self.topk = torch.empty((T, B, Td, s.k), dtype=torch.int32, device=device)
        # workspaces
        self.ws_idx = torch.empty(max(16, native.csa_index_topk_workspace_size(B, Td, self.cap["csa"], s.H_I, s.D_I,
                                                                                s.k)), dtype=torch.uint8, device=device)
        self.ws_att = {}
        for name in ("csa", "hca"):
            n = native.hybrid_attn_decode_workspace_size(B * Td, s.H, s.d_v, self.cap[name], s.k, s.W, name == "hca")
            self.ws_att[name] = torch.zeros(max(16, n), dtype=torch.uint8, device=device)
        # initial state, for restoring between runs
        self._init = {n: (self.ring[n].clone(), self.ringz[n].clone()) for n in ("csa", "hca")}
        if s.derive_keys:  # the loop overwrites the keys of new entries
            self._init["xk"] = self.ring_xk.clone()
            self._init["ik"] = (self.ik.clone(), self.iks.clone())

    def _to_ring(self, win, R):
        """Window rows of positions L-W .. L-1 ([B, W, ...]) placed at ring slots (position mod R)."""
        s = self.s
        if R == s.W and s.L % s.W == 0:
            return win
        ring = torch.zeros((win.shape[0], R) + tuple(win.shape[2:]), dtype=win.dtype, device=win.device)
        slots = torch.from_numpy((s.L - s.W + np.arange(s.W)) % R).to(win.device)
        ring[:, slots] = win
        return ring

    # ------------------------------------------------------------------ state
    def restore(self):
        """Put the windows back to their initial contents (entries past L are rewritten by the loop)."""
        for n in ("csa", "hca"):
            self.ring[n].copy_(self._init[n][0])
            self.ringz[n].copy_(self._init[n][1])
        if self.s.derive_keys:
            self.ring_xk.copy_(self._init["xk"])
            self.ik.copy_(self._init["ik"][0])
            self.iks.copy_(self._init["ik"][1])

    def host_state(self):
        """Host copies of the initial state and inputs (for the oracle). Per-step token inputs are
        [steps, B, draft, ...], without the draft axis for one-token steps."""
        h = lambda t: t.cpu().numpy()  # noqa: E731
        one = self.s.draft == 1
        hs = lambda t: h(t[:, :, 0] if one else t)  # noqa: E731
        st = {}
        for n in ("csa", "hca"):
            st[n] = dict(ring=h(self._init[n][0]).view(np.uint16), ringz=h(self._init[n][1]),
                         ckv=h(self.ckv[n]), scl=h(self.scl[n]), q=hs(self.q[n]).view(np.uint16),
                         xn=hs(self.xn[n]).view(np.uint16), zn=hs(self.zn[n]))
        st["ik"], st["iks"], st["iq"], st["iqs"] = h(self.ik), h(self.iks), h(self.iq), h(self.iqs)
        st["t0"], st["accepted"], st["R"] = self.t_host.copy(), self.accepted.copy(), dict(self.R)
        if self.s.derive_keys:
            st["ik"], st["iks"] = h(self._init["ik"][0]), h(self._init["ik"][1])
            st["ring_xk"], st["xkn"] = h(self._init["xk"]).view(np.uint16), hs(self.xkn).view(np.uint16)
        return st

    # ------------------------------------------------------------------ one step
    def step(self, i, stream=None, share=None, src=None, layers=("csa", "hca")):
        """Decode step i of both layers (draft tokens t0 .. t0 + draft - 1).

        layers: the layers whose calls are issued (both by default). The two layers of a pair
        share no buffer, so their calls may be issued on different streams.

        share (cross-layer index sharing of the CSA layer, with `src` another LayerPair of the
        same shapes that has already run step i):
          None      -- the CSA layer has its own KV, indexer keys and query (the default);
          "reuse"   -- its own KV, but no indexer call: it attends to src's top-k entries;
          "reindex" -- src's KV, window and indexer keys (no append or compression of its own),
                       with its own indexer query and hence its own top-k.
        """
        s = self.s
        B, D, W, Td = s.B, s.D, s.W, s.draft
        assert share in (None, "reuse", "reindex") and (share is None or src is not None)
        assert set(layers) <= {"csa", "hca"}
        kv = {"csa": src if share == "reindex" else self, "hca": self}
        fused = {}
        for name in layers:
            if kv[name] is not self:
                continue
            R, m = self.R[name], self.m[name]
            # the compression of a completed block reads the new tokens from the ring
            fused[name] = s.fuse_append and not self.blocks[name][i]
            if not fused[name]:
                native.cskv_ring_append(self.xn[name][i], self.zn[name][i], self.pos[i], self.ring[name],
                                        self.ringz[name], B, D, R, stream, T=Td)
            keys = name == "csa" and s.derive_keys
            if keys:
                native.cskv_ring_append(self.xkn[i], None, self.pos[i], self.ring_xk, None, B, s.D_I, R, stream, T=Td)
            fn = native.csa_compress if name == "csa" else native.hca_compress
            for slot0, p0, e0 in self.blocks[name][i]:
                fn(self.ring[name][:, slot0:], R * D, self.ringz[name][:, slot0:], R, p0, B, m, D,
                   s.d_rope, m, 0, s.rope_base, self.kv_code, self.ckv[name], self.scl[name],
                   self.cap[name], e0, stream, rms_eps=s.rms_eps)
                if keys:
                    native.csa_index_key_pool(self.ring_xk[:, slot0:], R * s.D_I, self.ringz[name][:, slot0:], R, B, m,
                                              s.D_I, m, self.ik, self.iks, self.cap[name], e0, stream)
        if "csa" not in layers:
            topk = None
        elif share == "reuse":
            topk = src.topk[i]
        else:
            ik = kv["csa"]
            native.csa_index_topk(self.iq[i], self.iqs[i], None, ik.ik, ik.iks, self.nvalid[i], B, Td,
                                  self.cap["csa"], s.H_I, s.D_I, s.k, self.topk[i], None, self.ws_idx, None, stream)
            topk = self.topk[i]
        for name in layers:
            c = kv[name]
            tk = topk if name == "csa" else None
            if fused.get(name):
                native.hybrid_attn_decode_append(self.q[name][i], self.qpos[i], c.ckv[name], c.scl[name],
                                                 self.attn_code, self.cap[name], self.nent[name][i], tk, s.k,
                                                 c.ring[name], c.ringz[name], self.xn[name][i], self.zn[name][i], W,
                                                 B, s.H, D, s.d_rope, s.d_v, s.rope_base, s.scale,
                                                 self.out[name][i], self.lse[name][i], self.ws_att[name], None,
                                                 stream, q_rms_eps=s.rms_eps, T=Td, R=c.R[name])
                continue
            native.hybrid_attn_decode(self.q[name][i], self.qpos[i], c.ckv[name], c.scl[name],
                                      self.attn_code, self.cap[name], self.nent[name][i],
                                      tk, s.k, c.ring[name], W, B, s.H, D,
                                      s.d_rope, s.d_v, s.rope_base, s.scale, self.out[name][i], self.lse[name][i],
                                      self.ws_att[name], None, stream, q_rms_eps=s.rms_eps, T=Td, R=c.R[name])

    def run(self, first, count, stream=None):
        for i in range(first, first + count):
            self.step(i, stream)

    # ------------------------------------------------------------------ accounting
    def step_bytes(self):
        """Algorithmic HBM bytes of one decode step (both layers), by component. A draft step reads
        each sequence's keys and entries once for all of its draft queries."""
        s = self.s
        n_c = self.n0["csa"]
        n_h = self.n0["hca"]
        Td = s.draft
        e = s.D // 2 + s.D // 32 if s.kv_dtype == "mxfp4" else s.D + 4   # stored entry bytes
        xi = s.D_I // 2 + s.D_I // 32        # MXFP4 key
        q = s.B * Td * s.H * s.D * 2
        o = s.B * Td * s.H * s.d_v * 2
        win = s.B * (s.W + Td - 1) * s.D * 2
        out = {
            "csa_index": s.B * n_c * xi + s.B * Td * s.H_I * xi + s.B * Td * s.k * 4,
            "csa_attn": s.B * Td * s.k * e + win + q + o + s.B * Td * s.k * 4,
            "hca_attn": s.B * n_h * e + win + q + o,
        }
        if s.derive_keys:  # key append (read + write) and, amortised over m steps, the pooling
            out["csa_keys"] = Td * (s.B * (2 * s.D_I * 2 + s.D_I * 2 + 4) + s.B * xi // s.m_csa)
        return out

    def step_flops(self):
        s = self.s
        n_c, n_h, Td = self.n0["csa"], self.n0["hca"], s.draft
        idx = 2 * s.B * Td * n_c * s.H_I * s.D_I
        att = lambda nk: 2 * s.B * Td * s.H * nk * (s.D + s.d_v)  # noqa: E731
        return {"csa_index": idx, "csa_attn": att(s.k + s.W), "hca_attn": att(n_h + s.W)}



def step_stack(pairs, i, share=None, side=None, split="chains"):
    """Decode step i of a stack of independent layer pairs, forked from the current stream.

    share: as in LayerPair.step, for pairs 1.. (pair 0 always indexes its own keys).
    side: None issues every call on the current stream, pair after pair. Otherwise a list of
    further streams, forked from the current stream at the start of the step and joined at its
    end. Under graph capture this records parallel branches per step.
    split: how the calls go to the streams --
      "chains": the pairs are cut into len(side) + 1 contiguous groups, one per stream, each
                group stepped pair after pair (CSA layer, then HCA layer), so every stream keeps
                the layer order of a model and the streams are independent micro-batches;
      "layers": (one side stream) the HCA layers of all pairs go to the side stream, beside the
                CSA layers (the HCA layer of a pair reads nothing its CSA layer writes).
    With share, pairs 1.. wait for pair 0's step before theirs.
    """
    shr = lambda p: None if p == 0 else share  # noqa: E731
    if not side:
        for p, pr in enumerate(pairs):
            pr.step(i, share=shr(p), src=pairs[0])
        return
    main = torch.cuda.current_stream()
    for st in side:
        st.wait_stream(main)
    if split == "layers":
        assert len(side) == 1 and share is None
        with torch.cuda.stream(side[0]):
            for pr in pairs:
                pr.step(i, layers=("hca",))
        for pr in pairs:
            pr.step(i, layers=("csa",))
    else:
        assert split == "chains"
        streams = [main] + list(side)
        n = len(streams)
        groups = [[p for p in range(len(pairs)) if p * n // len(pairs) == g] for g in range(n)]
        done0 = torch.cuda.Event() if share is not None else None
        for g, st in enumerate(streams):
            with torch.cuda.stream(st):
                for p in groups[g]:
                    if share is not None and p > 0 and g > 0:
                        st.wait_event(done0)
                    pairs[p].step(i, share=shr(p), src=pairs[0])
                    if p == 0 and done0 is not None:
                        done0.record(st)
    for st in side:
        main.wait_stream(st)
