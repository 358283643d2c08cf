"""Decode loop of one CSA layer and one HCA layer (interleaved 1:1) on the GPU.

Page "딥시크 V4 분석: CSA·HCA 어텐션으로 100만 토큰 컨텍스트를 저비용에 구현한 방법",
section "주요 인사이트": CSA and HCA layers alternate 1:1; section "쉽게 이해하기":
every layer keeps a window of the latest 128 tokens. Page "DeepSeek-V4가 이차적
어텐션 비용 없이 백만 토큰 컨텍스트를 달성하는 방법", section "두 가지 압축 전략:
CSA 및 HCA": CSA pools 4 tokens per entry and selects top-k with the FP4 indexer,
HCA pools 128 per entry and attends densely.

One decode step at position t (the same t for every sequence of the batch):
  1. each layer writes its new raw token and pooling logit to ring slot t mod W;
  2. if (t+1) % m == 0 the layer compresses ring slots of positions [t-m+1, t]
     (contiguous because m divides W) into entry (t+1)/m - 1;
  3. CSA: csa_index_topk over the visible entries, then hybrid_attn_decode on
     the selected entries + window; HCA: hybrid_attn_decode over all entries +
     window.
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
        assert s.L >= s.W
        sd = lambda t: synth.seed_of(s.seed, s.wid, t)  # noqa: E731
        B, D, T = s.B, s.D, s.steps
        self.n0 = {"csa": s.L // s.m_csa, "hca": s.L // s.m_hca}
        self.cap = {"csa": (s.L + T) // s.m_csa + 1, "hca": (s.L + T) // s.m_hca + 1}
        self.m = {"csa": s.m_csa, "hca": s.m_hca}
        self.ckv, self.scl, self.ring, self.ringz, self.q, self.xn, self.zn = {}, {}, {}, {}, {}, {}, {}
        for li, name in enumerate(("csa", "hca")):
            base = 100 * li
            c, sc = synth.fp8_rows_normal((B, self.cap[name], D), s.sigma, sd(base + 0), device)
            self.ckv[name], self.scl[name] = c, sc
            self.ring[name] = synth.normal_bf16_bits((B, s.W, D), s.sigma, sd(base + 1), device)
            self.ringz[name] = synth.normal((B, s.W), 1.0, sd(base + 2), device)
            self.q[name] = synth.normal_bf16_bits((T, B, s.H, D), s.sigma, sd(base + 3), device)
            self.xn[name] = synth.normal_bf16_bits((T, B, D), s.sigma, sd(base + 4), device)
            self.zn[name] = synth.normal((T, B), 1.0, sd(base + 5), device)
        # indexer keys of every entry (without derive_keys, future entries' keys are inputs too)
        # and queries
        self.ik, self.iks = synth.mxfp4_normal((B, self.cap["csa"], s.D_I), sd(10), device)
        self.iq, self.iqs = synth.mxfp4_normal((T, B, 1, s.H_I, s.D_I), sd(11), device)
        if s.derive_keys:  # per-token indexer keys: the window's and each new token's
            if s.dyadic_keys:
                g = synth.generator(sd(12), device)
                grid = lambda shape: synth.bf16_bits(  # noqa: E731
                    torch.randint(-64, 65, shape, generator=g, device=device).to(torch.float32) / 16)
                self.ring_xk, self.xkn = grid((B, s.W, s.D_I)), grid((T, B, s.D_I))
                self.ringz["csa"].zero_()
                self.zn["csa"].zero_()
            else:
                self.ring_xk = synth.normal_bf16_bits((B, s.W, s.D_I), 1.0, sd(12), device)
                self.xkn = synth.normal_bf16_bits((T, B, s.D_I), 1.0, sd(13), device)
        # per-step device scalars
        t = s.L + np.arange(T, dtype=np.int64)
        self.t_host = t
        self.pos = torch.from_numpy(np.repeat(t[:, None], B, 1)).to(device)
        self.nent, self.pos0c, self.entry0 = {}, {}, {}
        for name in ("csa", "hca"):
            m = self.m[name]
            n_after = (t + 1) // m
            self.nent[name] = torch.from_numpy(np.repeat(n_after[:, None].astype(np.int32), B, 1)).to(device)
            self.pos0c[name] = torch.from_numpy(np.repeat((t - m + 1)[:, None], B, 1)).to(device)
            self.entry0[name] = torch.from_numpy(np.repeat((n_after - 1)[:, None].astype(np.int32), B, 1)).to(device)
        self.nvalid = self.nent["csa"].view(T, B, 1)
        # outputs of every step
        self.out = {n: torch.empty((T, B, s.H, s.d_v), dtype=torch.int16, device=device) for n in ("csa", "hca")}
        self.lse = {n: torch.empty((T, B, s.H), dtype=torch.float32, device=device) for n in ("csa", "hca")}
        self.topk = torch.empty((T, B, 1, s.k), dtype=torch.int32, device=device)
        # workspaces
        self.ws_idx = torch.empty(max(16, native.csa_index_topk_workspace_size(B, 1, self.cap["csa"], s.H_I, s.D_I, s.k)),
                                  dtype=torch.uint8, device=device)
        self.ws_att = {}
        for name in ("csa", "hca"):
            n = native.hybrid_attn_decode_workspace_size(B, s.H, s.d_v, self.cap[name], s.k, s.W, name == "hca")
            self.ws_att[name] = torch.empty(max(16, n), dtype=torch.uint8, device=device)
        # initial state, for restoring between runs
        self._init = {n: (self.ring[n].clone(), self.ringz[n].clone()) for n in ("csa", "hca")}
        if s.derive_keys:  # the loop overwrites the keys of new entries
            self._init["xk"] = self.ring_xk.clone()
            self._init["ik"] = (self.ik.clone(), self.iks.clone())

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
        """Host copies of the initial state and inputs (for the oracle)."""
        h = lambda t: t.cpu().numpy()  # noqa: E731
        st = {}
        for n in ("csa", "hca"):
            st[n] = dict(ring=h(self._init[n][0]).view(np.uint16), ringz=h(self._init[n][1]),
                         ckv=h(self.ckv[n]), scl=h(self.scl[n]), q=h(self.q[n]).view(np.uint16),
                         xn=h(self.xn[n]).view(np.uint16), zn=h(self.zn[n]))
        st["ik"], st["iks"], st["iq"], st["iqs"] = h(self.ik), h(self.iks), h(self.iq), h(self.iqs)
        if self.s.derive_keys:
            st["ik"], st["iks"] = h(self._init["ik"][0]), h(self._init["ik"][1])
            st["ring_xk"], st["xkn"] = h(self._init["xk"]).view(np.uint16), h(self.xkn).view(np.uint16)
        return st

    # ------------------------------------------------------------------ one step
    def step(self, i, stream=None, share=None, src=None):
        """Decode step i of both layers.

        share (cross-layer index sharing of the CSA layer, with `src` another LayerPair of the
        same shapes that has already run step i):
          None      -- the CSA layer has its own KV, indexer keys and query (the default);
          "reuse"   -- its own KV, but no indexer call: it attends to src's top-k entries;
          "reindex" -- src's KV, window and indexer keys (no append or compression of its own),
                       with its own indexer query and hence its own top-k.
        """
        s = self.s
        B, D, W = s.B, s.D, s.W
        t = int(self.t_host[i])
        assert share in (None, "reuse", "reindex") and (share is None or src is not None)
        kv = {"csa": src if share == "reindex" else self, "hca": self}
        for name in ("csa", "hca"):
            if kv[name] is not self:
                continue
            native.cskv_ring_append(self.xn[name][i], self.zn[name][i], self.pos[i], self.ring[name],
                                    self.ringz[name], B, D, W, stream)
            keys = name == "csa" and s.derive_keys
            if keys:
                native.cskv_ring_append(self.xkn[i], None, self.pos[i], self.ring_xk, None, B, s.D_I, W, stream)
            m = self.m[name]
            if (t + 1) % m == 0:
                slot0 = (t - m + 1) % W
                fn = native.csa_compress if name == "csa" else native.hca_compress
                fn(self.ring[name][:, slot0:], W * D, self.ringz[name][:, slot0:], W, self.pos0c[name][i], B, m, D,
                   s.d_rope, m, 0, s.rope_base, native.CSKV_FP8_E4M3, self.ckv[name], self.scl[name],
                   self.cap[name], self.entry0[name][i], stream, rms_eps=s.rms_eps)
                if keys:
                    native.csa_index_key_pool(self.ring_xk[:, slot0:], W * s.D_I, self.ringz[name][:, slot0:], W, B, m,
                                              s.D_I, m, self.ik, self.iks, self.cap[name], self.entry0[name][i], stream)
        if share == "reuse":
            topk = src.topk[i]
        else:
            ik = kv["csa"]
            native.csa_index_topk(self.iq[i], self.iqs[i], None, ik.ik, ik.iks, self.nvalid[i], B, 1,
                                  self.cap["csa"], s.H_I, s.D_I, s.k, self.topk[i], None, self.ws_idx, None, stream)
            topk = self.topk[i]
        for name in ("csa", "hca"):
            c = kv[name]
            native.hybrid_attn_decode(self.q[name][i], self.pos[i], c.ckv[name], c.scl[name],
                                      native.CSKV_FP8_E4M3, self.cap[name], self.nent[name][i],
                                      topk if name == "csa" else None, s.k, c.ring[name], W, B, s.H, D,
                                      s.d_rope, s.d_v, s.rope_base, s.scale, self.out[name][i], self.lse[name][i],
                                      self.ws_att[name], None, stream, q_rms_eps=s.rms_eps)

    def run(self, first, count, stream=None):
        for i in range(first, first + count):
            self.step(i, stream)

    # ------------------------------------------------------------------ accounting
    def step_bytes(self):
        """Algorithmic HBM bytes of one decode step (both layers), by component."""
        s = self.s
        n_c = self.n0["csa"]
        n_h = self.n0["hca"]
        e = s.D + 4                          # fp8 entry + fp32 scale
        xi = s.D_I // 2 + s.D_I // 32        # MXFP4 key
        q = s.B * s.H * s.D * 2
        o = s.B * s.H * s.d_v * 2
        win = s.B * s.W * s.D * 2
        out = {
            "csa_index": s.B * n_c * xi + s.B * s.H_I * xi + s.B * s.k * 4,
            "csa_attn": s.B * s.k * e + win + q + o + s.B * s.k * 4,
            "hca_attn": s.B * n_h * e + win + q + o,
        }
        if s.derive_keys:  # key append (read + write) and, amortised over m steps, the pooling
            out["csa_keys"] = s.B * (2 * s.D_I * 2 + s.D_I * 2 + 4) + s.B * xi // s.m_csa
        return out

    def step_flops(self):
        s = self.s
        n_c, n_h = self.n0["csa"], self.n0["hca"]
        idx = 2 * s.B * n_c * s.H_I * s.D_I
        att = lambda nk: 2 * s.B * s.H * nk * (s.D + s.d_v)  # noqa: E731
        return {"csa_index": idx, "csa_attn": att(s.k + s.W), "hca_attn": att(n_h + s.W)}
