"""The CSA prefill pipeline on one prompt: compression, causal indexer + top-k, attention.

The 128K-token prompt workload (c4 in configs.py): x [L, D] raw bf16 tokens and their
pooling logits z [L] are compressed into L/m bf16 entries; every position t scores the
entries visible to it (j < (t+1)/m) with its MXFP4 indexer query and keeps the top k;
then every position attends to its k entries plus the causal window of W raw tokens.
Inputs are seeded synthetic tensors (synth.py), resident on the device.
"""
import numpy as np
import torch

from . import configs, native, synth


class CsaPrefill:
    """Device buffers and the three calls of one prefill; `w` is a csa_prefill workload."""

    def __init__(self, w=configs.C4, device="cuda", seed=0):
        assert w.kind == "csa_prefill" and w.L % w.m == 0
        self.w = w
        L, D, m = w.L, w.D, w.m
        self.N = N = L // m
        sid = lambda t: synth.seed_of(seed, w.wid, t)  # noqa: E731
        self.x = synth.normal_bf16_bits((L, D), w.sigma, sid(1), device)
        self.z = synth.normal((1, L), 1.0, sid(2), device)
        self.iq, self.iqs = synth.mxfp4_normal((1, L, w.H_I, w.D_I), sid(3), device)
        self.ik, self.iks = synth.mxfp4_normal((1, N, w.D_I), sid(4), device)
        self.q = synth.normal_bf16_bits((L, w.H, D), w.sigma, sid(5), device)
        self.pos0 = torch.zeros(1, dtype=torch.int64, device=device)
        self.nv = ((torch.arange(L, device=device, dtype=torch.int64) + 1) // m).to(torch.int32).view(1, L)
        self.ckv = torch.empty((N, D), dtype=torch.int16, device=device)
        self.idx = torch.empty((1, L, w.k), dtype=torch.int32, device=device)
        self.out = torch.empty((L, w.H, w.d_v), dtype=torch.int16, device=device)
        self.lse = torch.empty((L, w.H), dtype=torch.float32, device=device)
        self.ws_idx = torch.empty(max(16, native.csa_index_topk_workspace_size(1, L, N, w.H_I, w.D_I, w.k)),
                                  dtype=torch.uint8, device=device)
        self.ws_att = torch.zeros(max(16, native.hybrid_attn_prefill_workspace_size(L, w.H, w.d_v, N, w.k, w.W, 0)),
                                  dtype=torch.uint8, device=device)

    def compress(self, stream=None):
        w = self.w
        native.csa_compress(self.x, w.L * w.D, self.z, w.L, self.pos0, 1, w.L, w.D, w.d_rope, w.m, 0, w.rope_base,
                            native.CSKV_BF16, self.ckv, None, self.N, None, stream)

    def index(self, stream=None):
        w = self.w
        native.csa_index_topk(self.iq, self.iqs, None, self.ik, self.iks, self.nv, 1, w.L, self.N, w.H_I, w.D_I,
                              w.k, self.idx, None, self.ws_idx, None, stream)

    def attend(self, stream=None):
        w = self.w
        native.hybrid_attn_prefill(self.q, 0, w.L, self.ckv, None, native.CSKV_BF16, self.N, self.idx[0], w.k,
                                   self.x, w.W, w.H, w.D, w.d_rope, w.d_v, w.m, w.rope_base, w.softmax_scale,
                                   self.out, self.lse, self.ws_att, None, stream)

    # ------------------------------------------------------------------ accounting
    def work(self):
        """Algorithmic bytes and flops of each call (causal counts, not the padded ones)."""
        w = self.w
        L, D, N, m = w.L, w.D, self.N, w.m
        xi = w.D_I // 2 + w.D_I // 32
        pairs_idx = sum_visible(L, m)                     # (t, j) pairs scored
        pairs_att = att_pairs(L, m, w.k, w.W)
        return {
            "compress": {"bytes": L * (2 * D + 4) + N * 2 * D},
            "index": {"flops": 2 * pairs_idx * w.H_I * w.D_I,
                      "bytes": L * w.H_I * xi + N * xi + L * w.k * 4},
            "attend": {"flops": 2 * pairs_att * w.H * (D + w.d_v),
                       "bytes": L * w.H * D * 2 + L * w.H * w.d_v * 2 + L * w.k * 4 + N * 2 * D + L * 2 * D},
        }


def sum_visible(L, m):
    """sum over t < L of floor((t + 1) / m)."""
    n = np.arange(1, L + 1, dtype=np.int64) // m
    return int(n.sum())


def att_pairs(L, m, k, W):
    """sum over t < L of the keys position t attends to: min(k, visible entries) + window."""
    t = np.arange(L, dtype=np.int64)
    return int(np.minimum(k, (t + 1) // m).sum() + np.minimum(W, t + 1).sum())


def scaled(w, L):
    """The prefill workload at another prompt length (same structure)."""
    assert L % w.m == 0 and L >= w.m
    return configs.small(w, L=L)
