"""GPU checks of hybrid_attn_decode_append: the state update of a decode step fused into its
attention call must equal cskv_ring_append followed by hybrid_attn_decode, bit for bit (outputs,
lse, and the ring rows and pooling logits it writes), on both attention kernels."""
import numpy as np
import pytest
import torch

from compressed_sparse_kv_03_amd import native, synth
from tests.gpu_util import DEV, poisoned, say, up

pytestmark = pytest.mark.gpu

DT = {"bf16": native.CSKV_BF16, "fp8": native.CSKV_FP8_E4M3, "mxfp4": native.CSKV_MXFP4}


@pytest.fixture(params=[native.ATTN_G64, native.ATTN_G16], ids=["g64", "g16"])
def kernel_path(request):
    native.cskv_attn_path(request.param)
    yield request.param
    native.cskv_attn_path(native.ATTN_AUTO)


CASES = [
    # B, T, H, D, d_rope, d_v, N, k, W, R, dtype
    (3, 1, 64, 576, 64, 512, 700, 128, 128, 128, "fp8"),      # CSA-like gather, one-token step
    (3, 1, 64, 576, 64, 512, 300, 0, 128, 128, "fp8"),        # HCA-like dense
    (2, 3, 64, 576, 64, 512, 400, 64, 128, 132, "bf16"),      # 3-token draft, ring of W + 4 slots
    (2, 4, 20, 128, 64, 128, 90, 16, 8, 12, "mxfp4"),         # ragged heads, short window, draft
    (2, 2, 16, 128, 64, 128, 200, 32, 0, 4, "bf16"),          # no window: the append still happens
    (2, 5, 16, 128, 64, 128, 60, 0, 16, 20, "fp8"),           # the draft reaches across a ring wrap
]


def entries(dtype, B, N, D, seed):
    if dtype == "bf16":
        return synth.normal_bf16_bits((B, N, D), D ** -0.5, seed, DEV), None
    if dtype == "fp8":
        return synth.fp8_rows_normal((B, N, D), D ** -0.5, seed, DEV)
    return synth.mxfp4_rows_normal((B, N, D), D ** -0.5, seed, DEV)


@pytest.mark.parametrize("B,T,H,D,d_rope,d_v,N,k,W,R,dtype", CASES)
def test_decode_append_matches_append_then_decode(B, T, H, D, d_rope, d_v, N, k, W, R, dtype, kernel_path):
    say("decode append", B, T, H, D, d_rope, d_v, N, k, W, R, dtype, "path", kernel_path)
    sd = lambda t: synth.seed_of(7, 61, t)  # noqa: E731
    rng = np.random.default_rng(61)
    q = synth.normal_bf16_bits((B * T, H, D), D ** -0.5, sd(0), DEV)
    ckv, sc = entries(dtype, B, N, D, sd(1))
    ring = synth.normal_bf16_bits((B, R, D), D ** -0.5, sd(2), DEV)
    ringz = synth.normal((B, R), 1.0, sd(3), DEV)
    x_new = synth.normal_bf16_bits((B, T, D), D ** -0.5, sd(4), DEV)
    z_new = synth.normal((B, T), 1.0, sd(5), DEV)
    t0 = 4 * N + rng.integers(0, 3 * R, B)        # positions past every entry, ring offsets vary
    if T == 5:
        t0 = (np.arange(B) + 1) * R - 2              # the draft's slots wrap around the ring end
    qpos = (t0[:, None] + np.arange(T)[None, :]).reshape(-1)
    nent = np.minimum(N, (qpos + 1) // 4 - rng.integers(0, 3, B * T)).astype(np.int32)
    topk = None
    if k:
        tk = np.stack([rng.permutation(int(n))[:k] if n >= k else
                       np.concatenate([rng.permutation(int(n)), -np.ones(k - int(n), np.int64)]) for n in nent])
        tk[:, ::7] = -1
        topk = up(tk.astype(np.int32))
    pos = up(t0.astype(np.int64))
    qp, ne = up(qpos.astype(np.int64)), up(nent)
    wsn = native.hybrid_attn_decode_workspace_size(B * T, H, d_v, N, k, W, topk is None)
    ws = torch.zeros(max(wsn, 16), dtype=torch.uint8, device=DEV)
    # reference: append, then attend over the updated ring
    ring_a, ringz_a = ring.clone(), ringz.clone()
    out_a, lse_a = poisoned((B * T, H, d_v), torch.int16), poisoned((B * T, H), torch.float32)
    native.cskv_ring_append(x_new, z_new, pos, ring_a, ringz_a, B, D, R, T=T)
    native.hybrid_attn_decode(q, qp, ckv, sc, DT[dtype], N, ne, topk, max(k, 1), ring_a, W, B, H, D, d_rope, d_v,
                              10000.0, D ** -0.5, out_a, lse_a, ws, T=T, R=R)
    # fused
    ring_f, ringz_f = ring.clone(), ringz.clone()
    out_f, lse_f = poisoned((B * T, H, d_v), torch.int16), poisoned((B * T, H), torch.float32)
    native.hybrid_attn_decode_append(q, qp, ckv, sc, DT[dtype], N, ne, topk, max(k, 1), ring_f, ringz_f, x_new,
                                     z_new, W, B, H, D, d_rope, d_v, 10000.0, D ** -0.5, out_f, lse_f, ws, T=T, R=R)
    torch.cuda.synchronize()
    assert torch.equal(out_f, out_a), "output differs from append + decode"
    assert torch.equal(lse_f, lse_a), "lse differs from append + decode"
    assert torch.equal(ring_f, ring_a), "ring rows differ from cskv_ring_append's"
    assert torch.equal(ringz_f, ringz_a), "ring pooling logits differ from cskv_ring_append's"
    assert not torch.equal(ring_f, ring) or T == 0
