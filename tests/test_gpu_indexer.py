"""GPU parity of csa_index_topk: bit-exact indices (order included) and exact scores."""
import numpy as np
import pytest
import torch

from compressed_sparse_kv_03_amd import configs, native, synth
from oracle import indexer as oidx
from oracle import topk as otopk
from tests import parity
from tests.gpu_util import DEV, down, poisoned, say, up

pytestmark = pytest.mark.gpu


def run_index(iq, iqs, ik, iks, n_valid, k, head_w=None):
    B, T, H_I, half = iq.shape
    N_cap = ik.shape[1]
    D_I = half * 2
    ws_n = native.csa_index_topk_workspace_size(B, T, N_cap, H_I, D_I, k)
    ws = torch.zeros(max(ws_n, 16), dtype=torch.uint8, device=DEV)
    oi = poisoned((B, T, k), torch.int32)
    os_ = poisoned((B, T, k), torch.float32)
    native.csa_index_topk(iq, iqs, head_w, ik, iks, n_valid, B, T, N_cap, H_I, D_I, k, oi, os_, ws)
    return oi, os_


def check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_, head_w=None, rows=None):
    iqh, iqsh, ikh, iksh, nvh = down(iq), down(iqs), down(ik), down(iks), down(nv)
    hwh = None if head_w is None else down(head_w)
    oih, osh = down(oi), down(os_)
    B, T = nvh.shape
    for b in range(B):
        ts = range(T) if rows is None else rows
        for t in ts:
            sc = oidx.scores(iqh[b, t][None], iqsh[b, t][None], ikh[b], iksh[b], nvh[b, t][None],
                             None if hwh is None else hwh[b, t][None])
            idx, s = otopk.topk(sc, k)
            parity.topk_exact(oih[b, t], idx[0], f"top-k b={b} t={t}")
            assert np.array_equal(osh[b, t], s[0]), f"scores differ b={b} t={t}"


@pytest.mark.parametrize("H_I,D_I,k,N_cap", [(8, 128, 128, 5000), (4, 64, 128, 1024), (3, 32, 16, 333),
                                             (16, 256, 300, 9000), (8, 512, 1, 2100), (5, 160, 1024, 20000)])
def test_index_topk_small(H_I, D_I, k, N_cap):
    say("index small", H_I, D_I, k, N_cap)
    B, T = 2, 3
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 101 + D_I, DEV)
    ik, iks = synth.mxfp4_normal((B, N_cap, D_I), 102 + D_I, DEV)
    nv = up(np.array([[N_cap, N_cap // 3, 0], [17, min(k, N_cap), N_cap - 1]], np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_)


def test_index_topk_head_weights_and_negative_scores():
    say("index head weights")
    B, T, H_I, D_I, N, k = 1, 2, 8, 128, 3000, 64
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 111, DEV)
    ik, iks = synth.mxfp4_normal((B, N, D_I), 112, DEV)
    hw = up(np.array([[[1, -2, 0.5, -1, 4, 0.25, -0.5, 2]] * T], np.float32))
    nv = up(np.array([[N, 2000]], np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k, hw)
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_, head_w=hw)


def test_index_topk_ties_go_to_the_lower_index():
    """Keys drawn from 5 distinct patterns: scores collide massively; order must follow the index."""
    say("index ties")
    B, T, H_I, D_I, N, k = 2, 2, 8, 128, 7000, 256
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 121, DEV)
    base, bsc = synth.mxfp4_normal((5, D_I), 122, DEV)
    pick = torch.from_numpy(np.random.default_rng(0).integers(0, 5, (B, N))).to(DEV)
    ik, iks = base[pick].contiguous(), bsc[pick].contiguous()
    ik[1].zero_()                                   # sequence 1: every score is 0
    nv = up(np.array([[N, 300], [N, 5]], np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_)
    assert down(oi)[1, 0].tolist()[:10] == list(range(10))


@pytest.mark.parametrize("wname", ["c1_csa_tiny", "c2_csa_b32_64k"])
def test_index_topk_workload(wname):
    w = configs.ALL[wname]
    say("index", w.name)
    n = w.L // w.m
    iq, iqs = synth.mxfp4_normal((w.B, 1, w.H_I, w.D_I), synth.seed_of(0, w.wid, 10), DEV)
    ik, iks = synth.mxfp4_normal((w.B, n, w.D_I), synth.seed_of(0, w.wid, 11), DEV)
    nv = up(np.full((w.B, 1), n, np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, w.k)
    check_against_oracle(iq, iqs, ik, iks, nv, w.k, oi, os_)


def test_index_topk_hybrid_1m_shape():
    """The CSA layer of the 1M hybrid pair: 8 queries over 262144 entries each (one decode step)."""
    w = configs.C5
    say("index", w.name)
    n = w.L // w.m
    iq, iqs = synth.mxfp4_normal((w.B, 1, w.H_I, w.D_I), synth.seed_of(0, w.wid, 10), DEV)
    ik, iks = synth.mxfp4_normal((w.B, n + 64, w.D_I), synth.seed_of(0, w.wid, 11), DEV)
    nv = up(np.full((w.B, 1), n, np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, w.k)
    check_against_oracle(iq, iqs, ik, iks, nv, w.k, oi, os_)


def test_index_topk_many_queries_causal():
    """A causal prompt (n_valid = floor((t+1)/4)) with enough queries to take the query-parallel path."""
    say("index many queries causal")
    T, H_I, D_I, k = 4200, 8, 128, 128
    N = 16384
    iq, iqs = synth.mxfp4_normal((1, T, H_I, D_I), 131, DEV)
    ik, iks = synth.mxfp4_normal((1, N, D_I), 132, DEV)
    t0 = 4 * N - T                                   # last row sees all N entries
    nv = up(((np.arange(T) + t0 + 1) // 4).astype(np.int32)[None])
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    rows = sorted(set(np.random.default_rng(0).integers(0, T, 40).tolist()) | {0, T - 1})
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_, rows=rows)


def test_index_topk_when_the_sample_overstates_the_top():
    """Ten identical high-scoring keys sit on sampled entries (one at the start of each of the
    first ten sampled runs): the sampled bound admits fewer than k keys, so the exact fallback
    must produce the answer."""
    say("index sampled-bound fallback")
    B, H_I, D_I, k, N = 2, 8, 128, 128, 262144
    iq, iqs = synth.mxfp4_normal((B, 1, H_I, D_I), 141, DEV)
    ik, iks = synth.mxfp4_normal((B, N, D_I), 142, DEV)
    stride = N // 64                                  # sampled runs of 16 start at r * N / 64
    for b in range(B):
        for i in range(10):
            ik[b, i * stride] = iq[b, 0, 0]           # key = head-0 query codes: large positive dot
            iks[b, i * stride] = iqs[b, 0, 0]
    nv = up(np.full((B, 1), N, np.int32))
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_)
    got = down(oi)[:, 0]
    assert all(set(range(0, 10 * stride, stride)) <= set(got[b].tolist()) for b in range(B))


@pytest.mark.parametrize("B,T,H_I,D_I,k,N,ties", [
    (2, 150, 8, 128, 128, 3000, False),    # two queries per MFMA row tile; ragged last query block
    (1, 300, 16, 256, 64, 2500, False),    # one query per row tile, two 128-wide k steps
    (1, 270, 5, 160, 16, 1100, False),     # partial second k step, 5 heads
    (1, 260, 4, 512, 1, 700, False),       # four k steps, k = 1
    (2, 200, 8, 128, 100, 9000, True),     # massive score ties, several entry chunks
])
def test_index_topk_query_blocks(B, T, H_I, D_I, k, N, ties):
    """Many queries per call (the query-block path): every row bit-exact, arbitrary n_valid."""
    say("index query blocks", B, T, H_I, D_I, k, N, ties)
    rng = np.random.default_rng(T + D_I)
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 151 + D_I, DEV)
    if ties:
        base, bsc = synth.mxfp4_normal((6, D_I), 152, DEV)
        pick = torch.from_numpy(rng.integers(0, 6, (B, N))).to(DEV)
        ik, iks = base[pick].contiguous(), bsc[pick].contiguous()
    else:
        ik, iks = synth.mxfp4_normal((B, N, D_I), 153 + D_I, DEV)
    nvh = rng.integers(0, N + 1, (B, T)).astype(np.int32)
    nvh[:, :3] = [0, 1, min(k, N)]
    hw = None
    if ties:
        hw = up(rng.choice(np.array([1.0, -1.0, 0.5, 2.0], np.float32), (B, T, H_I)))
    oi, os_ = run_index(iq, iqs, ik, iks, up(nvh), k, hw)
    check_against_oracle(iq, iqs, ik, iks, up(nvh), k, oi, os_, head_w=hw)


@pytest.mark.parametrize("B,T,N,k,ties", [(1, 300, 1024, 128, False), (1, 300, 1024, 128, True),
                                          (2, 150, 1000, 128, False)])
def test_index_topk_query_blocks_single_chunk_k128(B, T, N, k, ties):
    """Few query blocks over at most 1024 entries: the query-block kernel takes one entry chunk and
    writes each row's ordered top-k itself (no merge kernel), after many reductions of the per-query
    candidate buffers (k = 128 of up to 1024 visible entries). Every row bit-exact."""
    say("index query blocks single chunk", B, T, N, k, ties)
    rng = np.random.default_rng(T + N)
    iq, iqs = synth.mxfp4_normal((B, T, 8, 128), 161, DEV)
    if ties:
        base, bsc = synth.mxfp4_normal((4, 128), 162, DEV)
        pick = torch.from_numpy(rng.integers(0, 4, (B, N))).to(DEV)
        ik, iks = base[pick].contiguous(), bsc[pick].contiguous()
    else:
        ik, iks = synth.mxfp4_normal((B, N, 128), 163, DEV)
    nvh = np.minimum(N, (np.arange(T)[None, :] * 7 + 3 + 11 * np.arange(B)[:, None])).astype(np.int32)
    nvh[:, :3] = [0, 1, k]
    oi, os_ = run_index(iq, iqs, ik, iks, up(nvh), k)
    check_against_oracle(iq, iqs, ik, iks, up(nvh), k, oi, os_)


def test_index_topk_query_blocks_many_rows_single_chunk():
    """16384 causal queries over 8192 entries: enough query blocks that each takes the whole entry
    range in one chunk (64 tiles, the c4 prefill's regime at a quarter of its length). 512 rows
    against the oracle, and every row against the decode kernels (calls of 256 queries)."""
    say("index query blocks many rows")
    T, N, k = 16384, 8192, 128
    iq, iqs = synth.mxfp4_normal((1, T, 8, 128), 171, DEV)
    ik, iks = synth.mxfp4_normal((1, N, 128), 172, DEV)
    nvh = ((np.arange(T) + 1) // 2).clip(max=N).astype(np.int32)[None]
    nv = up(nvh)
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    rows = sorted(set(np.random.default_rng(1).choice(T, 500, replace=False).tolist()) | {0, 1, 2, 255, 256, T - 1})
    check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_, rows=rows)
    ref, _ = run_index(iq[:, :256], iqs[:, :256], ik, iks, nv[:, :256], k)
    bad = 0
    for t0 in range(0, T, 256):
        r, _ = run_index(iq[:, t0:t0 + 256], iqs[:, t0:t0 + 256], ik, iks, nv[:, t0:t0 + 256], k)
        bad += int((r[0] != oi[0, t0:t0 + 256]).any(dim=1).sum().item())
    assert bad == 0, f"{bad} rows differ from the decode kernels"


def test_index_topk_workspace_reuse():
    """Decode-path calls in a row on one workspace, which carries nothing from one call to the
    next: different inputs and visible counts per call (one sequence seeing a single entry), every
    call checked."""
    say("index workspace reuse")
    B, T, H_I, D_I, N, k = 8, 1, 8, 128, 40000, 128
    ws = torch.empty(max(16, native.csa_index_topk_workspace_size(B, T, N, H_I, D_I, k)), dtype=torch.uint8,
                     device=DEV)
    for call, (seed, n_lo) in enumerate(((121, 30000), (122, 1), (123, 39000))):
        iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), seed, DEV)
        ik, iks = synth.mxfp4_normal((B, N, D_I), seed + 10, DEV)
        nv = up(np.linspace(n_lo, N, B).astype(np.int32).reshape(B, T))
        oi, os_ = poisoned((B, T, k), torch.int32), poisoned((B, T, k), torch.float32)
        native.csa_index_topk(iq, iqs, None, ik, iks, nv, B, T, N, H_I, D_I, k, oi, os_, ws)
        check_against_oracle(iq, iqs, ik, iks, nv, k, oi, os_, rows=[0])


@pytest.mark.parametrize("B,T,k,N,ties", [
    (3, 5, 128, 20000, False),   # query groups of 4 and 1 (three padding queries), several chunks
    (2, 2, 256, 9000, True),     # groups of 2, massive score ties
    (4, 3, 16, 3000, False),     # one padding query per group, chunks of a few hundred entries
    (1, 6, 1, 70000, True),      # k = 1, ties, chunks of 280 entries
])
def test_index_topk_draft_queries(B, T, k, N, ties):
    """Draft steps (T queries per sequence, each with its own visible count): one key stream per
    group of queries (kernel M). Every row bit-exact against the oracle, scores included."""
    say("index draft queries", B, T, k, N, ties)
    rng = np.random.default_rng(7 * T + k)
    H_I, D_I = 8, 128
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 171 + T, DEV)
    if ties:
        base, bsc = synth.mxfp4_normal((4, D_I), 172, DEV)
        pick = torch.from_numpy(rng.integers(0, 4, (B, N))).to(DEV)
        ik, iks = base[pick].contiguous(), bsc[pick].contiguous()
    else:
        ik, iks = synth.mxfp4_normal((B, N, D_I), 173 + T, DEV)
    # causal visibility inside the draft: nondecreasing along t, one sequence short of k
    nvh = np.sort(rng.integers(N // 2, N + 1, (B, T)), axis=1).astype(np.int32)
    nvh[0] = np.minimum(nvh[0], np.arange(T) * max(1, k // 3))
    hw = up(rng.choice(np.array([1.0, -1.0, 0.5, 2.0], np.float32), (B, T, H_I))) if ties else None
    oi, os_ = run_index(iq, iqs, ik, iks, up(nvh), k, hw)
    check_against_oracle(iq, iqs, ik, iks, up(nvh), k, oi, os_, head_w=hw)


def test_index_topk_draft_queries_1m_shape():
    """Four draft queries per sequence at the 1M-context decode shape (8 x 262144 entries): every
    row equal to the single-query path's (one call per draft position), two rows against the
    oracle."""
    say("index draft 1m")
    B, T, H_I, D_I, N, k = 8, 4, 8, 128, 262144, 128
    iq, iqs = synth.mxfp4_normal((B, T, H_I, D_I), 181, DEV)
    ik, iks = synth.mxfp4_normal((B, N, D_I), 182, DEV)
    nvh = (N - 64 + np.arange(T)[None, :] * 16 + np.zeros((B, 1), np.int64)).astype(np.int32)
    nv = up(nvh)
    oi, os_ = run_index(iq, iqs, ik, iks, nv, k)
    for t in range(T):
        oi1, os1 = run_index(iq[:, t:t + 1].contiguous(), iqs[:, t:t + 1].contiguous(), ik, iks,
                             nv[:, t:t + 1].contiguous(), k)
        assert torch.equal(oi[:, t], oi1[:, 0]), f"draft position {t}: indices differ from the single-query path"
        assert torch.equal(os_[:, t].view(torch.int32), os1[:, 0].view(torch.int32)), f"draft position {t}: scores differ"
    torch.cuda.synchronize()
    iqh, iqsh, ikh, iksh, oih = down(iq), down(iqs), down(ik), down(iks), down(oi)
    for b, t in ((0, 0), (7, 3)):
        sc = oidx.scores(iqh[b, t][None], iqsh[b, t][None], ikh[b], iksh[b], nvh[b, t][None])
        parity.topk_exact(oih[b, t], otopk.topk(sc, k)[0][0], f"draft 1m b={b} t={t}")
