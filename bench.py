"""Benchmark: hybrid CSA+HCA attention decode at 1M context on one MI355X.

Workload (the 1M-context hybrid layer pair): batch 8, context 2^20, one CSA
layer (m=4, top-k 128, MXFP4 indexer 8x128) and one HCA layer (m=128, dense),
64 query heads on one shared KV head of 512+64 dims, fp8 compressed caches with
per-entry scales, bf16 128-token windows; every decode step appends a token to
each layer and re-compresses every m tokens. A "step" is one decode step of the
layer pair for the whole batch (8 tokens). Inputs are synthetic and resident
in HBM before timing starts.

So that every step reads its caches from HBM rather than from the 256 MB
Infinity Cache (one pair's per-step working set, ~186 MB, would fit in it), the
timed loop runs a stack of P independent layer pairs per step, as consecutive
layers of a model do; throughput is reported per layer pair.

Prints one JSON line. --gpus above 1 is refused: this build runs on one GPU.
"""
import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=256, help="timed decode steps (K)")
    ap.add_argument("--warmup", type=int, default=8, help="untimed decode steps before timing (W)")
    ap.add_argument("--pairs", type=int, default=4, help="independent layer pairs per step (MALL eviction)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--kernel-reps", type=int, default=30)
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a 1 GiB device copy (PMC calibration) and exit")
    ap.add_argument("--index-only", action="store_true",
                    help="only run --steps csa_index_topk calls on the 1M-context indexer inputs (for profilers)")
    ap.add_argument("--share", choices=["none", "reuse", "reindex"], default="none",
                    help="cross-layer index sharing: the CSA layers of pairs 1.. reuse pair 0's top-k, or "
                         "re-index pair 0's KV and keys with their own queries")
    ap.add_argument("--derive-keys", action="store_true",
                    help="the CSA layers pool each new entry's indexer key from per-token keys in the loop")
    ap.add_argument("--rms-norm", action="store_true",
                    help="unit-gain RMSNorm (eps 1e-6) of the new compressed entries and of the queries")
    ap.add_argument("--draft", type=int, default=1,
                    help="draft tokens checked per decode step (multi-token decode, causal inside the draft; "
                         "every draft token accepted, value counts positions)")
    ap.add_argument("--kv", choices=["fp8", "mxfp4"], default="fp8",
                    help="storage of the compressed entries (mxfp4: OCP MX e2m1 codes + E8M0 per 32 dims)")
    ap.add_argument("--prefill", action="store_true",
                    help="only time the 128K-token CSA prefill (compress, causal index + top-k, attention); "
                         "--steps timed runs of each call after one warm-up")
    return ap.parse_args()


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


INDEX_SOURCES = ["compressed_sparse_kv_03_amd/csrc/indexer.hip", "compressed_sparse_kv_03_amd/csrc/topk_select.cuh",
                 "compressed_sparse_kv_03_amd/csrc/common.cuh"]


def pmc_traffic(bytes_per_launch_sha):
    """HBM bytes per launch from the committed rocprofv3 PMC summary, if it matches the current source."""
    p = os.path.join(ROOT, "profiles", "pmc_csa_index_topk_1m.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    if rec.get("source_sha") != bytes_per_launch_sha:
        return None
    return rec.get("traffic_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only; --gpus {args.gpus} is not supported "
              "(decode shards by sequence; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    from compressed_sparse_kv_03_amd import hybrid, native

    native.lib()  # fail loudly if the HIP library is missing
    dev = "cuda"
    if args.calib_copy:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        a.fill_(1)
        torch.cuda.synchronize()
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": 1 << 30}))
        return

    if args.index_only:
        index_only(args, dev)
        return
    if args.prefill:
        prefill_bench(args, dev)
        return

    K, W, P = args.steps, args.warmup, args.pairs
    spec_kw = dict(steps=K, derive_keys=args.derive_keys, rms_eps=1e-6 if args.rms_norm else 0.0, draft=args.draft,
                   kv_dtype=args.kv)
    pairs = [hybrid.LayerPair(hybrid.LayerPairSpec(seed=p, **spec_kw), dev) for p in range(P)]
    spec = pairs[0].s
    torch.cuda.synchronize()

    share = None if args.share == "none" else args.share

    def step_all(i):
        for p_, pr_ in enumerate(pairs):
            if p_ == 0 or share is None:
                pr_.step(i)
            else:
                pr_.step(i, share=share, src=pairs[0])

    # ---- warmup: W eager steps of every pair, then restore the windows
    for i in range(min(W, K)):
        step_all(i)
    torch.cuda.synchronize()
    for pr in pairs:
        pr.restore()

    # ---- capture the K-step loop of the P-pair stack in one HIP graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step_all(i)
    torch.cuda.synchronize()
    for pr in pairs:
        pr.restore()
    torch.cuda.synchronize()

    # ---- timed region: exactly K steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = e0.elapsed_time(e1)
    ms_per_step = ms / K
    tokens = spec.B * spec.draft * K * P    # positions checked (every draft token accepted)
    value = tokens / (ms / 1e3)             # layer-pair decode tokens per second
    sb = pairs[0].step_bytes()
    sf = pairs[0].step_flops()
    step_bytes = sum(sb.values())
    # with reuse, pairs 1.. read no indexer keys
    stack_bytes = step_bytes * P - (sb["csa_index"] * (P - 1) if share == "reuse" else 0)
    hbm_gbs = stack_bytes / (ms_per_step / 1e3) / 1e9

    # ---- per-call timings with a cold Infinity Cache (512 MB write before each launch)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    pr = pairs[0]
    pr.restore()

    def timed(fn, reps):
        ts = []
        for _ in range(reps):
            flush.fill_(0)
            a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a_.record()
            fn()
            b_.record()
            torch.cuda.synchronize()
            ts.append(a_.elapsed_time(b_))
        ts = np.array(ts)
        return float(np.median(ts)), float(np.percentile(ts, 10)), float(np.percentile(ts, 90)), float(ts.mean())

    s_ = pr.s
    i0 = 0

    def run_index():
        native.csa_index_topk(pr.iq[i0], pr.iqs[i0], None, pr.ik, pr.iks, pr.nvalid[i0], s_.B, s_.draft, pr.cap["csa"],
                              s_.H_I, s_.D_I, s_.k, pr.topk[i0], None, pr.ws_idx)

    def run_attn(name):
        def f():
            native.hybrid_attn_decode(pr.q[name][i0], pr.qpos[i0], pr.ckv[name], pr.scl[name], pr.kv_code,
                                      pr.cap[name], pr.nent[name][i0], pr.topk[i0] if name == "csa" else None,
                                      s_.k, pr.ring[name], s_.W, s_.B, s_.H, s_.D, s_.d_rope, s_.d_v, s_.rope_base,
                                      s_.scale, pr.out[name][i0], pr.lse[name][i0], pr.ws_att[name],
                                      q_rms_eps=s_.rms_eps, T=s_.draft, R=pr.R[name])
        return f

    reps = args.kernel_reps
    t_idx = timed(run_index, reps)
    t_csa = timed(run_attn("csa"), reps)
    t_hca = timed(run_attn("hca"), reps)
    idx_bytes = sb["csa_index"]
    achieved = idx_bytes / (t_idx[3] / 1e3) / 1e9
    idx_sha = source_sha(INDEX_SOURCES)
    traffic = pmc_traffic(idx_sha) if spec.draft == 1 else None   # counters were taken on one query per sequence

    rec = {
        "metric": "hybrid-attn decode tokens/s & HBM GB/s at 1M ctx; indexer+top-k µs/query",
        "value": round(value, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"{'mxfp4' if args.kv == 'mxfp4' else 'fp8-e4m3'} KV / mxfp4 indexer / bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) draws; no checkpoints)",
        "config": {
            "workload": "c5_hybrid_1m: CSA(m=4,k=128,FP4 indexer 8x128)+HCA(m=128) layer pair, decode batch 8, "
                        f"context 2^20, H=64, D=512+64, {args.kv} entries, bf16 window 128",
            "batch": spec.B, "context": spec.L, "layer_pairs_per_step": P,
            "tokens_per_step_per_pair": spec.B * spec.draft,
            **({"draft_tokens_per_step": spec.draft} if spec.draft > 1 else {}),
            **({"index_keys": "derived in the loop (per-token keys pooled, MXFP4)"} if args.derive_keys else {}),
            **({"normalisation": "RMSNorm (unit gain, eps 1e-6) of new entries and queries"} if args.rms_norm else {}),
            **({} if share is None else {"index_sharing": f"{share}: CSA layers of pairs 1..{P - 1} "
                                                          f"{'take pair 0 top-k' if share == 'reuse' else 're-index pair 0 KV'}"}),
        },
        "hbm_gbs": round(hbm_gbs, 1),
        "step_bytes_per_pair": step_bytes,
        "step_flops_per_pair": sum(sf.values()),
        "indexer_topk_us_per_query": round(t_idx[0] * 1e3 / (spec.B * spec.draft), 3),
        "kernels_cold_ms": {
            "csa_index_topk": {"median": t_idx[0], "p10": t_idx[1], "p90": t_idx[2]},
            "hybrid_attn_decode_csa": {"median": t_csa[0], "p10": t_csa[1], "p90": t_csa[2]},
            "hybrid_attn_decode_hca": {"median": t_hca[0], "p10": t_hca[1], "p90": t_hca[2]},
        },
        "roofline": {
            "kernel": "csa_index_topk (index_chunk_decode_kernel + index_final_decode_kernel), "
                      "8 queries x 262144 entries",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": PEAK_HBM_GBS,
            "unit": "GB/s",
            "frac": round(achieved / PEAK_HBM_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": idx_bytes,
            "avg_launch_ms": round(t_idx[3], 5),
        },
        "wall_s_timed": round(t_wall, 4),
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pairs[0])
    print(json.dumps(rec))


def index_only(args, dev):
    """csa_index_topk alone on the 1M-context decode inputs: 8 queries, 262144 visible entries of
    8x128 MXFP4 keys, k = 128 (the same shapes as the layer pair's indexer)."""
    import torch

    from compressed_sparse_kv_03_amd import hybrid, native, synth

    s = hybrid.LayerPairSpec()
    n_cap = (s.L + s.steps) // s.m_csa + 1
    n = s.L // s.m_csa
    iq, iqs = synth.mxfp4_normal((s.B, 1, s.H_I, s.D_I), synth.seed_of(s.seed, s.wid, 11), dev)
    ik, iks = synth.mxfp4_normal((s.B, n_cap, s.D_I), synth.seed_of(s.seed, s.wid, 10), dev)
    nv = torch.full((s.B, 1), n, dtype=torch.int32, device=dev)
    oi = torch.empty((s.B, 1, s.k), dtype=torch.int32, device=dev)
    ws = torch.empty(max(16, native.csa_index_topk_workspace_size(s.B, 1, n_cap, s.H_I, s.D_I, s.k)),
                     dtype=torch.uint8, device=dev)
    flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)

    def call():
        native.csa_index_topk(iq, iqs, None, ik, iks, nv, s.B, 1, n_cap, s.H_I, s.D_I, s.k, oi, None, ws)

    for _ in range(args.warmup):
        call()
    ts = []
    for i in range(args.steps):
        flush.fill_(i & 255)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        call()
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    print(json.dumps({"index_only_calls": args.steps, "mean_ms": sum(ts) / len(ts), "min_ms": min(ts)}))


def prefill_bench(args, dev):
    """The 128K-token CSA prefill: each call timed alone with HIP events (median of --steps runs)."""
    import torch

    from compressed_sparse_kv_03_amd import configs, prefill

    w = configs.C4
    p = prefill.CsaPrefill(w, dev)
    calls = {"compress": p.compress, "index": p.index, "attend": p.attend}
    for f in calls.values():  # warm-up, in pipeline order
        f()
    torch.cuda.synchronize()
    work = p.work()
    peaks = {"compress": ("hbm", PEAK_HBM_GBS, "GB/s"), "index": ("mfma", 10100.0, "TFLOP/s"),
             "attend": ("mfma", 2500.0, "TFLOP/s")}
    res = {}
    for name, f in calls.items():
        ts = []
        for _ in range(max(1, args.steps)):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            f()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        ms = sorted(ts)[len(ts) // 2]
        bound, peak, unit = peaks[name]
        r = {"ms": round(ms, 4), "bytes": work[name]["bytes"], "GB/s": round(work[name]["bytes"] / ms / 1e6, 1)}
        if "flops" in work[name]:
            r["flops"] = work[name]["flops"]
            r["TFLOP/s"] = round(work[name]["flops"] / ms / 1e9, 1)
        achieved = r["GB/s"] if bound == "hbm" else r["TFLOP/s"]
        r["roofline"] = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                         "frac": round(achieved / peak, 4)}
        res[name] = r
    total_ms = sum(r["ms"] for r in res.values())
    rec = {"prefill": w.name, "runs": max(1, args.steps), "calls": res, "total_ms": round(total_ms, 4),
           "positions_per_s": round(w.L / (total_ms / 1e3), 1)}
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = prefill_cpu_baseline(p)
    print(json.dumps(rec))


def prefill_cpu_baseline(p, n_pos=256):
    """The fp64 oracle on the host cores for a sample of prefill positions (spread over the prompt):
    index + top-k over the visible entries, the entries those positions select, and attention."""
    import numpy as np

    from oracle import attention as oatt
    from oracle import compress as ocomp
    from oracle import indexer as oidx
    from oracle import topk as otopk

    w = p.w
    m = w.m
    rows = np.linspace(w.L // 8, w.L - 1, n_pos).astype(np.int64)
    xh = p.x.cpu().numpy().view(np.uint16)
    zh = p.z.cpu().numpy()[0]
    ikh, iksh = p.ik.cpu().numpy()[0], p.iks.cpu().numpy()[0]
    iqh, iqsh = p.iq[0, rows].cpu().numpy(), p.iqs[0, rows].cpu().numpy()
    qh = p.q[rows].cpu().numpy().view(np.uint16)
    cores = len(os.sched_getaffinity(0))
    t0 = time.perf_counter()
    ent = np.zeros((p.N, w.D), np.uint16)
    for r, t in enumerate(rows):
        sc = oidx.scores(iqh[r][None], iqsh[r][None], ikh, iksh, np.array([(t + 1) // m]))
        idx, _ = otopk.topk(sc, w.k)
        for j in idx[0]:
            if j >= 0:
                _, bits, _ = ocomp.compress(xh[j * m:(j + 1) * m], zh[j * m:(j + 1) * m], j * m, m, w.d_rope,
                                            w.rope_base, "bf16")
                ent[j] = bits[0]
        oatt.prefill_one(qh[r], int(t), 0, oatt.Entries(ent, None, "bf16"), m, idx[0], xh, w.W, w.d_rope, w.d_v,
                         w.rope_base, w.softmax_scale)
    dt = time.perf_counter() - t0
    return {"value": round(n_pos / dt, 3), "unit": "positions/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_pos} positions of the 128K-token prefill (index + top-k over their visible entries, "
                      f"compression of the entries they select, attention; fp64 numpy oracle, {dt:.1f} s)"}


def cpu_baseline(pair):
    """The fp64 oracle on the host cores: the first decode steps of one layer pair, all 8 sequences."""
    import numpy as np

    from oracle import hybrid as ohyb

    spec = pair.s
    st = pair.host_state()
    cores = len(os.sched_getaffinity(0))
    layers = {}
    for name, m in (("csa", spec.m_csa), ("hca", spec.m_hca)):
        h = st[name]
        layers[name] = ohyb.Layer(name, m, spec.W, spec.d_rope, spec.d_v, spec.rope_base, spec.scale, h["ckv"],
                                  h["scl"], "fp8", np.full(spec.B, spec.L // m), h["ring"].copy(), h["ringz"].copy(),
                                  k=spec.k, ik=st["ik"] if name == "csa" else None,
                                  ik_scale=st["iks"] if name == "csa" else None)
    n_steps = 2
    t0 = time.perf_counter()
    for i in range(n_steps):
        t = np.full(spec.B, spec.L + i)
        for name, lay in layers.items():
            h = st[name]
            iq = st["iq"][i][:, 0] if name == "csa" else None
            iqs = st["iqs"][i][:, 0] if name == "csa" else None
            lay.step(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs)
    dt = time.perf_counter() - t0
    return {"value": round(spec.B * n_steps / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} decode steps x {spec.B} sequences of one CSA+HCA layer pair at 1M context "
                      f"(fp64 numpy oracle, {dt:.1f} s, {platform.processor() or platform.machine()})"}


if __name__ == "__main__":
    main()
