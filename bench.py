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
layers of a model do; throughput is reported per layer pair. The pairs are
independent (each has its own synthetic queries and tokens), so by default a
step runs them as two micro-batches: pairs 0-1 on one stream and pairs 2-3 on a
second, each stream stepping its pairs in layer order (CSA, HCA, CSA, HCA), the
two streams forked and joined once per step. --streams 1 issues every call on
one stream.

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
    ap.add_argument("--attn-only", choices=["csa", "hca"], default=None,
                    help="only run --steps hybrid_attn_decode calls of one layer of the 1M-context pair "
                         "(for profilers; a 512 MB write between calls empties the Infinity Cache)")
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
    ap.add_argument("--no-peaks", action="store_true",
                    help="skip the measured HBM / MFMA ceilings (libcskv_peaks.so) reported beside the spec peaks")
    ap.add_argument("--qk-fp4", action="store_true",
                    help="with --kv mxfp4: entry logits on the scaled FP4 x FP8 MFMA from the stored codes "
                         "(CSKV_QK_FP4) instead of widening the entries to bf16")
    ap.add_argument("--streams", type=int, default=2,
                    help="streams a step's calls are issued on (1: every call on one stream)")
    ap.add_argument("--attn-cus", type=int, default=-1,
                    help="CUs the 64-head attention's split plan counts on in the timed loop (cskv_attn_cu_budget; "
                         "-1: 256 / streams, i.e. the whole GPU on one stream); the cold per-call timings plan "
                         "for the whole GPU")
    ap.add_argument("--attn-path", type=int, choices=[0, 1, 2], default=0,
                    help="attention kernel of the timed loop (cskv_attn_path: 0 by shape, 1 the 64-head kernel, "
                         "2 the 16-head kernel); the cold per-call timings choose by shape")
    ap.add_argument("--split", choices=["chains", "layers"], default="chains",
                    help="with --streams > 1: chains = the pairs cut into one contiguous group per stream, each "
                         "stepped in layer order (independent micro-batches); layers = (2 streams) the HCA layers "
                         "of all pairs beside the CSA layers")
    ap.add_argument("--prefill", action="store_true",
                    help="only time the 128K-token CSA prefill (compress, causal index + top-k, attention); "
                         "--steps timed runs of each call after one warm-up")
    ap.add_argument("--workload", choices=["c5", "c2", "c3"], default="c5",
                    help="c5: the 1M-context hybrid layer pair (the default line); c2: CSA decode, batch 32, 64K "
                         "context, bf16 entries (indexer + gather attention); c3: HCA decode, batch 16, 1M context, "
                         "fp8 entries (dense attention)")
    return ap.parse_args()


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), else the machine type."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.machine()


def source_sha(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


INDEX_SOURCES = ["compressed_sparse_kv_03_amd/csrc/indexer.hip", "compressed_sparse_kv_03_amd/csrc/topk_select.cuh",
                 "compressed_sparse_kv_03_amd/csrc/common.cuh"]
ATTN_SOURCES = ["compressed_sparse_kv_03_amd/csrc/attention.hip", "compressed_sparse_kv_03_amd/csrc/attention_g16.hip",
                "compressed_sparse_kv_03_amd/csrc/attention_call.h", "compressed_sparse_kv_03_amd/csrc/common.cuh"]
PMC_FILES = {"csa_index_topk": ("pmc_csa_index_topk_1m.json", INDEX_SOURCES),
             "hybrid_attn_decode_hca": ("pmc_hybrid_attn_hca_1m.json", ATTN_SOURCES),
             "hybrid_attn_decode_csa": ("pmc_hybrid_attn_csa_1m.json", ATTN_SOURCES)}


def pmc_traffic(call):
    """HBM bytes per launch of a call from its committed rocprofv3 PMC summary, if that summary was
    taken on the current source (else None)."""
    name, files = PMC_FILES[call]
    p = os.path.join(ROOT, "profiles", name)
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p))
    except Exception:
        return None
    if rec.get("source_sha") != source_sha(files):
        return None
    return rec.get("traffic_bytes_per_launch")


def measured_peaks(dev):
    """Measured ceilings on this GPU, from libcskv_peaks.so (include/cskv_peaks.h): an 8 GiB
    streaming read (best of 4096/8192 workgroups, median of 7 launches) and independent MFMA
    chains (1024 workgroups of 4 waves, median of 5 launches) for bf16, fp4 and fp8."""
    import ctypes

    import numpy as np
    import torch

    from compressed_sparse_kv_03_amd import build_lib
    L = ctypes.CDLL(build_lib.PEAKS_LIB)
    L.cskv_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.cskv_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def time_ms(launch, reps):
        launch()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            launch()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts))

    nbytes = 8 << 30
    buf = torch.ones(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(65536, dtype=torch.float32, device=dev)
    best = 0.0
    for blocks in (4096, 8192):
        def rd():
            rc = L.cskv_peak_hbm_read(ctypes.c_void_p(buf.data_ptr()), nbytes, ctypes.c_void_p(sink.data_ptr()),
                                      blocks, stream)
            assert rc == 0, rc
        best = max(best, nbytes / (time_ms(rd, 7) / 1e3) / 1e9)
    del buf
    out = {"hbm_read_GBs": round(best, 1)}
    iters, blocks = 4096, 1024
    for kind, name, fl in ((0, "mfma_bf16_TFLOPs", 32768), (1, "mfma_fp4_TFLOPs", 131072),
                           (2, "mfma_fp8_TFLOPs", 131072)):
        def mm():
            rc = L.cskv_peak_mfma(kind, iters, blocks, ctypes.c_void_p(sink.data_ptr()), stream)
            assert rc == 0, rc
        out[name] = round(blocks * 4 * iters * 4 * fl / (time_ms(mm, 5) / 1e3) / 1e12, 1)
    out["method"] = ("8 GiB non-temporal streaming read; 4 independent 32x32 MFMA chains per wave (bf16 32x32x16, "
                     "scaled e2m1 and e4m3 32x32x64)")
    return out


def with_measured(r, peaks):
    """Adds the fraction of the measured ceiling matching a roofline record's bound and unit."""
    if peaks is None:
        return r
    if r["unit"] == "GB/s":
        pm = peaks["hbm_read_GBs"]
    else:
        pm = peaks.get(r.get("mfma_type", "mfma_bf16_TFLOPs"))
    r["peak_measured"] = pm
    r["frac_measured"] = round(r["achieved"] / pm, 4) if pm else None
    return r


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
    if args.workload != "c5":
        attn_workload_bench(args, dev)
        return

    K, W, P = args.steps, args.warmup, args.pairs
    if args.qk_fp4 and args.kv != "mxfp4":
        sys.exit("--qk-fp4 needs --kv mxfp4")
    spec_kw = dict(steps=K, derive_keys=args.derive_keys, rms_eps=1e-6 if args.rms_norm else 0.0, draft=args.draft,
                   kv_dtype=args.kv, qk_fp4=args.qk_fp4)
    if args.attn_only:
        pr = hybrid.LayerPair(hybrid.LayerPairSpec(seed=0, **spec_kw), dev)
        s_, name = pr.s, args.attn_only
        pr.step(0)  # step 0's top-k (the indexer) and state, which the calls below reuse
        flush = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
        for i in range(W + K):
            flush.fill_(i & 255)
            native.hybrid_attn_decode(pr.q[name][0], pr.qpos[0], pr.ckv[name], pr.scl[name], pr.kv_code,
                                      pr.cap[name], pr.nent[name][0], pr.topk[0] if name == "csa" else None,
                                      s_.k, pr.ring[name], s_.W, s_.B, s_.H, s_.D, s_.d_rope, s_.d_v, s_.rope_base,
                                      s_.scale, pr.out[name][0], pr.lse[name][0], pr.ws_att[name],
                                      q_rms_eps=s_.rms_eps, T=s_.draft, R=pr.R[name])
        torch.cuda.synchronize()
        print(json.dumps({"attn_only": name, "calls": W + K}))
        return
    pairs = [hybrid.LayerPair(hybrid.LayerPairSpec(seed=p, **spec_kw), dev) for p in range(P)]
    spec = pairs[0].s
    torch.cuda.synchronize()

    share = None if args.share == "none" else args.share

    # further streams (default priority, like the first) for the parallel branches of a step
    if args.streams < 1 or args.streams > P or (args.split == "layers" and args.streams != 2):
        sys.exit("--streams: 1 .. pairs (exactly 2 with --split layers)")
    if args.split == "layers" and share is not None:
        sys.exit("--split layers takes no --share (the sharing layers wait for pair 0's step)")
    side = [torch.cuda.Stream() for _ in range(args.streams - 1)]
    # the workspaces were sized for the whole-GPU plan, which needs the most splits
    attn_cus = 256 // args.streams if args.attn_cus < 0 else args.attn_cus
    native.cskv_attn_cu_budget(attn_cus)
    native.cskv_attn_path(args.attn_path)

    def step_all(i):
        hybrid.step_stack(pairs, i, share=share, side=side, split=args.split)

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

    # ---- per-call timings with a cold Infinity Cache (512 MB write before each launch), each call
    # alone on the GPU and planned for all of it
    native.cskv_attn_cu_budget(0)
    native.cskv_attn_path(0)
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
    calls = {"csa_index_topk": (t_idx, sb["csa_index"], sf["csa_index"],
                                "csa_index_topk (index_chunk_decode_kernel + index_final_decode_kernel), "
                                f"{spec.B * spec.draft} queries x {pairs[0].n0['csa']} entries"),
             "hybrid_attn_decode_csa": (t_csa, sb["csa_attn"], sf["csa_attn"],
                                        f"hybrid_attn_decode, CSA: {spec.B * spec.draft} queries x ({spec.k} top-k "
                                        f"entries + {spec.W} window), 64 heads (16-head kernel + merge)"),
             "hybrid_attn_decode_hca": (t_hca, sb["hca_attn"], sf["hca_attn"],
                                        f"hybrid_attn_decode, HCA: {spec.B * spec.draft} queries x "
                                        f"({pairs[0].n0['hca']} entries + {spec.W} window), 64 heads "
                                        "(64-head kernel + merge)")}

    peaks = None if args.no_peaks else measured_peaks(dev)   # after the timed runs

    def roofline(call):
        t, nbytes, nflops, what = calls[call]
        gbs = nbytes / (t[3] / 1e3) / 1e9
        tf = nflops / (t[3] / 1e3) / 1e12
        # the bound the kernel's own work is nearer to: bytes at 8 TB/s vs bf16 MFMA flops at 2.5 PFLOP/s
        mfma = call != "csa_index_topk" and tf / 2500.0 > gbs / PEAK_HBM_GBS
        r = {"kernel": what, "bound": "mfma" if mfma else "hbm",
             "achieved": round(tf if mfma else gbs, 1), "peak": 2500.0 if mfma else PEAK_HBM_GBS,
             "unit": "TFLOP/s" if mfma else "GB/s"}
        r["frac"] = round(r["achieved"] / r["peak"], 4)
        r["traffic"] = pmc_traffic(call) if spec.draft == 1 else None  # counters: one query per sequence
        r["algorithmic_bytes_per_launch"] = nbytes
        r["algorithmic_flops_per_launch"] = nflops
        r["avg_launch_ms"] = round(t[3], 5)
        return r

    # the dominant call: the one moving the most algorithmic bytes (the indexer, 77% of the step's);
    # its cold-call time and the HCA attention's are close, so ranking by time would flip between runs
    dominant = max(calls, key=lambda c: calls[c][1])

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
        "dtype": f"{'mxfp4' if args.kv == 'mxfp4' else 'fp8-e4m3'} KV / mxfp4 indexer / "
                 f"{'fp4xfp8 MFMA for entry logits, ' if args.qk_fp4 else ''}bf16 MFMA, fp32 accumulate",
        "data": "synthetic (seeded N(0,1) draws; no checkpoints)",
        "config": {
            "workload": "c5_hybrid_1m: CSA(m=4,k=128,FP4 indexer 8x128)+HCA(m=128) layer pair, decode batch 8, "
                        f"context 2^20, H=64, D=512+64, {args.kv} entries, bf16 window 128",
            "batch": spec.B, "context": spec.L, "layer_pairs_per_step": P,
            "streams": args.streams,
            "attn_cu_budget": attn_cus,
            **({"attn_path": {1: "64-head kernel", 2: "16-head kernel"}[args.attn_path]} if args.attn_path else {}),
            **({"stream_split": ("pairs in one contiguous group per stream, each stepped in layer order "
                                 "(independent micro-batches)") if args.split == "chains" else
                "the HCA layers of all pairs on the second stream beside the CSA layers"}
               if args.streams > 1 else {}),
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
        "roofline": with_measured(roofline(dominant), peaks),
        "roofline_calls": {c: with_measured(roofline(c), peaks) for c in calls if c != dominant},
        "roofline_step": with_measured({"bound": "hbm", "achieved": round(hbm_gbs, 1), "peak": PEAK_HBM_GBS,
                                        "unit": "GB/s", "frac": round(hbm_gbs / PEAK_HBM_GBS, 4),
                                        "what": "algorithmic bytes of the whole layer-pair step / the step's time"},
                                       peaks),
        "measured_peaks": peaks,
        "wall_s_timed": round(t_wall, 4),
    }

    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(pairs[0])
    print(json.dumps(rec))


def attn_workload_bench(args, dev):
    """c2 (CSA decode, batch 32, 65536-token context: 16384 bf16 entries per sequence, indexer 8x128
    MXFP4 top-128 + gather attention over the top-k and a 128-token window) or c3 (HCA decode,
    batch 16, 2^20-token context: 8192 fp8 entries per sequence, dense attention + window). One
    step = the layer's calls for the whole batch; P independent caches are cycled so that each step
    reads its entries from HBM rather than from the Infinity Cache. Inputs are synthetic (the
    generator's seeded N(0, 1/D) draws) and resident before timing."""
    import numpy as np
    import torch

    from compressed_sparse_kv_03_amd import configs, native, synth

    w = configs.C2 if args.workload == "c2" else configs.C3
    B, H, D, dv, W, k = w.B, w.H, w.D, w.d_v, w.W, w.k
    n = w.L // w.m
    t = w.L - 1
    P = 4 if args.workload == "c3" else 1   # c2's 604 MB of entries already exceed the cache
    dense = args.workload == "c3"
    kv = native.CSKV_FP8_E4M3 if dense else native.CSKV_BF16
    st = []
    for p in range(P):
        d = {"q": synth.normal_bf16_bits((B, H, D), w.sigma, synth.seed_of(p, w.wid, 2), dev),
             "ring": synth.normal_bf16_bits((B, W, D), w.sigma, synth.seed_of(p, w.wid, 4), dev)}
        if dense:
            d["ckv"], d["sc"] = synth.fp8_rows_normal((B, n, D), w.sigma, synth.seed_of(p, w.wid, 3), dev)
        else:
            d["ckv"], d["sc"] = synth.normal_bf16_bits((B, n, D), w.sigma, synth.seed_of(p, w.wid, 3), dev), None
            d["iq"], d["iqs"] = synth.mxfp4_normal((B, 1, w.H_I, w.D_I), synth.seed_of(p, w.wid, 11), dev)
            d["ik"], d["iks"] = synth.mxfp4_normal((B, n, w.D_I), synth.seed_of(p, w.wid, 10), dev)
            d["topk"] = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
        st.append(d)
    qpos = torch.full((B,), t, dtype=torch.int64, device=dev)
    nent = torch.full((B,), n, dtype=torch.int32, device=dev)
    nv = torch.full((B, 1), n, dtype=torch.int32, device=dev)
    out = torch.empty((B, H, dv), dtype=torch.int16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    ws = torch.empty(max(16, native.hybrid_attn_decode_workspace_size(B, H, dv, n, k, W, dense)), dtype=torch.uint8,
                     device=dev)
    wsi = None if dense else torch.empty(max(16, native.csa_index_topk_workspace_size(B, 1, n, w.H_I, w.D_I, k)),
                                         dtype=torch.uint8, device=dev)

    def index(d):
        native.csa_index_topk(d["iq"], d["iqs"], None, d["ik"], d["iks"], nv, B, 1, n, w.H_I, w.D_I, k, d["topk"],
                              None, wsi)

    def attend(d):
        native.hybrid_attn_decode(d["q"], qpos, d["ckv"], d["sc"], kv, n, nent, None if dense else d["topk"], k,
                                  d["ring"], W, B, H, D, w.d_rope, dv, w.rope_base, w.softmax_scale, out, lse, ws)

    def step(i):
        d = st[i % P]
        if not dense:
            index(d)
        attend(d)

    K = args.steps
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(K):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1)
    ms_step = ms / K
    eb = D * (1 if dense else 2) + (4 if dense else 0)          # stored entry bytes
    q_o = B * H * (D + dv) * 2
    win = B * W * D * 2
    attn_bytes = (B * n * eb if dense else B * k * eb + B * k * 4) + win + q_o
    idx_bytes = 0 if dense else B * n * (w.D_I // 2 + w.D_I // 32) + B * w.H_I * (w.D_I // 2 + w.D_I // 32) + B * k * 4
    attn_flops = 2 * B * H * ((n if dense else k) + W) * (D + dv)
    # the attention call alone (its own graph): the HBM roofline of the gather / dense attention
    g2 = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g2):
        for i in range(K):
            attend(st[i % P])
    g2.replay()
    torch.cuda.synchronize()
    e0.record()
    g2.replay()
    e1.record()
    torch.cuda.synchronize()
    ms_attn = e0.elapsed_time(e1) / K
    gbs = attn_bytes / (ms_attn / 1e3) / 1e9
    rec = {
        "metric": "hybrid-attn decode tokens/s & HBM GB/s at 1M ctx; indexer+top-k µs/query",
        "value": round(B * K / (ms / 1e3), 1), "unit": "tokens/s", "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": ("fp8-e4m3" if dense else "bf16") + " KV / bf16 MFMA, fp32 accumulate"
                 + ("" if dense else " / mxfp4 indexer"),
        "data": "synthetic (seeded N(0,1/D) draws; no checkpoints)",
        "config": {"workload": w.name + (": HCA decode, batch 16, context 2^20, 8192 fp8 entries + window 128"
                                         if dense else ": CSA decode, batch 32, context 65536, 16384 bf16 entries, "
                                                       "MXFP4 indexer 8x128, top-128 + window 128"),
                   "batch": B, "context": w.L, "caches_cycled": P},
        "hbm_gbs_step": round((attn_bytes + idx_bytes) / (ms_step / 1e3) / 1e9, 1),
        "roofline": {"kernel": "hybrid_attn_decode (attention kernel + merge)", "bound": "hbm",
                     "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None,
                     "algorithmic_bytes_per_launch": attn_bytes, "algorithmic_flops_per_launch": attn_flops,
                     "avg_launch_ms": round(ms_attn, 5),
                     "mfma_frac_bf16": round(attn_flops / (ms_attn / 1e3) / 1e12 / 2500.0, 4)},
    }
    peaks = None if args.no_peaks else measured_peaks(dev)
    with_measured(rec["roofline"], peaks)
    rec["measured_peaks"] = peaks
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
    bounds = {"compress": ("hbm", PEAK_HBM_GBS, "GB/s", None), "index": ("mfma", 10100.0, "TFLOP/s", "mfma_fp4_TFLOPs"),
              "attend": ("mfma", 2500.0, "TFLOP/s", "mfma_bf16_TFLOPs")}
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
        bound, peak, unit, mtype = bounds[name]
        r = {"ms": round(ms, 4), "bytes": work[name]["bytes"], "GB/s": round(work[name]["bytes"] / ms / 1e6, 1)}
        if "flops" in work[name]:
            r["flops"] = work[name]["flops"]
            r["TFLOP/s"] = round(work[name]["flops"] / ms / 1e9, 1)
        achieved = r["GB/s"] if bound == "hbm" else r["TFLOP/s"]
        r["roofline"] = {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                         "frac": round(achieved / peak, 4), **({"mfma_type": mtype} if mtype else {})}
        res[name] = r
    peaks = None if args.no_peaks else measured_peaks(dev)
    for r in res.values():
        with_measured(r["roofline"], peaks)
    total_ms = sum(r["ms"] for r in res.values())
    rec = {"prefill": w.name, "runs": max(1, args.steps), "calls": res, "total_ms": round(total_ms, 4),
           "positions_per_s": round(w.L / (total_ms / 1e3), 1), "measured_peaks": peaks}
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
    return {"value": round(n_pos / dt, 3), "unit": "positions/s", "cores": cores, "kind": "oracle", "cpu": cpu_model(),
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
    n_steps, Td = 4, spec.draft   # about 12 s of host work
    t0 = time.perf_counter()
    for i in range(n_steps):
        t = np.full(spec.B, spec.L + i * Td)
        for name, lay in layers.items():
            h = st[name]
            if Td == 1:
                iq = st["iq"][i][:, 0] if name == "csa" else None
                iqs = st["iqs"][i][:, 0] if name == "csa" else None
                lay.step(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs)
            else:  # every draft token accepted, as on the GPU
                iq = st["iq"][i] if name == "csa" else None
                iqs = st["iqs"][i] if name == "csa" else None
                lay.step_draft(t, h["xn"][i], h["zn"][i], h["q"][i], iq, iqs)
    dt = time.perf_counter() - t0
    pos = "positions" if Td > 1 else "steps"
    return {"value": round(spec.B * Td * n_steps / dt, 4), "unit": "tokens/s", "cores": cores, "kind": "oracle",
            "sample": f"{n_steps} decode steps x {spec.B} sequences{f' x {Td} draft {pos}' if Td > 1 else ''} of one "
                      f"CSA+HCA layer pair at 1M context (fp64 numpy oracle, {dt:.1f} s)", "cpu": cpu_model()}


if __name__ == "__main__":
    main()
