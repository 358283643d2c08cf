"""The five workloads (shapes, distributions) and smaller variants used by tests.

c1  CSA decode, tiny:  B=1, context 4096, 16 query heads on one KV head, D=128
    (last 64 dims rotated, base 10000), m=4 -> 1024 entries, indexer 4x64
    MXFP4, top-k 128, window 128.
c2  CSA decode:        B=32, context 65536 (16384 entries), 64 heads, D=512+64,
    bf16 entries N(0,1)/sqrt(576), indexer 8x128 MXFP4, top-k 128, window 128.
c3  HCA decode:        B=16, context 2^20, m=128 -> 8192 entries, fp8 e4m3 with
    per-entry scale, 64 heads, dense, window 128.
c4  CSA prefill:       one 131072-token prompt, m=4 (32768 entries), causal
    indexer 8x128 MXFP4 top-k 128 per position, 64 heads, D=512+64, bf16.
c5  hybrid layer pair: B=8, context 2^20, one CSA layer (m=4, top-k 128, FP4
    indexer 8x128) and one HCA layer (m=128), fp8 entries, bf16 windows of
    128; 256 decode steps appending tokens and re-compressing every m tokens.
"""
from dataclasses import dataclass, replace


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    kind: str            # csa_decode | hca_decode | csa_prefill | hybrid
    B: int
    L: int               # context length (decode: the query sits at position L-1; hybrid: loop starts at L)
    H: int
    D: int
    d_rope: int
    d_v: int
    m: int = 4
    k: int = 128
    W: int = 128
    H_I: int = 8
    D_I: int = 128
    ckv_dtype: str = "bf16"
    steps: int = 1
    rope_base: float = 10000.0
    std: float = 0.0     # N(0, std^2) for q / k / v; 0 -> 1/sqrt(D)
    compress_on_gpu: bool = False

    @property
    def sigma(self):
        return self.std if self.std > 0 else self.D ** -0.5

    @property
    def softmax_scale(self):
        return self.D ** -0.5


C1 = Workload("c1_csa_tiny", 1, "csa_decode", B=1, L=4096, H=16, D=128, d_rope=64, d_v=128, H_I=4, D_I=64,
              compress_on_gpu=True)
C2 = Workload("c2_csa_b32_64k", 2, "csa_decode", B=32, L=65536, H=64, D=576, d_rope=64, d_v=512)
C3 = Workload("c3_hca_b16_1m", 3, "hca_decode", B=16, L=1 << 20, H=64, D=576, d_rope=64, d_v=512, m=128,
              ckv_dtype="fp8", compress_on_gpu=True)
C4 = Workload("c4_csa_prefill_128k", 4, "csa_prefill", B=1, L=131072, H=64, D=576, d_rope=64, d_v=512,
              compress_on_gpu=True)
C5 = Workload("c5_hybrid_1m", 5, "hybrid", B=8, L=1 << 20, H=64, D=576, d_rope=64, d_v=512, ckv_dtype="fp8",
              steps=256)

ALL = {w.name: w for w in (C1, C2, C3, C4, C5)}


def small(w, **kw):
    """A reduced copy of a workload for oracle-sized parity runs (same structure, smaller sizes)."""
    return replace(w, name=w.name + "_small", **kw)
