"""CPU checks of the C ABI: every declared symbol is exported, and argument validation returns the
documented codes before anything touches a GPU."""
import os
import re

import pytest

from compressed_sparse_kv_03_amd import native

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "cskv.h")


def declared():
    txt = open(HDR).read()
    return re.findall(r"CSKV_API\s+(?:const\s+char\*|int|size_t)\s+([a-z_]+)\(", txt)


def test_library_exports_every_declared_symbol():
    names = declared()
    assert len(names) == 17
    L = native.lib()
    for n in names:
        assert getattr(L, n, None) is not None, f"{n} not exported"
    assert set(names) == set(native.exported_symbols())
    assert L.cskv_abi_version() == 3


@pytest.mark.parametrize("code,text", [(0, "ok"), (-1, "invalid argument"), (-2, "shape not supported"),
                                       (-3, "workspace"), (-4, "HIP launch")])
def test_strerror(code, text):
    assert text in native.lib().cskv_strerror(code).decode()


def test_compress_validation():
    L = native.lib()
    # (x, xs, z, zs, pos0, B, n_tok, D, d_rope, m, off, base, dtype, out, out_scale, oss, e0, rms_eps, stream)
    bad = [
        (None, 0, None, 0, None, 1, 4, 8, 0, 0, 0, 1e4, 0, None, None, 1, None, 0.0, None),          # m = 0
        (None, 0, None, 0, None, 1, 6, 8, 0, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None),          # n_tok % m
        (None, 0, None, 0, None, 1, 4, 12, 0, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None),         # D % 8
        (None, 0, None, 0, None, 1, 4, 16, 4, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None),         # d_rope % 8
        (None, 0, None, 0, None, 1, 4, 16, 0, 4, 0, 1e4, 7, None, None, 1, None, 0.0, None),         # dtype
        (None, 64, None, 4, None, 1, 4, 16, 0, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None),        # null x
        (16, 64, 16, 4, 16, 1, 4, 16, 0, 4, 0, 1e4, 1, 16, None, 1, None, 0.0, None),                # fp8 w/o scale
        (8, 64, 16, 4, 16, 1, 4, 16, 0, 4, 0, 1e4, 0, 16, None, 1, None, 0.0, None),                 # misaligned
        (None, 0, None, 0, None, 1, 4, 16, 0, 4, 0, 1e4, 0, None, None, 1, None, -1.0, None),        # rms_eps < 0
    ]
    for args in bad:
        assert L.csa_compress(*args) == -1, args
    assert L.csa_compress(None, 0, None, 0, None, 1, 4, 2048, 0, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None) == -2
    assert L.hca_compress(None, 0, None, 0, None, 1, 0, 16, 0, 4, 0, 1e4, 0, None, None, 1, None, 0.0, None) == 0


def test_index_key_pool_validation():
    L = native.lib()
    # (xk, xks, z, zs, B, n_tok, D_I, m, out, out_scale, oss, e0, stream)
    assert L.csa_index_key_pool(None, 0, None, 0, 1, 4, 128, 0, None, None, 1, None, None) == -1    # m = 0
    assert L.csa_index_key_pool(None, 0, None, 0, 1, 6, 128, 4, None, None, 1, None, None) == -1    # n_tok % m
    assert L.csa_index_key_pool(None, 0, None, 0, 1, 4, 96, 4, None, None, 1, None, None) == -2     # D_I
    assert L.csa_index_key_pool(None, 512, None, 4, 1, 4, 128, 4, None, None, 1, None, None) == -1  # null
    assert L.csa_index_key_pool(8, 512, 16, 4, 1, 4, 128, 4, 16, 16, 1, None, None) == -1          # misaligned
    assert L.csa_index_key_pool(16, 256, 16, 4, 1, 4, 128, 4, 16, 16, 1, None, None) == -1         # stride
    assert L.csa_index_key_pool(None, 0, None, 0, 1, 0, 128, 4, None, None, 1, None, None) == 0     # empty


def test_index_validation():
    L = native.lib()
    args = lambda **kw: dict(dict(iq=16, iqs=16, hw=None, ik=16, iks=16, nv=16, B=1, T=1, N=100, H=8, D=128,  # noqa
                                  k=128, oi=16, os=None, ws=16, wsb=1 << 20, s=None), **kw)

    def call(**kw):
        a = args(**kw)
        return L.csa_index_topk(a["iq"], a["iqs"], a["hw"], a["ik"], a["iks"], a["nv"], a["B"], a["T"], a["N"],
                                a["H"], a["D"], a["k"], a["oi"], a["os"], a["ws"], a["wsb"], a["s"])
    assert call(D=100) == -1
    assert call(D=1024) == -2
    assert call(H=17) == -2
    assert call(k=0) == -1
    assert call(k=2000) == -2
    assert call(iq=None) == -1
    assert call(ws=None) == -3
    assert call(wsb=8) == -3
    assert L.csa_index_topk_workspace_size(1, 1, 100, 8, 128, 128) > 0


def test_attention_validation():
    L = native.lib()

    def dec(**kw):
        a = dict(q=16, qp=16, ckv=16, sc=16, dt=1, N=100, ne=16, tk=None, k=128, win=16, W=128, B=1, H=64,
                 D=576, dr=64, dv=512, base=1e4, scale=0.04, out=16, lse=None, ws=16, wsb=1 << 30, eps=0.0,
                 T=1, R=0, s=None)
        a.update(kw)
        return L.hybrid_attn_decode(*a.values())
    assert dec(D=100) == -1
    assert dec(D=320, dv=256) == -2          # (D, d_v) pair not compiled
    assert dec(dv=600) == -1
    assert dec(H=0) == -1
    assert dec(dt=5) == -1
    assert dec(q=None) == -1
    assert dec(sc=None) == -1
    assert dec(ws=None, wsb=0, N=20000) == -3    # 20128 keys are split: partials need a workspace
    assert dec(eps=-1.0) == -1
    assert dec(T=0) == -1
    assert dec(R=100) == -1                  # ring smaller than the window
    assert dec(T=2) == -1                    # a 2-token draft needs R >= W + 1 (R = 0 means R = W)
    assert dec(T=3, R=129) == -1             # ... and a 3-token one R >= W + 2
    assert dec(eps=float("nan")) == -1
    assert dec(dt=native.CSKV_FP8_E4M3 | native.CSKV_QK_FP4) == -1    # FP4 logits need MXFP4 entries
    assert dec(dt=native.CSKV_MXFP4 | native.CSKV_QK_FP4, D=160, dv=128) == -1  # ... and D % 64 == 0
    assert dec(dt=native.CSKV_MXFP4 | 0x200) == -1                     # an unknown flag
    assert L.hybrid_attn_decode_workspace_size(8, 64, 512, 8194, 128, 128, 1) > 0

    def dec_na(**kw):     # the allocation-free variant: same arguments without ws / ws_bytes
        a = dict(q=16, qp=16, ckv=16, sc=16, dt=1, N=100, ne=16, tk=None, k=128, win=16, W=128, B=1, H=64,
                 D=576, dr=64, dv=512, base=1e4, scale=0.04, out=16, lse=None, eps=0.0, T=1, R=0, s=None)
        a.update(kw)
        return L.hybrid_attn_decode_noalloc(*a.values())
    assert dec_na(D=100) == -1
    assert dec_na(q=None) == -1
    assert dec_na(T=2) == -1
    # 16 queries over 65536 dense entries need 17 splits of partials: more than the static scratch,
    # refused before any HIP call
    assert L.hybrid_attn_decode_workspace_size(16, 64, 512, 65536, 0, 128, 1) > native.NOALLOC_SCRATCH_BYTES
    assert dec_na(B=16, N=65536) == -3
    assert L.cskv_attn_path(3) == -1 and L.cskv_attn_path(-1) == -1
    assert L.cskv_attn_path(0) == 0
    # a smaller CU budget plans fewer, longer splits of the 1M HCA key set (smaller workspace)
    assert L.cskv_attn_cu_budget(-1) == -1 and L.cskv_attn_cu_budget(4097) == -1
    full = L.hybrid_attn_decode_workspace_size(8, 64, 512, 8194, 128, 128, 1)
    assert L.cskv_attn_cu_budget(128) == 0
    half = L.hybrid_attn_decode_workspace_size(8, 64, 512, 8194, 128, 128, 1)
    assert L.cskv_attn_cu_budget(0) == 0
    assert 0 < half < full and L.hybrid_attn_decode_workspace_size(8, 64, 512, 8194, 128, 128, 1) == full
    def dec_ap(**kw):     # the call with the state update: rings and new tokens instead of win
        a = dict(q=16, qp=16, ckv=16, sc=16, dt=1, N=100, ne=16, tk=None, k=128, ring=16, rz=None, x=16, z=None,
                 W=128, B=1, H=64, D=576, dr=64, dv=512, base=1e4, scale=0.04, out=16, lse=None, ws=None, wsb=0,
                 eps=0.0, T=1, R=0, s=None)
        a.update(kw)
        return L.hybrid_attn_decode_append(*a.values())
    assert dec_ap(ring=None) == -1                      # no ring to write
    assert dec_ap(x=None) == -1                         # no new tokens
    assert dec_ap(z=16) == -1                           # z_new without ring_z
    assert dec_ap(W=0, R=0) == -1                       # no ring slots at all
    assert dec_ap(W=0, R=2, T=3) == -1                  # fewer slots than new tokens
    assert dec_ap(T=2, R=128) == -1                     # R < W + T - 1
    assert dec_ap(B=1 << 16, R=1 << 14) == -1           # B * R >= 2^30 (row encoding)
    assert dec_ap(x=24) == -1                           # x_new not 16-byte aligned
    assert dec_ap(D=100) == -1                          # the decode requirements hold as well
    pre = lambda **kw: L.hybrid_attn_prefill(*dict(dict(q=16, p0=0, T=10, ckv=16, sc=None, dt=0, N=2, tk=None,  # noqa
                                                        k=1, x=16, W=128, H=16, D=128, dr=64, dv=128, m=4,
                                                        base=1e4, scale=0.1, out=16, lse=None, ws=None, wsb=0,
                                                        eps=0.0, s=None), **kw).values())
    assert pre(m=0) == -1
    assert pre(T=0) == 0
    assert pre(x=None) == -1


def test_ring_append_validation():
    L = native.lib()
    # (x_new, z_new, pos, ring_x, ring_z, B, T, D, R, stream)
    assert L.cskv_ring_append(16, None, 16, 16, None, 1, 0, 64, 8, None) == -1     # T = 0
    assert L.cskv_ring_append(16, None, 16, 16, None, 1, 9, 64, 8, None) == -1     # T > R
    assert L.cskv_ring_append(16, None, 16, 16, None, 1, 2, 60, 8, None) == -1     # D % 8
    assert L.cskv_ring_append(16, 16, 16, 16, None, 1, 2, 64, 8, None) == -1       # z_new without ring_z
    assert L.cskv_ring_append(None, None, 16, 16, None, 1, 2, 64, 8, None) == -1   # null


def test_peaks_library_exports_and_validation():
    """The measurement helpers (include/cskv_peaks.h): every declared symbol exported, bad
    arguments refused before any launch."""
    import ctypes

    from compressed_sparse_kv_03_amd import build_lib
    hdr = os.path.join(os.path.dirname(HDR), "cskv_peaks.h")
    names = re.findall(r"CSKV_PEAKS_API\s+(?:const\s+char\*|int)\s+([a-z_]+)\(", open(hdr).read())
    assert sorted(names) == ["cskv_peak_hbm_read", "cskv_peak_mfma", "cskv_peaks_last_error"]
    L = ctypes.CDLL(build_lib.PEAKS_LIB)
    for n in names:
        assert getattr(L, n, None) is not None, f"{n} not exported"
    L.cskv_peak_hbm_read.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p]
    L.cskv_peak_mfma.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    assert L.cskv_peak_hbm_read(None, 1 << 20, 16, 1024, None) == -1
    assert L.cskv_peak_hbm_read(16, 100, 16, 1024, None) == -1          # size not a multiple of 16
    assert L.cskv_peak_hbm_read(16, 1 << 20, 16, 0, None) == -1
    assert L.cskv_peak_mfma(3, 1, 1, 16, None) == -1
    assert L.cskv_peak_mfma(0, 0, 1, 16, None) == -1
    assert L.cskv_peak_mfma(0, 1, 1, None, None) == -1
