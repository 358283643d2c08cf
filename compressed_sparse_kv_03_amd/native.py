"""ctypes binding of libcskv.so (the C ABI declared in include/cskv.h).

Argument marshalling only: every wrapper turns torch tensors into device
pointers and the current HIP stream, calls the C function of the same name,
and raises CskvError on a non-zero return. All computation happens in the
library's HIP kernels; there is no fallback path.
"""
import ctypes
import os

import torch

# CSKV_LIB_PATH selects another build of the library (the host-sanitized one in CPU tests)
_LIB_PATH = os.environ.get("CSKV_LIB_PATH") or os.path.join(os.path.dirname(os.path.abspath(__file__)), "libcskv.so")

CSKV_BF16 = 0
CSKV_FP8_E4M3 = 1
CSKV_MXFP4 = 2
CSKV_QK_FP4 = 0x100   # OR-ed into CSKV_MXFP4 for the attention calls: QK^T on the scaled FP4 MFMA

_p, _i, _i64, _f, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t

_SIGS = {
    "cskv_abi_version": ([], _i),
    "cskv_strerror": ([_i], ctypes.c_char_p),
    "cskv_last_error": ([], ctypes.c_char_p),
    "csa_compress": ([_p, _i64, _p, _i64, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _p, _i64, _p, _f, _p], _i),
    "hca_compress": ([_p, _i64, _p, _i64, _p, _i, _i, _i, _i, _i, _i, _f, _i, _p, _p, _i64, _p, _f, _p], _i),
    "csa_index_topk": ([_p, _p, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i, _p, _p, _p, _sz, _p], _i),
    "csa_index_topk_workspace_size": ([_i, _i, _i, _i, _i, _i], _sz),
    "hybrid_attn_decode": ([_p, _p, _p, _p, _i, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f, _f,
                            _p, _p, _p, _sz, _f, _i, _i, _p], _i),
    "hybrid_attn_decode_workspace_size": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "hybrid_attn_decode_append": ([_p, _p, _p, _p, _i, _i, _p, _p, _i, _p, _p, _p, _p, _i, _i, _i, _i, _i, _i,
                                   _f, _f, _p, _p, _p, _sz, _f, _i, _i, _p], _i),
    "cskv_attn_path": ([_i], _i),
    "cskv_attn_cu_budget": ([_i], _i),
    "hybrid_attn_decode_noalloc": ([_p, _p, _p, _p, _i, _i, _p, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f, _f,
                                    _p, _p, _f, _i, _i, _p], _i),
    "hybrid_attn_prefill": ([_p, _i64, _i, _p, _p, _i, _i, _p, _i, _p, _i, _i, _i, _i, _i, _i, _f, _f,
                             _p, _p, _p, _sz, _f, _p], _i),
    "hybrid_attn_prefill_workspace_size": ([_i, _i, _i, _i, _i, _i, _i], _sz),
    "cskv_ring_append": ([_p, _p, _p, _p, _p, _i, _i, _i, _i, _p], _i),
    "csa_index_key_pool": ([_p, _i64, _p, _i64, _i, _i, _i, _i, _p, _p, _i64, _p, _p], _i),
}

_lib = None


class CskvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"cskv error {code}: {msg}")
        self.code = code


def lib():
    """Load libcskv.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError(f"{_LIB_PATH} is missing: build it with "
                              "`python -m compressed_sparse_kv_03_amd.build_lib`")
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, ret) in _SIGS.items():
            fn = getattr(L, name, None)
            if fn is None:      # reported by missing_symbols(); calling it raises AttributeError
                continue
            fn.argtypes = args
            fn.restype = ret
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def missing_symbols():
    L = lib()
    return [n for n in _SIGS if getattr(L, n, None) is None]


def _ptr(t):
    if t is None:
        return None
    assert isinstance(t, torch.Tensor), type(t)
    return t.data_ptr()


def _stream(stream=None):
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def _check(rc):
    if rc != 0:
        L = lib()
        raise CskvError(rc, f"{L.cskv_strerror(rc).decode()}: {L.cskv_last_error().decode()}")


# ------------------------------------------------------------------ compression
def _compress(name, x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D, d_rope, m, entry_pos_offset,
              rope_base, out_dtype, out, out_scale, out_seq_stride, out_entry0, rms_eps, stream):
    fn = getattr(lib(), name)
    _check(fn(_ptr(x), x_seq_stride, _ptr(z), z_seq_stride, _ptr(pos0), B, n_tok, D, d_rope, m,
              entry_pos_offset, rope_base, out_dtype, _ptr(out), _ptr(out_scale), out_seq_stride,
              _ptr(out_entry0), rms_eps, _stream(stream)))


def csa_compress(x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D, d_rope, m, entry_pos_offset,
                 rope_base, out_dtype, out, out_scale, out_seq_stride, out_entry0=None, stream=None, *, rms_eps=0.0):
    _compress("csa_compress", x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D, d_rope, m,
              entry_pos_offset, rope_base, out_dtype, out, out_scale, out_seq_stride, out_entry0, rms_eps, stream)


def hca_compress(x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D, d_rope, m, entry_pos_offset,
                 rope_base, out_dtype, out, out_scale, out_seq_stride, out_entry0=None, stream=None, *, rms_eps=0.0):
    _compress("hca_compress", x, x_seq_stride, z, z_seq_stride, pos0, B, n_tok, D, d_rope, m,
              entry_pos_offset, rope_base, out_dtype, out, out_scale, out_seq_stride, out_entry0, rms_eps, stream)


def csa_index_key_pool(xk, xk_seq_stride, z, z_seq_stride, B, n_tok, D_I, m, out_ik, out_ik_scale,
                       out_seq_stride, out_entry0=None, stream=None):
    _check(lib().csa_index_key_pool(_ptr(xk), xk_seq_stride, _ptr(z), z_seq_stride, B, n_tok, D_I, m, _ptr(out_ik),
                                    _ptr(out_ik_scale), out_seq_stride, _ptr(out_entry0), _stream(stream)))


# ------------------------------------------------------------------ indexer + top-k
def csa_index_topk_workspace_size(B, T, N_cap, H_I, D_I, k):
    return lib().csa_index_topk_workspace_size(B, T, N_cap, H_I, D_I, k)


def csa_index_topk(iq, iq_scale, head_w, ik, ik_scale, n_valid, B, T, N_cap, H_I, D_I, k, out_idx,
                   out_score, ws, ws_bytes=None, stream=None):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().csa_index_topk(_ptr(iq), _ptr(iq_scale), _ptr(head_w), _ptr(ik), _ptr(ik_scale),
                                _ptr(n_valid), B, T, N_cap, H_I, D_I, k, _ptr(out_idx), _ptr(out_score),
                                _ptr(ws), ws_bytes, _stream(stream)))


# ------------------------------------------------------------------ attention
def hybrid_attn_decode_workspace_size(B, H, d_v, N_cap, k, W, dense):
    return lib().hybrid_attn_decode_workspace_size(B, H, d_v, N_cap, k, W, int(dense))


def hybrid_attn_decode(q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, win, W, B, H,
                       D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, ws, ws_bytes=None,
                       stream=None, *, q_rms_eps=0.0, T=1, R=0):
    """B sequences x T queries (rows b*T + j of q, q_pos, n_entries, topk_idx, out, out_lse);
    rings of R slots (0: R = W)."""
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hybrid_attn_decode(_ptr(q), _ptr(q_pos), _ptr(ckv), _ptr(ckv_scale), ckv_dtype, N_cap,
                                    _ptr(n_entries), _ptr(topk_idx), k, _ptr(win), W, B, H, D, d_rope, d_v,
                                    rope_base, softmax_scale, _ptr(out), _ptr(out_lse), _ptr(ws), ws_bytes,
                                    q_rms_eps, T, R, _stream(stream)))


def hybrid_attn_decode_append(q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, ring_x, ring_z,
                              x_new, z_new, W, B, H, D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, ws,
                              ws_bytes=None, stream=None, *, q_rms_eps=0.0, T=1, R=0):
    """cskv_ring_append of the step's T new tokens per sequence (x_new [B, T, D], z_new [B, T] or
    None) into ring_x / ring_z, then hybrid_attn_decode over ring_x, in one call."""
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hybrid_attn_decode_append(_ptr(q), _ptr(q_pos), _ptr(ckv), _ptr(ckv_scale), ckv_dtype, N_cap,
                                           _ptr(n_entries), _ptr(topk_idx), k, _ptr(ring_x), _ptr(ring_z),
                                           _ptr(x_new), _ptr(z_new), W, B, H, D, d_rope, d_v, rope_base,
                                           softmax_scale, _ptr(out), _ptr(out_lse), _ptr(ws), ws_bytes, q_rms_eps,
                                           T, R, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024   # CSKV_NOALLOC_SCRATCH_BYTES
ATTN_AUTO, ATTN_G64, ATTN_G16 = 0, 1, 2     # cskv_attn_path


def cskv_attn_path(path):
    """Which attention kernel the attention calls run (0: by shape, 1: 64-head, 2: 16-head)."""
    _check(lib().cskv_attn_path(path))


def cskv_attn_cu_budget(cus):
    """CUs the 64-head attention kernel's split plan counts on (0: the whole GPU)."""
    _check(lib().cskv_attn_cu_budget(cus))


def hybrid_attn_decode_noalloc(q, q_pos, ckv, ckv_scale, ckv_dtype, N_cap, n_entries, topk_idx, k, win, W, B, H,
                               D, d_rope, d_v, rope_base, softmax_scale, out, out_lse, stream=None, *,
                               q_rms_eps=0.0, T=1, R=0):
    """hybrid_attn_decode with the split partials in the library's static per-GPU scratch."""
    _check(lib().hybrid_attn_decode_noalloc(_ptr(q), _ptr(q_pos), _ptr(ckv), _ptr(ckv_scale), ckv_dtype, N_cap,
                                            _ptr(n_entries), _ptr(topk_idx), k, _ptr(win), W, B, H, D, d_rope,
                                            d_v, rope_base, softmax_scale, _ptr(out), _ptr(out_lse), q_rms_eps,
                                            T, R, _stream(stream)))


def hybrid_attn_prefill_workspace_size(T, H, d_v, N, k, W, dense):
    return lib().hybrid_attn_prefill_workspace_size(T, H, d_v, N, k, W, int(dense))


def hybrid_attn_prefill(q, pos0, T, ckv, ckv_scale, ckv_dtype, N, topk_idx, k, x, W, H, D, d_rope, d_v, m,
                        rope_base, softmax_scale, out, out_lse, ws, ws_bytes=None, stream=None, *, q_rms_eps=0.0):
    if ws_bytes is None:
        ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    _check(lib().hybrid_attn_prefill(_ptr(q), pos0, T, _ptr(ckv), _ptr(ckv_scale), ckv_dtype, N,
                                     _ptr(topk_idx), k, _ptr(x), W, H, D, d_rope, d_v, m, rope_base,
                                     softmax_scale, _ptr(out), _ptr(out_lse), _ptr(ws), ws_bytes,
                                     q_rms_eps, _stream(stream)))


# ------------------------------------------------------------------ decode state update
def cskv_ring_append(x_new, z_new, pos, ring_x, ring_z, B, D, R, stream=None, *, T=1):
    """T tokens per sequence (x_new [B, T, D]) into rings of R slots: slot (pos[b] + i) mod R."""
    _check(lib().cskv_ring_append(_ptr(x_new), _ptr(z_new), _ptr(pos), _ptr(ring_x), _ptr(ring_z), B, T, D, R,
                                  _stream(stream)))
