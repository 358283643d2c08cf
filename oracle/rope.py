"""Partial rotary position embedding (RoPE), adjacent-pair form, in fp64.

Test infrastructure: see the package docstring.

[P5] section "두 가지 압축 전략: CSA 및 HCA" states that both CSA and HCA use
partial RoPE; the pages give no pairing or frequency rule. Reading taken: the
RoFormer rule (Su et al., 2021) on the LAST d_rope dims of a vector, pairs
(2i, 2i+1) of that slice, theta_i = base^(-2i/d_rope), angle p*theta_i formed
in fp64. Dims [0, D - d_rope) are left untouched.
"""
import numpy as np


def inv_freq(d_rope, base):
    i = np.arange(d_rope // 2, dtype=np.float64)
    return base ** (-2.0 * i / d_rope)


def apply(u, pos, d_rope, base):
    """Rotate the last d_rope dims of u [..., D] at integer positions pos (broadcast to u[..., 0])."""
    u = np.array(u, dtype=np.float64, copy=True)
    if d_rope == 0:
        return u
    assert d_rope % 2 == 0 and d_rope <= u.shape[-1]
    D = u.shape[-1]
    pos = np.asarray(pos, dtype=np.float64)
    phi = pos[..., None] * inv_freq(d_rope, base)  # [..., d_rope/2]
    c, s = np.cos(phi), np.sin(phi)
    x0 = u[..., D - d_rope + 0::2].copy()
    x1 = u[..., D - d_rope + 1::2].copy()
    u[..., D - d_rope + 0::2] = x0 * c - x1 * s
    u[..., D - d_rope + 1::2] = x0 * s + x1 * c
    return u
