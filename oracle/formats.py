"""Storage formats, decoded exactly to fp64 and encoded by round-to-nearest-even.

Test infrastructure: see the package docstring.

Formats are the public definitions, written out here from their specifications:
  bf16      the top 16 bits of an IEEE binary32, 8 significant bits.
  e4m3fn    OCP 8-bit floating point (OFP8) E4M3: bias 7, no infinities,
            S.1111.111 is NaN, largest finite 448, subnormal step 2^-9.
  e2m1      OCP Microscaling (MX v1.0) FP4 element: magnitudes
            {0, 0.5, 1, 1.5, 2, 3, 4, 6}, sign in bit 3.
  E8M0      OCP MX shared scale: 2^(E-127); E = 255 is NaN.
Packing of two e2m1 codes per byte: element 2i in the low nibble of byte i.
The configurations' quantised inputs come from the CSA description in [P5]
("lightning indexer in FP4") and the stated per-entry fp8 caches.
"""
import numpy as np


def _round_sig(v, p, emin):
    """Round fp64 values to p significant bits, RNE, with subnormals below 2^emin.

    quantum = 2^(max(floor(log2|v|), emin) - (p-1)); v/quantum is exact in fp64
    (power-of-two divide) and np.rint rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.zeros_like(v)
    nz = v != 0
    e = np.floor(np.log2(np.abs(v[nz])))
    # guard floor(log2) against fp64 log2 rounding at exact powers of two
    e = np.where(np.abs(v[nz]) < 2.0 ** e, e - 1, e)
    e = np.where(np.abs(v[nz]) >= 2.0 ** (e + 1), e + 1, e)
    e = np.maximum(e, emin)
    q = 2.0 ** (e - (p - 1))
    out[nz] = np.rint(v[nz] / q) * q
    return out


# ---------------------------------------------------------------- bf16
def bf16_to_f64(bits):
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """RNE to bf16 (finite inputs within the bf16 normal range or zero)."""
    r = _round_sig(v, 8, -126)
    f = r.astype(np.float32)  # exact: r has 8 significant bits
    assert np.all(np.isfinite(f)), "bf16 overflow"
    return (f.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- e4m3fn
E4M3_MAX = 448.0


def e4m3_to_f64(codes):
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * 2.0 ** (e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return s * mag


def f64_to_e4m3(v):
    """RNE to e4m3fn with saturation to +-448 (finite inputs)."""
    v = np.asarray(v, dtype=np.float64)
    r = _round_sig(v, 4, -6)
    r = np.clip(r, -E4M3_MAX, E4M3_MAX)
    mag = np.abs(r)
    sign = np.where(np.signbit(r), 0x80, 0)
    code = np.zeros(v.shape, dtype=np.int64)
    nz = mag > 0
    e = np.floor(np.log2(mag[nz])).astype(np.int64)
    sub = e < -6
    m_norm = np.rint((mag[nz] / 2.0 ** e - 1.0) * 8).astype(np.int64)
    m_sub = np.rint(mag[nz] / 2.0 ** -9).astype(np.int64)
    cz = np.where(sub, m_sub, ((e + 7) << 3) | m_norm)
    code[nz] = cz
    return (code | sign).astype(np.uint8)


# ---------------------------------------------------------------- MXFP4
E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_to_f64(codes):
    c = np.asarray(codes, dtype=np.int64)
    return np.where(c & 8, -1.0, 1.0) * E2M1_MAG[c & 7]


def unpack_fp4(packed):
    """[..., n/2] bytes -> [..., n] codes; element 2i is the low nibble of byte i."""
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = p & 15
    out[..., 1::2] = p >> 4
    return out


def e8m0_to_f64(e):
    e = np.asarray(e, dtype=np.int64)
    assert np.all(e != 255), "E8M0 NaN scale"
    return 2.0 ** (e - 127.0)


def mxfp4_to_f64(packed, scales):
    """Decode MXFP4: packed [..., D/2] bytes, scales [..., D/32] E8M0 -> [..., D] fp64."""
    vals = e2m1_to_f64(unpack_fp4(packed))
    s = e8m0_to_f64(scales)
    D = vals.shape[-1]
    assert s.shape[-1] * 32 == D
    return vals * np.repeat(s, 32, axis=-1)


# OCP MX v1.0 encoding. The block exponent range is a reading: [-3, 0] keeps every indexer
# score exact in fp32 for unit-scale inputs (the span bound of the indexer's exactness argument),
# and it is the range the configurations' index keys use.
MX_E_MIN, MX_E_MAX = -3, 0
# the full E8M0 range, for stored KV entries (no exactness constraint there)
MX_KV_E_MIN, MX_KV_E_MAX = -127, 127
E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0])  # midpoints between magnitudes


def _floor_log2(a):
    """floor(log2 a) for a > 0, exact at powers of two."""
    e = np.floor(np.log2(a))
    e = np.where(a < 2.0 ** e, e - 1, e)
    return np.where(a >= 2.0 ** (e + 1), e + 1, e)


def e2m1_round(mag):
    """Nearest e2m1 magnitude code (0..7) of mag >= 0, ties to the even code, saturating at 6."""
    mag = np.asarray(mag, dtype=np.float64)
    code = np.searchsorted(E2M1_MIDS, mag, side="left")      # number of midpoints below mag
    at_mid = (code < 7) & (mag == E2M1_MIDS[np.minimum(code, 6)])
    # on a midpoint: between codes `code` and `code + 1`; keep the even one
    return np.where(at_mid & (code % 2 == 1), code + 1, code).astype(np.int64)


def f64_to_mxfp4(x, e_min=MX_E_MIN, e_max=MX_E_MAX):
    """MXFP4 encoding of x [..., D] (D % 32 == 0): per block of 32, shared exponent
    E = floor(log2 max|block|) - 2 (2 is the largest e2m1 exponent), limited to [e_min, e_max]
    (an all-zero block takes e_min); elements |v| / 2^E rounded to the nearest e2m1 magnitude,
    ties to the even code, saturating at 6; sign in bit 3. Returns (packed [..., D/2] with
    element 2i in the low nibble, E8M0 scales [..., D/32] = E + 127)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    assert D % 32 == 0
    xb = x.reshape(x.shape[:-1] + (D // 32, 32))
    amax = np.abs(xb).max(axis=-1)
    E = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - 2, e_min)
    E = np.clip(E, e_min, e_max).astype(np.int64)
    mag = np.abs(xb) / (2.0 ** E)[..., None]
    code = e2m1_round(mag) | np.where(np.signbit(xb) & (mag > 0), 8, 0)
    code = code.reshape(x.shape).astype(np.uint8)
    packed = (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    return packed, (E + 127).astype(np.uint8)

