"""Pins of oracle.formats against library casts and the OCP specifications' tables."""
import os

import numpy as np
import torch

from oracle import formats

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    for line in open(os.path.join(GOLD, name)):
        line = line.strip()
        if line and not line.startswith("#"):
            a, b = line.split()[:2]
            rows.append((a, float(b)))
    return rows


def test_bf16_decode_matches_torch():
    bits = np.random.default_rng(0).integers(0, 1 << 16, 4096, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    got = formats.bf16_to_f64(bits)
    fin = np.isfinite(ref)
    assert np.array_equal(got[fin], ref[fin])


def test_bf16_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    v32 = (rng.standard_normal(20000) * np.exp2(rng.integers(-20, 20, 20000))).astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(formats.f64_to_bf16(v32.astype(np.float64)), ref)


def test_bf16_ties_round_to_even():
    # 1 + 2^-8 is halfway between bf16 1.0 and 1.0078125: RNE keeps 1.0 (even mantissa)
    assert formats.f64_to_bf16(np.array([1.0 + 2.0 ** -8]))[0] == 0x3F80
    # 1 + 3*2^-8 is halfway between 1.0078125 (odd) and 1.015625 (even): goes up
    assert formats.f64_to_bf16(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 0x3F82


def test_e4m3_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    got = formats.e4m3_to_f64(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(got[ok], ref[ok])


def test_e4m3_spec_points():
    for code, val in _read_table("ocp_e4m3fn_points.txt"):
        c = int(code, 16)
        assert formats.e4m3_to_f64(np.array([c]))[0] == val
        if c not in (0x80,):
            assert formats.f64_to_e4m3(np.array([val]))[0] == c


def test_e4m3_encode_matches_torch_in_range():
    rng = np.random.default_rng(2)
    v = (rng.uniform(-448, 448, 50000) * np.exp2(rng.integers(-12, 1, 50000))).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = formats.f64_to_e4m3(v.astype(np.float64))
    # -0 vs +0 for values that round to zero: compare decoded values
    assert np.array_equal(formats.e4m3_to_f64(got), formats.e4m3_to_f64(ref))


def test_e4m3_midpoints_round_to_even_and_saturate():
    codes = np.arange(0, 0x7E, dtype=np.uint8)
    lo = formats.e4m3_to_f64(codes)
    hi = formats.e4m3_to_f64(codes + 1)
    mid = (lo + hi) / 2
    got = formats.f64_to_e4m3(mid)
    even = np.where(codes % 2 == 0, codes, codes + 1)
    assert np.array_equal(got, even.astype(np.uint8))
    assert formats.f64_to_e4m3(np.array([460.0, 1e6, -1e6]))[0] == 0x7E
    assert formats.f64_to_e4m3(np.array([-1e6]))[0] == 0xFE


def test_e2m1_matches_ocp_mx_table():
    tab = _read_table("ocp_mx_e2m1.txt")
    assert len(tab) == 16
    for code, val in tab:
        c = int(code, 2)
        got = formats.e2m1_to_f64(np.array([c]))[0]
        assert got == val and np.signbit(got) == np.signbit(val)


def test_fp4_unpack_low_nibble_first_and_mx_scale():
    packed = np.array([[0x21, 0x7F] + [0] * 14], dtype=np.uint8)   # codes 1,2,15,7 then zeros
    scales = np.array([[128]], dtype=np.uint8)                       # 2^(128-127) = 2
    v = formats.mxfp4_to_f64(packed, scales)
    assert v.shape == (1, 32)
    assert list(v[0, :4]) == [1.0, 2.0, -12.0, 12.0]
    assert np.all(v[0, 4:] == 0)
    assert formats.e8m0_to_f64(np.array([127, 0, 254])).tolist() == [1.0, 2.0 ** -127, 2.0 ** 127]


def test_mxfp4_encode_hand_values_ties_to_even_and_saturation():
    """OCP MX v1.0 FP4 by hand: block max 6 -> E = floor(log2 6) - 2 = 0; every midpoint between
    two e2m1 magnitudes goes to the even code; beyond 6 saturates; a negative value keeps bit 3."""
    x = np.zeros((1, 32))
    x[0, :14] = [6, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 5.5, -0.75, 0.3, 0.74, 5.99, -0.1]
    p, s = formats.f64_to_mxfp4(x)
    assert s.tolist() == [[127]]
    codes = formats.unpack_fp4(p)[0, :14].tolist()
    assert codes == [7, 0, 2, 2, 4, 4, 6, 6, 7, 8 | 2, 1, 1, 7, 8 | 0]


def test_mxfp4_block_exponent_limits_and_zero_block():
    """E = floor(log2 amax) - 2 within [-3, 0]: amax 100 would need E = 4 (clipped to 0, values
    saturate at 6); amax 0.01 would need E = -9 (clipped to -3: 0.01 / 0.125 rounds to 0); amax 1
    gives E = -2 exactly (a power of two); an all-zero block takes E = -3 and zero codes."""
    x = np.zeros((4, 32))
    x[0, 0], x[0, 1] = 100.0, 2.0
    x[1, 0] = 0.01
    x[2, 0], x[2, 1] = 1.0, -0.375
    p, s = formats.f64_to_mxfp4(x)
    assert s[:, 0].tolist() == [127, 124, 125, 124]
    c = formats.unpack_fp4(p)
    assert c[0, :2].tolist() == [7, 4]          # 100 -> 6 (saturated), 2 -> 2.0
    assert c[1, 0] == 0                          # 0.08 of a step -> 0
    assert c[2, :2].tolist() == [6, 8 | 3]       # 1 / 0.25 = 4 -> code 6; -0.375 / 0.25 = -1.5 -> code 3
    assert np.all(c[3] == 0)


def test_mxfp4_round_trip_of_representable_values():
    """Every value on the e2m1 grid times 2^E (with the block maximum fixing E) decodes to itself."""
    rng = np.random.default_rng(3)
    for E in range(-3, 1):
        codes = rng.integers(0, 16, (50, 64))
        codes[:, 0] = 7                                          # block maxima 6 * 2^E fix E
        codes[:, 32] = 15
        v = formats.e2m1_to_f64(codes) * 2.0 ** E
        p, s = formats.f64_to_mxfp4(v)
        assert np.all(s == E + 127)
        back = formats.mxfp4_to_f64(p, s)
        assert np.array_equal(back, np.where(v == 0, 0.0, v))   # -0 is stored as +0 only when zero


def test_mxfp4_nearest_value_brute_force():
    """Against a brute-force search over all 16 codes: the decoded value is a nearest grid value
    of v / 2^E (clipped to +-6), and on exact midpoints the even magnitude code is taken."""
    rng = np.random.default_rng(4)
    v = rng.normal(0, 1.3, (200, 32))
    v[:, 5] = rng.choice(formats.E2M1_MIDS, 200) * rng.choice([-1, 1], 200) * 0.5   # exact midpoints
    p, s = formats.f64_to_mxfp4(v)
    E = s.astype(np.int64) - 127
    got = formats.mxfp4_to_f64(p, s) / np.repeat(2.0 ** E, 32, axis=-1)
    target = np.clip(v / np.repeat(2.0 ** E, 32, axis=-1), -6, 6)
    grid = formats.e2m1_to_f64(np.arange(16))
    dist = np.abs(target[..., None] - grid)
    assert np.allclose(np.abs(got - target), dist.min(axis=-1), rtol=0, atol=0)
    codes = formats.unpack_fp4(p)
    mids = np.isin(np.abs(target), formats.E2M1_MIDS)
    assert mids.any() and np.all((codes[mids] & 7) % 2 == 0)


def test_mxfp4_full_exponent_range_for_kv_entries():
    """KV entries use the whole E8M0 range: E = floor(log2 amax) - 2 unclipped; decoding is
    within one e2m1 step (2^(E+1) at the top of a block, after saturation at 6 * 2^E)."""
    rng = np.random.default_rng(31)
    x = rng.standard_normal((6, 64)) * np.array([1e-30, 1e-3, 1.0, 7.0, 1e4, 1e30])[:, None]
    codes, scales = formats.f64_to_mxfp4(x, formats.MX_KV_E_MIN, formats.MX_KV_E_MAX)
    amax = np.abs(x.reshape(6, 2, 32)).max(axis=-1)
    E = np.floor(np.log2(amax)) - 2
    assert np.array_equal(scales.astype(np.int64) - 127, E.astype(np.int64))
    back = formats.mxfp4_to_f64(codes, scales)
    assert np.all(np.abs(back - x) <= np.repeat(2.0 ** (E + 1), 32, axis=-1))
    # one hand value: amax 12 -> E = 1, 12 / 2 = 6 -> code 7; 5 / 2 = 2.5 ties to code 4 (2.0)
    v = np.zeros(32)
    v[0], v[1] = 12.0, -5.0
    c, s = formats.f64_to_mxfp4(v[None], formats.MX_KV_E_MIN, formats.MX_KV_E_MAX)
    assert s[0, 0] == 128 and (c[0, 0] & 0xF) == 7 and (c[0, 0] >> 4) == 0x8 | 4
