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
