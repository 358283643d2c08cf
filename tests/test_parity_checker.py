"""The parity checks must reject planted mistakes (planted in oracle outputs, on the CPU)."""
import numpy as np
import pytest

from oracle import attention, formats, indexer, topk
from tests import parity


@pytest.fixture(scope="module")
def oracle_case():
    rng = np.random.default_rng(0)
    iq = rng.integers(0, 256, (1, 4, 32), dtype=np.uint8)
    ik = rng.integers(0, 256, (1024, 32), dtype=np.uint8)
    sc = indexer.scores(iq, np.full((1, 4, 2), 127, np.uint8), ik, np.full((1024, 2), 127, np.uint8), np.array([1024]))
    idx, s = topk.topk(sc, 128)
    H, D = 16, 64
    ckv = formats.f64_to_bf16(rng.standard_normal((1024, D)) / 8)
    ring = formats.f64_to_bf16(rng.standard_normal((128, D)) / 8)
    q = formats.f64_to_bf16(rng.standard_normal((H, D)))
    o, _ = attention.decode_one(q, 4095, attention.Entries(ckv, None, "bf16"), 1024, idx[0], ring, 128, 32, D,
                                10000.0, 1 / 8)
    return idx, s, o


def test_checker_accepts_the_oracle_itself(oracle_case):
    idx, _, o = oracle_case
    parity.topk_exact(idx, idx)
    parity.attn_close(formats.f64_to_bf16(o), o)


def test_checker_rejects_one_swapped_index(oracle_case):
    idx, _, _ = oracle_case
    bad = idx.copy()
    bad[0, [3, 4]] = bad[0, [4, 3]]
    with pytest.raises(parity.ParityError):
        parity.topk_exact(bad, idx)


def test_checker_rejects_a_flipped_tie_order(oracle_case):
    idx, s, _ = oracle_case
    ties = [i for i in range(127) if s[0, i] == s[0, i + 1]]
    assert ties, "fixture should contain tied scores"
    bad = idx.copy()
    i = ties[0]
    bad[0, [i, i + 1]] = bad[0, [i + 1, i]]
    with pytest.raises(parity.ParityError):
        parity.topk_exact(bad, idx)


def test_checker_rejects_a_replaced_entry(oracle_case):
    idx, _, _ = oracle_case
    bad = idx.copy()
    bad[0, -1] = next(j for j in range(1024) if j not in set(idx[0].tolist()))
    with pytest.raises(parity.ParityError):
        parity.topk_exact(bad, idx)


def test_checker_rejects_output_off_by_6e3_relative(oracle_case):
    _, _, o = oracle_case
    rng = np.random.default_rng(1)
    noise = rng.standard_normal(o.shape)
    noise *= 6e-3 * np.linalg.norm(o) / np.linalg.norm(noise)
    with pytest.raises(parity.ParityError):
        parity.attn_close(formats.f64_to_bf16(o + noise), o)


def test_compress_checks_reject_errors_beyond_the_fp32_bound():
    from oracle import compress as ocomp
    rng = np.random.default_rng(2)
    m, D = 4, 64
    x = formats.f64_to_bf16(rng.standard_normal((8 * m, D)))
    z = rng.standard_normal(8 * m).astype(np.float32)
    e, stored, _ = ocomp.compress(x, z, 0, m, 16, 10000.0, "bf16")
    mag = ocomp.magnitude(x, z, m, 16)
    parity.compress_bf16_close(stored, e, mag, m)
    bad = stored.copy()
    bad[3, 5] = np.uint16(int(bad[3, 5]) + 2)                  # two ulp away
    with pytest.raises(parity.ParityError):
        parity.compress_bf16_close(bad, e, mag, m)
    _, codes, s = ocomp.compress(x, z, 0, m, 16, 10000.0, "fp8")
    parity.compress_fp8_close(codes, s, e, mag, m)
    with pytest.raises(parity.ParityError):
        parity.compress_fp8_close(codes, s * (1 + 1e-4), e, mag, m)
    badc = codes.copy()
    badc[2, 7] = np.uint8(int(badc[2, 7]) + 1 if badc[2, 7] & 0x7F < 0x7E else int(badc[2, 7]) - 1)
    with pytest.raises(parity.ParityError):
        parity.compress_fp8_close(badc, s, e, mag, m)


def test_rms_bound_rejects_a_missing_or_wrong_normalisation():
    """The normalised-entry bound accepts the oracle's own rounding and rejects the unnormalised
    entry and one normalised with a 1% larger factor (planted in oracle outputs)."""
    from oracle import compress
    rng = np.random.default_rng(5)
    m, D, dr = 4, 128, 64
    x = formats.f64_to_bf16(rng.standard_normal((8 * m, D)) * 0.3)
    z = rng.standard_normal(8 * m).astype(np.float32)
    e, bits, _ = compress.compress(x, z, 40, m, dr, 10000.0, "bf16", rms_eps=1e-6)
    e0, bits0, _ = compress.compress(x, z, 40, m, dr, 10000.0, "bf16")
    mag = compress.magnitude(x, z, m, dr)
    v = compress.pool(formats.bf16_to_f64(x), z.astype(np.float64), m)
    d = parity.rms_error_bound(v, mag, e, m, dr, 1e-6)
    parity.compress_bf16_close(bits, e, mag, m, d=d)
    with pytest.raises(parity.ParityError):
        parity.compress_bf16_close(bits0, e, mag, m, d=d)
    with pytest.raises(parity.ParityError):
        parity.compress_bf16_close(formats.f64_to_bf16(e * 1.01), e, mag, m, d=d)
