"""Pins of the oracle's W12 format (lossless 12-bit storage of bf16 weights).

The SpecPilot digest (airadar.tv — "Reasons") names the format: each bf16 weight split into three
4-bit planes and rebuilt bit for bit in the GEMM's registers, with no loss. The reading the oracle
implements (one even exponent window of 16 fields per matrix, plane 2 = sign and the offset of
the exponent's upper bits, everything else an exception kept at full width) is pinned here by
what must hold independently of how it is coded:
  * lossless: decoding returns every one of the 65536 bf16 bit patterns exactly, at every base;
  * the exception set, computed in the float domain (a normal value fits iff
    2^(b-127) <= |v| < 2^(b-111)), matches the oracle's flags;
  * the window it picks is the brute-force best over all bases (fewest exceptions, lowest base);
  * on N(0, 0.02) weights the exception fraction matches the normal distribution's tails;
  * 12 bits per value: the planes hold 1.5 bytes per value, plus the exceptions;
  * hand-worked codes.
"""
import math

import numpy as np
import pytest

import oracle

ALL = np.arange(65536, dtype=np.uint16)


def as_float(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def fits_float_domain(bits: np.ndarray, b: int) -> np.ndarray:
    """Whether each bf16 value's exponent lies in the window [b, b + 15], decided from the value:
    normal numbers by magnitude, zero/subnormals (field 0) and inf/nan (field 255) by class."""
    with np.errstate(invalid="ignore"):
        f = as_float(bits).astype(np.float64)
        a = np.abs(f)
        normal = np.isfinite(f) & (a >= 2.0 ** -126)
        tiny = np.isfinite(f) & (a < 2.0 ** -126)
        out = np.zeros(bits.shape, bool)
        out[normal] = (a[normal] >= 2.0 ** (b - 127)) & (a[normal] < 2.0 ** (b - 111))
    out[tiny] = b == 0
    out[~np.isfinite(f)] = b == 240
    return out


@pytest.mark.parametrize("b", list(range(0, 241, 2)))
def test_w12_lossless_every_pattern(b):
    c = oracle.w12_encode(ALL, b)
    assert c.base == b
    np.testing.assert_array_equal(oracle.w12_decode(c), ALL)
    # 16 exponent fields x 2 signs x 128 mantissas fit; the rest are exceptions
    assert c.esc_idx.size == 65536 - 16 * 256
    esc = np.zeros(65536, bool)
    esc[c.esc_idx] = True
    np.testing.assert_array_equal(~esc, fits_float_domain(ALL, b))
    assert np.all(c.nib[esc] == 0)
    assert np.all(c.nib < 16)


def test_w12_decode_ignores_planes_of_exceptions():
    # whatever the planes hold for an exception, the listed value wins
    c = oracle.w12_encode(ALL, 118)
    c.lo = c.lo.copy()
    c.nib = c.nib.copy()
    c.lo[c.esc_idx] = 0x5a
    c.nib[c.esc_idx] = 0x7
    np.testing.assert_array_equal(oracle.w12_decode(c), ALL)


def test_w12_hand_codes():
    # -2^-7 = 0xBC00: s = 1, e = 120, m = 0; base 116 -> low byte 0, plane 2 = 8 | (4 >> 1)
    c = oracle.w12_encode(np.array([0xBC00, 0x3F80, 0x3C01, 0x0000], np.uint16), 116)
    assert c.lo.tolist() == [0x00, 0x80, 0x01, 0x00]
    # 1.0 = 0x3F80: e = 127, inside [116, 131], (127 - 116) >> 1 = 5; 0x3C01: e = 120 -> 2
    assert c.nib.tolist()[:3] == [8 | 2, 5, 2]
    # zero (field 0) is an exception for any base but 0
    assert c.esc_idx.tolist() == [3]
    assert c.esc_val.tolist() == [0]


def brute_base(bits):
    best, best_b = -1, None
    for b in range(0, 241, 2):
        n = int(fits_float_domain(bits, b).sum())
        if n > best:
            best, best_b = n, b
    return best_b


@pytest.mark.parametrize("sigma", [0.02, 1.0, 1e-3, 300.0, 3e-30])
def test_w12_base_is_brute_force_best(sigma):
    rng = np.random.default_rng(7)
    w = oracle.to_bf16((rng.standard_normal(20000) * sigma).astype(np.float32))
    assert oracle.w12_base(w) == brute_base(w)


def test_w12_base_tie_takes_lowest():
    # two clusters 32 fields apart, equal sizes: the windows covering either tie -> lowest base
    lo = oracle.to_bf16(np.full(100, 2.0 ** -20, np.float32))
    hi = oracle.to_bf16(np.full(100, 2.0 ** 12, np.float32))
    w = np.concatenate([lo, hi])
    b = oracle.w12_base(w)
    assert b == brute_base(w)
    c = oracle.w12_encode(w)
    assert c.esc_idx.tolist() == list(range(100, 200))


def test_w12_normal_weights_tail_fraction():
    """N(0, 0.02) weights: the exceptions are the values below 2^(b-127) or at least 2^(b-111) in
    magnitude, so their fraction is the normal law's mass there (bf16 rounding moves a value
    across a power of two only within half an ulp, which is negligible here)."""
    n = 1 << 22
    rng = np.random.default_rng(11)
    w = oracle.to_bf16((rng.standard_normal(n) * 0.02).astype(np.float32))
    c = oracle.w12_encode(w)
    np.testing.assert_array_equal(oracle.w12_decode(c), w)
    b = c.base
    lo, hi = 2.0 ** (b - 127) / 0.02, 2.0 ** (b - 111) / 0.02
    p = math.erf(lo / math.sqrt(2)) + math.erfc(hi / math.sqrt(2))
    got = c.esc_idx.size / n
    assert abs(got - p) <= 5 * math.sqrt(p * (1 - p) / n) + 1e-7, (got, p)
    # the window keeps almost everything: about 1e-4 of N(0, 0.02) weights are exceptions
    assert 1e-5 < got < 1e-3
    # 12 bits per value in the planes
    assert c.lo.nbytes + c.nib.nbytes / 2 == 1.5 * n
