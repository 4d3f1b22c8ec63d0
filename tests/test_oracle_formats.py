"""Pins for the oracle's number-format encoders (CPU only).

Each encoder is checked against something other than itself: hand-worked fixtures under
tests/golden/, torch's own FP8/BF16 casts (library routines), and brute-force nearest
searches over the whole value set written independently here with exact rationals.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from conftest import parse_golden


def _golden_pairs(name):
    out = []
    for row in parse_golden(name):
        parts = row.split()
        out.append((float.fromhex(parts[0]), int(parts[1], 16 if "rceil" not in name else 10)))
    return out


# ---- E4M3 -----------------------------------------------------------------------

def _e4m3_values_exact():
    """All 127 non-negative finite E4M3 magnitudes as Fractions, from the bit layout."""
    vals = []
    for c in range(0x7F):
        e, m = c >> 3, c & 7
        vals.append(Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7))
    return vals


E4M3 = _e4m3_values_exact()


def _brute_e4m3(y: float) -> int:
    """Independent nearest search: exact rational distance to every code, ties -> even."""
    if y != y:
        return 0x7F
    s = 0x80 if np.signbit(y) else 0
    a = Fraction(abs(y))
    if a >= 448:
        return s | 0x7E
    best = min(range(0x7F), key=lambda c: (abs(E4M3[c] - a), c % 2))
    return s | best


def test_e4m3_golden():
    for v, code in _golden_pairs("e4m3_hand.txt"):
        assert int(oracle.e4m3_from_f64([v])[0]) == code, (v.hex(), hex(code))


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_to_f64(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def test_e4m3_encode_matches_torch_cast():
    """torch's float32 -> float8_e4m3fn cast rounds to nearest even; it agrees with the
    oracle on every FP32 value up to 464 (above that torch gives NaN, the oracle saturates)."""
    rng = np.random.default_rng(1)
    mags = [E4M3[c] for c in range(0x7F)]
    mids = [(mags[i] + mags[i + 1]) / 2 for i in range(0x7E)]
    pts = []
    for q in mags + mids:
        f = float(q)
        pts += [f, np.nextafter(np.float32(f), np.float32(0)), np.nextafter(np.float32(f), np.float32(1e9))]
    rnd = np.concatenate([
        rng.uniform(0, 448, 200000),
        np.exp2(rng.uniform(-20, 8.8, 200000)),
        rng.uniform(0, 2.0 ** -6, 50000),
    ])
    x = np.concatenate([np.array(pts, np.float64), rnd]).astype(np.float32)
    x = x[np.abs(x) <= 464]
    x = np.concatenate([x, -x])
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_from_f64(x.astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(x[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_e4m3_brute_force_nearest():
    rng = np.random.default_rng(2)
    y = np.concatenate([rng.normal(0, 100, 3000), np.exp2(rng.uniform(-14, 10, 3000)) * rng.choice([-1, 1], 3000)])
    got = oracle.e4m3_from_f64(y)
    for yi, gi in zip(y, got):
        assert int(gi) == _brute_e4m3(float(yi)), float(yi)


# ---- E2M1 -----------------------------------------------------------------------

E2M1 = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2), Fraction(3), Fraction(4), Fraction(6)]


def _brute_e2m1(y: float) -> int:
    s = 0x8 if np.signbit(y) else 0
    a = Fraction(abs(y))
    if a >= 6:
        return s | 7
    return s | min(range(8), key=lambda c: (abs(E2M1[c] - a), c % 2))


def test_e2m1_golden():
    for v, code in _golden_pairs("e2m1_hand.txt"):
        assert int(oracle.e2m1_from_f64([v])[0]) == code, (v.hex(), hex(code))


def test_e2m1_decode_table():
    got = oracle.e2m1_to_f64(np.arange(16, dtype=np.uint8))
    want = [float(v) for v in E2M1] + [-float(v) for v in E2M1]
    assert list(got) == want
    assert np.signbit(got[8])


def test_e2m1_brute_force_nearest():
    rng = np.random.default_rng(3)
    y = np.concatenate([rng.uniform(-8, 8, 20000), [float(v) for v in E2M1],
                        [float((E2M1[i] + E2M1[i + 1]) / 2) for i in range(7)]])
    got = oracle.e2m1_from_f64(y)
    for yi, gi in zip(y, got):
        assert int(gi) == _brute_e2m1(float(yi)), float(yi)


# ---- BF16 -----------------------------------------------------------------------

def test_bf16_matches_torch_cast_on_fp32():
    """torch's float32 -> bfloat16 cast is round-to-nearest-even; for inputs that are
    FP32 values the oracle's binary64 rounding must agree bit for bit."""
    rng = np.random.default_rng(4)
    bits = rng.integers(0, 1 << 32, 1 << 21, dtype=np.uint64).astype(np.uint32)
    # every tie and near-tie pattern in the low 16 bits, over a spread of exponents
    hi = rng.integers(0, 1 << 16, 4096, dtype=np.uint32) << 16
    lows = np.array([0x7FFF, 0x8000, 0x8001, 0x0000, 0xFFFF, 0x0001], np.uint32)
    bits = np.concatenate([bits, (hi[:, None] | lows[None, :]).ravel()])
    x = bits.view(np.float32)
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_from_f64(x.astype(np.float64))
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(float(x[i]), hex(ref[i]), hex(got[i])) for i in bad[:5]]


def test_bf16_nearest_on_binary64():
    """Binary64 inputs that are not FP32 values: the code's value is the nearest BF16,
    ties to even, checked against both neighbours with exact rationals."""
    rng = np.random.default_rng(5)
    v = rng.normal(0, 1, 3000) * np.exp2(rng.integers(-140, 120, 3000))
    got = oracle.bf16_from_f64(v)
    dec = oracle.bf16_to_f64(got)
    for vi, gi, di in zip(v, got, dec):
        a = Fraction(float(vi))
        d = Fraction(float(di))
        for nb in (int(gi) - 1, int(gi) + 1):
            if (nb & 0x7FFF) >= 0x7F80 or nb < 0 or nb > 0xFFFF:
                continue
            dn = Fraction(float(oracle.bf16_to_f64([nb])[0]))
            assert abs(a - d) < abs(a - dn) or (abs(a - d) == abs(a - dn) and int(gi) % 2 == 0)


def test_bf16_overflow_and_specials():
    big = float(np.float32(3.3961e38))
    assert int(oracle.bf16_from_f64([1e39])[0]) == 0x7F80
    assert int(oracle.bf16_from_f64([-1e39])[0]) == 0xFF80
    assert int(oracle.bf16_from_f64([0.0])[0]) == 0x0000
    assert int(oracle.bf16_from_f64([-0.0])[0]) == 0x8000
    assert int(oracle.bf16_from_f64([2.0 ** -133])[0]) == 0x0001
    assert int(oracle.bf16_from_f64([2.0 ** -134])[0]) == 0x0000  # tie -> even (zero)
    assert int(oracle.bf16_from_f64([3 * 2.0 ** -134])[0]) == 0x0002  # tie 1/2 -> even 2
    assert int(oracle.bf16_from_f64([big])[0]) in (0x7F7F, 0x7F80)
    # (2 - 2^-8) * 2^127 is the tie between the largest finite BF16 and 2^128: goes to Inf
    assert int(oracle.bf16_from_f64([(2 - 2.0 ** -8) * 2.0 ** 127])[0]) == 0x7F80
    assert int(oracle.bf16_from_f64([(2 - 2.0 ** -7) * 2.0 ** 127])[0]) == 0x7F7F


# ---- RCEIL E8M0 -------------------------------------------------------------------

def _brute_rceil(amax: float) -> int:
    a = Fraction(amax)
    for e in range(-127, 128):
        if 448 * Fraction(2) ** e >= a:
            return e
    return 127


def test_rceil_golden():
    for v, byte in _golden_pairs("rceil_hand.txt"):
        assert oracle.mx_scale_exponent(v) + 127 == byte, (v.hex(), byte)


def test_rceil_brute_force():
    rng = np.random.default_rng(6)
    amax = np.abs(np.concatenate([
        rng.normal(0, 1, 500) * np.exp2(rng.integers(-149, 128, 500)),
        [448.0 * 2.0 ** k for k in range(-127, 120, 7)],
        [np.nextafter(448.0 * 2.0 ** k, 1e300) for k in range(-127, 120, 7)],
    ]))
    amax = amax[np.isfinite(amax)]
    for a in amax:
        assert oracle.mx_scale_exponent(float(a)) == _brute_rceil(float(a)), float(a)


def test_rceil_all_bf16_amax():
    """Every non-negative finite BF16 amax against FP64 ceil(log2(amax/448)), clamped."""
    import math
    for b in range(0, 0x7F80, 7):
        a = float(oracle.bf16_to_f64([b])[0])
        want = -127 if a == 0 else max(-127, min(127, math.ceil(math.log2(a / 448.0))))
        # log2 in binary64 is exact at powers of two, which are the only boundary cases
        assert oracle.mx_scale_exponent(a) == want, (hex(b), a)
