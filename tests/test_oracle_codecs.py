"""Pins for the oracle's number codecs (bf16, E4M3, E2M1).

Each codec is checked against something other than itself: exact rational
nearest-value search over every representable value (ties to the even
code), the OCP format definitions written as closed forms, and torch's own
conversions where torch has one.  The pages name the formats only (bf16
compute_dtype; "nvfp4" = E2M1 codes with E4M3 scales; "Nunchaku Lite" docs,
"Supported quantization types" and "NunchakuLiteQuantizationConfig").
"""
from bisect import bisect_left
from fractions import Fraction

import numpy as np
import pytest
import torch


# ---------------------------------------------------------------- helpers

def _nearest_even(values, codes, v):
    """Nearest of sorted exact ``values`` to Fraction v; on a tie the even code."""
    i = bisect_left(values, v)
    if i == 0:
        return codes[0]
    if i == len(values):
        return codes[-1]
    lo, hi = values[i - 1], values[i]
    dlo, dhi = v - lo, hi - v
    if dlo < dhi:
        return codes[i - 1]
    if dhi < dlo:
        return codes[i]
    return codes[i - 1] if codes[i - 1] % 2 == 0 else codes[i]


def _bf16_table():
    vals, codes = [], []
    for c in range(0x7F80):               # every finite non-negative bf16
        e, m = c >> 7, c & 0x7F
        v = Fraction(m, 128) * Fraction(2) ** -126 if e == 0 else \
            (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)
        vals.append(v)
        codes.append(c)
    vals.append(Fraction(2) ** 128)       # overflow candidate -> inf (even code)
    codes.append(0x7F80)
    return vals, codes


def _e4m3_table():
    vals, codes = [], []
    for c in range(0x7F):                 # 0x7F is NaN
        f, m = c >> 3, c & 7
        v = Fraction(m, 8) * Fraction(2) ** -6 if f == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (f - 7)
        vals.append(v)
        codes.append(c)
    return vals, codes


E2M1_MAGS = [Fraction(0), Fraction(1, 2), Fraction(1), Fraction(3, 2), Fraction(2),
             Fraction(3), Fraction(4), Fraction(6)]

BF16_VALS, BF16_CODES = _bf16_table()
E4M3_VALS, E4M3_CODES = _e4m3_table()


def _brute_bf16(x: float) -> int:
    v = Fraction(x)
    sign = 0x8000 if (x < 0 or (x == 0 and np.signbit(x))) else 0
    return sign | _nearest_even(BF16_VALS, BF16_CODES, abs(v))


def _brute_e4m3(x: float) -> int:
    v = Fraction(x)
    sign = 0x80 if np.signbit(x) else 0
    return sign | _nearest_even(E4M3_VALS, E4M3_CODES, abs(v))   # saturates at 448


def _brute_e2m1(x: float) -> int:
    v = Fraction(x)
    sign = 8 if np.signbit(x) else 0
    return sign | _nearest_even(E2M1_MAGS, list(range(8)), abs(v))


# ------------------------------------------------------------------- bf16

def test_bf16_decode_is_top_half_of_binary32(oracle):
    h = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    got = oracle.bf16_to_f32(h).view(np.uint32)
    assert np.array_equal(got, h.astype(np.uint32) << 16)


def test_f32_to_bf16_matches_torch(oracle):
    rng = np.random.default_rng(11)
    bits = rng.integers(0, 1 << 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    v = v[np.isfinite(v)]
    # add exact bf16 midpoints (ties) around 1.0
    v = np.concatenate([v, np.float32([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 0.0, -0.0])])
    got = oracle.f32_to_bf16(v)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # the two probes the format definition fixes
    assert oracle.f32_to_bf16(np.float32([1 + 2 ** -8]))[0] == 0x3F80         # tie -> even (1.0)
    assert oracle.f32_to_bf16(np.float32([1 + 3 * 2 ** -8]))[0] == 0x3F82     # tie -> even (1.015625)


def test_f64_to_bf16_single_rounding_brute_force(oracle):
    rng = np.random.default_rng(12)
    xs = list(rng.standard_normal(1500) * np.exp(rng.uniform(-20, 20, 1500)))
    # values that double rounding (f64 -> f32 -> bf16) would get wrong:
    # just above a bf16 midpoint by less than half an fp32 ulp
    xs += [1 + 2 ** -8 + 2 ** -40, -(1 + 2 ** -8 + 2 ** -40), 3 * (1 + 2 ** -8 + 2 ** -45)]
    # subnormal range, overflow boundary, exact midpoints
    xs += [2.0 ** -130, 3 * 2.0 ** -134, 2.0 ** -134, 2.0 ** -135, 2.0 ** -140,
           (2 - 2 ** -8) * 2.0 ** 127, (2 - 2 ** -8) * 2.0 ** 127 * (1 - 2 ** -30), 1e300, -1e300]
    for x in xs:
        got = int(oracle.f64_to_bf16(np.float64([x]))[0])
        assert got == _brute_bf16(x), (x, hex(got))
    assert int(oracle.f64_to_bf16(np.float64([1 + 2 ** -8 + 2 ** -40]))[0]) == 0x3F81


# ------------------------------------------------------------------- E4M3

def test_e4m3_decode_all_codes_match_torch(oracle):
    codes = np.arange(256, dtype=np.uint8)
    got = oracle.e4m3_to_f32(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))
    assert got[0x7E] == 448.0 and got[0x01] == 2.0 ** -9 and got[0x08] == 2.0 ** -6


def test_e4m3_encode_brute_force_and_torch(oracle):
    rng = np.random.default_rng(13)
    v = (rng.standard_normal(20000) * np.exp(rng.uniform(-9, 7, 20000))).astype(np.float32)
    mids = np.array([float((a + b) / 2) for a, b in zip(E4M3_VALS[:-1], E4M3_VALS[1:])], np.float32)
    v = np.concatenate([v, mids, -mids, np.float32([0.0, -0.0, 17.0, 464.0, 500.0, 1e6, 2 ** -10,
                                                    2 ** -11, 3 * 2 ** -11])])
    got = oracle.f32_to_e4m3(v)
    for x, g in zip(v[::7].tolist() + mids.tolist(), np.concatenate([got[::7], got[20000:20000 + len(mids)]])):
        assert int(g) == _brute_e4m3(x), (x, hex(int(g)))
    small = np.abs(v) <= 448
    ref = torch.from_numpy(v[small]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(got[small], ref)
    # 17 is the midpoint of 16 and 18 -> 16 (0x58, even mantissa); saturation; underflow
    assert [int(oracle.f32_to_e4m3(np.float32([t]))[0]) for t in (17.0, 464.0, 1e6, 2 ** -10)] == \
        [0x58, 0x7E, 0x7E, 0x00]


# ------------------------------------------------------------------- E2M1

def test_e2m1_decode_table(oracle):
    got = oracle.e2m1_to_f32(np.arange(16, dtype=np.uint8))
    mags = [float(m) for m in E2M1_MAGS]
    assert got[:8].tolist() == mags
    assert got[8:].tolist() == [-m for m in mags]
    assert np.signbit(got[8])          # code 0x8 is -0


def test_e2m1_encode_brute_force(oracle):
    rng = np.random.default_rng(14)
    v = (rng.standard_normal(5000) * 3).astype(np.float32)
    mids = [float((a + b) / 2) for a, b in zip(E2M1_MAGS[:-1], E2M1_MAGS[1:])]
    eps = [np.nextafter(np.float32(m), np.float32(0)) for m in mids] + \
          [np.nextafter(np.float32(m), np.float32(9)) for m in mids]
    v = np.concatenate([v, np.float32(mids), -np.float32(mids), np.float32(eps),
                        np.float32([0.0, -0.0, -0.1, 6.0, 7.0, 1e9, -1e9])])
    got = oracle.f32_to_e2m1(v)
    for x, g in zip(v.tolist(), got.tolist()):
        assert g == _brute_e2m1(x), (x, g)
    # ties go to the even code: 0.25->0, 0.75->1.0, 1.25->1.0, 1.75->2, 2.5->2, 3.5->4, 5->4
    assert oracle.f32_to_e2m1(np.float32(mids)).tolist() == [0, 2, 2, 4, 4, 6, 6]
    assert int(oracle.f32_to_e2m1(np.float32([-0.1]))[0]) == 0x8   # sign kept on zero
