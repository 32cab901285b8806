"""CPU pins of the host-side FP6 layout reference (tests/fp6_layout.py) that
the FP6 GPU tests compare against: the E2M3 format's values from its
definition, every int4 code's encoding, and the block layout on hand-built
cases."""
import numpy as np
import pytest

from tests import fp6_layout as f6


def test_e2m3_values_by_definition():
    # exponent 0: subnormals m/8; exponent e: 2^(e-1) * (1 + m/8); sign bit 5
    assert f6.e2m3_value(0b000100) == 0.5
    assert f6.e2m3_value(0b001000) == 1.0
    assert f6.e2m3_value(0b010110) == 3.5
    assert f6.e2m3_value(0b011111) == 7.5            # largest magnitude of the format
    assert f6.e2m3_value(0b111000) == -4.0
    vals = f6.e2m3_value(np.arange(32))
    assert np.all(np.diff(vals) > 0)                 # monotone over the positive codes


def test_every_int4_code_is_exact_and_round_trips():
    q = np.arange(-8, 8)
    codes = f6.e2m3_encode(q / 2.0)
    assert np.array_equal(f6.e2m3_value(codes) * 2.0, q)
    # the encodings of 0..7 and -8 written out
    assert codes[8:].tolist() == [0, 4, 8, 12, 16, 18, 20, 22]
    assert codes[0] == 32 | 24
    with pytest.raises(ValueError):
        f6.e2m3_encode(np.array([4.25]))             # 8.5 / 2 is not an int4 code


def test_block_layout_hand_case():
    # one row, one group: channel k holds code (k % 15) - 7
    q = (np.arange(64) % 15 - 7)[None, :]
    b = f6.fp6_layout_from_q(q)
    assert b.shape == (1, 48)
    words = b.view(np.uint32)[0]
    # half 0 field 0 = channel 0 = -7 -> value -3.5 -> code 32 | 22 = 54, bits 0..5 of word 0
    assert words[0] & 63 == 54
    # half 1 field 0 = channel 32: 32 % 15 - 7 = -5 -> -2.5 -> 32 | 18 = 50, bits 0..5 of word 4
    assert words[4] & 63 == 50
    # half 0 field 31 = channel 31: 31 % 15 - 7 = -6 -> -3 -> 32 | 20 = 52, bits 186..191 = word 5 of
    # the string = block word 9, bits 26..31
    assert (words[9] >> 26) & 63 == 52
    # half 1 field 31 = channel 63: 63 % 15 - 7 = -4 -> -2 -> 32 | 16 = 48, block word 11, bits 26..31
    assert (words[11] >> 26) & 63 == 48
    # field 5 straddles words 0 and 1 of the string: bits 30..35 hold channel 5 (5 - 7 = -2 -> 32 | 8 = 40)
    assert ((words[0] >> 30) | ((words[1] & 15) << 2)) & 63 == 40


def test_layout_round_trip_and_nibbles():
    rng = np.random.default_rng(3)
    q = rng.integers(-8, 8, (5, 192))
    b = f6.fp6_layout_from_q(q)
    assert b.shape == (5, 144)
    assert np.array_equal(f6.q_from_fp6_layout(b, 192), q)
    nib = np.zeros((5, 96), np.uint8)
    nib[:] = ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
    assert np.array_equal(f6.fp6_layout_from_nibbles(nib, 192), b)
