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
    # one row, one group: channel k holds code (k % 15) - 7; the row is row 0
    # of tile 0, so its chunks sit unrotated at bytes 0, 16, 32
    q = (np.arange(64) % 15 - 7)[None, :]
    b = f6.fp6_layout_from_q(q, fill=0)
    assert b.shape == (12288,)                           # one 128-row tile x one pair of groups
    words = b[:48].view(np.uint32)
    # half 0 field 0 = channel 0 = -7 -> value -3.5 -> code 32 | 22 = 54, bits 0..5 of word 0
    assert words[0] & 63 == 54
    # half 1 field 0 = channel 32: 32 % 15 - 7 = -5 -> -2.5 -> 32 | 18 = 50, bits 0..5 of chunk 1
    assert words[4] & 63 == 50
    # half 0 field 31 = channel 31: 31 % 15 - 7 = -6 -> -3 -> 32 | 20 = 52: bits 186..191 of the
    # string = its word 5, bits 26..31 = chunk 2, word 1
    assert (words[9] >> 26) & 63 == 52
    # half 1 field 31 = channel 63: 63 % 15 - 7 = -4 -> -2 -> 32 | 16 = 48: chunk 2, word 3
    assert (words[11] >> 26) & 63 == 48
    # field 5 straddles words 0 and 1 of the string: bits 30..35 hold channel 5 (5 - 7 = -2 -> 32 | 8 = 40)
    assert ((words[0] >> 30) | ((words[1] & 15) << 2)) & 63 == 40
    assert not b[48:].any()                              # the pair's second group: padding


def test_tiled_addressing_hand_cases():
    K = 256                                              # 4 groups, 2 pairs
    # row 5 (rotation 1), group 3 (pair 1, second group), chunk 2: slot (3 + 2 + 1) % 6 = 0
    assert f6.chunk_offset(5, 3, 2, K) == 1 * 12288 + 5 * 96 + 0
    # row 3 (rotation 0), group 2, chunk 1: slot 1
    assert f6.chunk_offset(3, 2, 1, K) == 12288 + 3 * 96 + 16
    # row 130: tile 1, row 2 of it; group 0, chunk 0
    assert f6.chunk_offset(130, 0, 0, K) == 2 * 12288 + 2 * 96
    # K/64 odd: 3 groups -> 2 pairs per tile, the second half-empty
    assert f6.fp6_codes_bytes(130, 192) == 2 * 2 * 12288
    # every chunk of a full tile lands on its own 16 bytes
    offs = {f6.chunk_offset(r, g, c, K) for r in range(128) for g in range(4) for c in range(3)}
    assert len(offs) == 128 * 4 * 3 and min(offs) == 0 and max(offs) == 2 * 12288 - 16


def test_rotation_and_half_swap_hand_cases():
    # p = row % 128: rot = ((p >> 2) ^ (p >> 3)) & 1, swap = ((p >> 3) ^ (p >> 4)) & 1
    assert [f6.rot(r) for r in (0, 4, 8, 12, 16, 24, 132)] == [0, 1, 1, 0, 0, 1, 1]
    assert [f6.half_swap(r) for r in (0, 8, 16, 24, 136)] == [0, 1, 1, 0, 1]
    # row 8: rotated by one chunk, so group 0's chunk 2 sits in slot 3 and
    # group 1's chunk 2 (slot 5 + 1) wraps to slot 0
    assert f6.chunk_offset(8, 0, 2, 128) == 8 * 96 + 48
    assert f6.chunk_offset(8, 1, 2, 128) == 8 * 96 + 0
    # row 8 is swapped: chunk 2 holds words 4-5 of half 1 first.  Channel 63
    # (half 1, field 31) lives in bits 26..31 of that half's word 5.
    q = np.zeros((9, 128), np.int64)
    q[8, 63] = 3                                          # 1.5 -> code 12
    q[8, 31] = -2                                         # half 0, field 31: -1 -> code 32 | 8 = 40
    b = f6.fp6_layout_from_q(q, fill=0)
    w = b[8 * 96 + 48: 8 * 96 + 64].view(np.uint32)      # the chunk in slot 3
    assert (w[1] >> 26) & 63 == 12                        # half 1 first ...
    assert (w[3] >> 26) & 63 == 40                        # ... then half 0
    assert np.array_equal(f6.q_from_fp6_layout(b, 9, 128), q)


def test_layout_round_trip_and_nibbles():
    rng = np.random.default_rng(3)
    for R, K in ((5, 192), (130, 256)):
        q = rng.integers(-8, 8, (R, K))
        b = f6.fp6_layout_from_q(q)
        assert b.shape == (f6.fp6_codes_bytes(R, K),)
        assert np.array_equal(f6.q_from_fp6_layout(b, R, K), q)
        nib = ((q[:, 0::2] & 15) | ((q[:, 1::2] & 15) << 4)).astype(np.uint8)
        assert np.array_equal(f6.fp6_layout_from_nibbles(nib, K), b)
