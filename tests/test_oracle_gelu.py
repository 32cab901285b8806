"""Pins of the oracle's GELU (tanh form) on bf16 values.

The original engine runs the MLP's GELU fused into its kernels ("Nunchaku
Lite" docs, section "Fused kernels").  The oracle takes the tanh form,
evaluates it in fp64 in a cancellation-free rewriting and rounds once to
bf16 (readings: the pages name neither variant nor precision).  Here it is
pinned, for every one of the 65536 bf16 inputs, to an independent
arbitrary-precision evaluation of the textbook formula
    gelu(y) = y/2 * (1 + tanh( sqrt(2/pi) * (y + 0.044715 y^3) ))
with its own rounding to bf16 written from the format's definition.
"""
import mpmath
import numpy as np

import oracle

_MP = mpmath.mp.clone()
_MP.dps = 90   # results reach 2^-133 while 1 + tanh(u) cancels down to ~1e-45


def _exact_gelu(y):
    with mpmath.workdps(90):
        y = mpmath.mpf(y)
        u = mpmath.sqrt(2 / mpmath.pi) * (y + mpmath.mpf("0.044715") * y ** 3)
        return y / 2 * (1 + mpmath.tanh(u))


def _round_bf16(v):
    """Nearest bf16 (ties to even) of an mpmath value; returns (bits,
    distance of |v| from the nearest rounding midpoint in units of the
    bf16 spacing there)."""
    with mpmath.workdps(90):
        sign = 0x8000 if v < 0 else 0
        a = abs(v)
        if a == 0:
            return sign, mpmath.mpf(0.5)
        _, e = mpmath.frexp(a)             # a in [2^(e-1), 2^e)
        ex = max(int(e) - 1, -126)         # fixed spacing 2^-133 below 2^-126
        q = a / mpmath.ldexp(1, ex - 7)    # exact: a power-of-two scaling
        fl = mpmath.floor(q)
        frac = q - fl
        n = int(fl) + (1 if frac > 0.5 or (frac == 0.5 and int(fl) % 2 == 1) else 0)
        dist = abs(frac - mpmath.mpf(0.5))
        if ex == -126 and n < 128:         # subnormal
            return sign | n, dist
        if n == 256:                       # carried into the next binade
            ex, n = ex + 1, 128
        if ex > 127:
            return sign | 0x7F80, dist
        return sign | ((ex + 127) << 7) | (n - 128), dist


def test_gelu_matches_arbitrary_precision_for_every_bf16():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.gelu_tanh_bf16(bits)
    vals = oracle.bf16_to_f32(bits)
    finite = np.isfinite(vals)
    mismatches = []
    min_dist = mpmath.mpf(1)
    for i in np.nonzero(finite)[0]:
        y = float(vals[i])
        v = _exact_gelu(y)
        want, dist = _round_bf16(v)
        if v == 0:
            # y = 0, or 1 + tanh(u) cancelled to 0 at this precision (|v| below
            # |y| 1e-90, far under half the least subnormal): a zero with
            # the sign of y, as gelu(y) = y sigma(2u) has
            want = int(bits[i]) & 0x8000
        if int(got[i]) != want:
            mismatches.append((hex(int(bits[i])), hex(int(got[i])), hex(want)))
        if abs(y) >= 2.0 ** -100 and want & 0x7FFF:
            min_dist = min(min_dist, dist)
    assert not mismatches, f"{len(mismatches)} inputs differ, e.g. {mismatches[:5]}"
    # Away from the tiny-input ties no exact value comes within 2^-13 of a
    # spacing of a rounding midpoint (the closest, ~2^-12.6, is at y ~ 0.52):
    # any evaluation whose error stays below that rounds every input
    # correctly -- fp64 (error ~2^-44 spacings) with a wide margin.
    assert min_dist > 2.0 ** -13, float(min_dist)


def test_gelu_nonfinite_and_signed_zero():
    x = np.array([0x7F80, 0xFF80, 0x7FC0, 0xFFC1, 0x0000, 0x8000], np.uint16)
    y = oracle.gelu_tanh_bf16(x)
    assert y[0] == 0x7F80                  # +inf
    assert y[1] == 0x8000                  # -inf -> -0 (the limit)
    assert (y[2] & 0x7F80) == 0x7F80 and (y[2] & 0x7F)    # NaN stays NaN
    assert (y[3] & 0x7F80) == 0x7F80 and (y[3] & 0x7F)
    assert y[4] == 0x0000 and y[5] == 0x8000


def test_gelu_tiny_inputs_round_toward_the_positive_correction():
    """For tiny y, gelu(y) = y/2 + (positive term far below one spacing):
    an exact half-spacing y/2 rounds up (toward +infinity)."""
    x = np.array([0x0001, 0x8001, 0x0003, 0x8003, 0x0081, 0x8081, 0x0002, 0x8002], np.uint16)
    want = np.array([0x0001, 0x8000, 0x0002, 0x8001, 0x0041, 0x8040, 0x0001, 0x8001], np.uint16)
    assert np.array_equal(oracle.gelu_tanh_bf16(x), want)


def test_gelu_quantize_act_is_quantize_of_gelu():
    rng = np.random.default_rng(7)
    from bit_w4a4_quantized_svdq_amd import synth
    x = synth.to_bf16_bits(rng.standard_normal((5, 128)) * 2)
    sm = synth.to_bf16_bits(rng.uniform(0.5, 2.0, 128))
    ld = synth.to_bf16_bits(rng.standard_normal((16, 128)) * 0.05)
    a = oracle.gelu_quantize_act(oracle.INT4, x, sm, ld)
    b = oracle.quantize_act(oracle.INT4, oracle.gelu_tanh_bf16(x), sm, ld)
    for u, v in zip(a, b):
        assert np.array_equal(u, v)
