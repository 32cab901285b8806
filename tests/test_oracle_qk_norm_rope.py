"""Pins of the oracle's per-head RMSNorm + rotary embedding of Q and K.

The original engine fuses the grouped QKV projection with RMSNorm and RoPE
("Nunchaku Lite" docs, section "Fused kernels"); head size 128, adjacent
channel pairs and one rounding to bf16 are readings.  Each case below has a
closed-form answer or an invariant that a plausible slip (the mean over half
a head, the other pair layout, the opposite rotation, the Q weight on K,
touching V, dropping eps) breaks."""
import math

import numpy as np

import oracle

D, P = 128, 64


def _bf(v):
    return oracle.f64_to_bf16(np.asarray(v, np.float64))


def _f(b):
    return oracle.bf16_to_f32(np.asarray(b, np.uint16)).astype(np.float64)


def _run(y, qw=None, kw=None, eps=0.0, cos=None, sin=None):
    y = _bf(y) if y.dtype != np.uint16 else y
    M, N = y.shape
    qw = _bf(np.ones(D)) if qw is None else qw
    kw = _bf(np.ones(D)) if kw is None else kw
    cos = np.ones((M, P), np.float32) if cos is None else cos
    sin = np.zeros((M, P), np.float32) if sin is None else sin
    return oracle.qk_norm_rope(y, qw, kw, eps, cos, sin)


def test_rms_is_over_the_whole_head():
    y = np.zeros((1, 3 * D))
    y[0, :64], y[0, 64:128] = 1.0, 3.0            # Q head: rms = sqrt((64 + 576) / 128) = sqrt(5)
    y[0, 128:256] = -2.0                          # K head: rms 2
    out = _f(_run(y))
    assert np.array_equal(out[0, :64], _f(_bf(np.full(64, 1 / math.sqrt(5)))))
    assert np.array_equal(out[0, 64:128], _f(_bf(np.full(64, 3 / math.sqrt(5)))))
    assert np.array_equal(out[0, 128:256], np.full(128, -1.0))


def test_rotation_pairs_adjacent_channels_counterclockwise():
    y = np.zeros((1, 3 * D))
    y[0, 0] = 1.0                                  # Q head 0: only channel 0; n_0 = sqrt(128)
    cos = np.ones((1, P), np.float32)
    sin = np.zeros((1, P), np.float32)
    cos[0, 0], sin[0, 0] = 0.0, 1.0                # pair 0 turned by +90 degrees
    out = _f(_run(y, cos=cos, sin=sin))
    want = np.zeros(D)
    want[1] = _f(_bf([math.sqrt(128)]))[0]         # (n0, 0) -> (0, n0): channel 1, not channel 64
    assert np.array_equal(out[0, :D], want)


def test_rotation_keeps_each_pairs_length():
    rng = np.random.default_rng(3)
    M, H = 6, 2
    y = rng.standard_normal((M, 3 * H * D))
    w = _bf(rng.uniform(0.5, 1.5, D))
    th = rng.uniform(-math.pi, math.pi, (M, P))
    plain = _f(_run(y, qw=w, kw=w))
    rot = _f(_run(y, qw=w, kw=w, cos=np.cos(th).astype(np.float32), sin=np.sin(th).astype(np.float32)))
    a = plain[:, : 2 * H * D].reshape(M, -1, 2)
    b = rot[:, : 2 * H * D].reshape(M, -1, 2)
    la, lb = np.hypot(a[..., 0], a[..., 1]), np.hypot(b[..., 0], b[..., 1])
    assert np.allclose(la, lb, rtol=2 ** -6, atol=1e-30)
    # and the angle: b = R(theta) a, up to bf16 rounding
    cs = np.tile(np.cos(th), (1, 2 * H)).reshape(M, -1)
    sn = np.tile(np.sin(th), (1, 2 * H)).reshape(M, -1)
    assert np.allclose(b[..., 0], a[..., 0] * cs - a[..., 1] * sn, rtol=0, atol=2 ** -6 * la.max())


def test_q_and_k_weights_and_untouched_v():
    y = np.ones((2, 3 * 2 * D)) * 0.5
    y[:, 4 * D:] = np.arange(2 * D) * 0.25 - 7.0    # V columns
    qw, kw = _bf(np.full(D, 2.0)), _bf(np.full(D, 3.0))
    yb = _bf(y)
    out = _run(yb, qw=qw, kw=kw)
    assert np.array_equal(_f(out[:, : 2 * D]), np.full((2, 2 * D), 2.0))
    assert np.array_equal(_f(out[:, 2 * D: 4 * D]), np.full((2, 2 * D), 3.0))
    assert np.array_equal(out[:, 4 * D:], yb[:, 4 * D:])


def test_eps_enters_the_mean_square():
    y = np.full((1, 3 * D), 1e-3)
    out = _f(_run(y, eps=1e-6))                    # 1e-3 / sqrt(1e-6 + 1e-6)
    y0 = _f(_bf([1e-3]))[0]
    want = _f(_bf([y0 / math.sqrt(y0 ** 2 + 1e-6)]))[0]
    assert np.all(out[0, : 2 * D] == want) and abs(want - 1 / math.sqrt(2)) < 1e-2
    zero = _f(_run(np.zeros((1, 3 * D)), eps=1e-6))
    assert np.all(zero == 0.0)
