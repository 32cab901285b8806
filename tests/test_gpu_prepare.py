"""Offline weight preparation on the GPU against the oracle: smoothing
factors and the 4-bit residual's codes and scales, bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.gpu_helpers import announce, empty, poison, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gpu_smooth(x, W):
    s = poison(empty((x.shape[1],), "bf16"))
    capi.svdq_smooth_factors(to_dev(x, "bf16"), to_dev(W, "bf16"), s)
    torch.cuda.synchronize()
    return to_host(s, "bf16")


def _gpu_qweight(prec, W, smooth, up, down):
    N, K = W.shape
    codes = poison(empty((N, K // 2), "u8"))
    scales = poison(empty((N, K // 64), "bf16") if prec == 0 else empty((N, K // 16), "u8"))
    capi.svdq_quantize_weight(prec, to_dev(W, "bf16"), to_dev(smooth, "bf16"), to_dev(up, "bf16"),
                              to_dev(down, "bf16"), codes, scales)
    torch.cuda.synchronize()
    return to_host(codes, "u8"), to_host(scales, "bf16" if prec == 0 else "u8")


@pytest.mark.parametrize("M,N,K", [(200, 96, 448), (1, 1, 64), (33, 257, 4160)])
def test_smooth_factors_exact(M, N, K):
    rng = np.random.default_rng(5000 + M + N + K)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 50), replace=False)] *= 80.0
    W = rng.standard_normal((N, K)) * 0.02
    x[:, 3] = 0.0                                   # a column never activated: factor 1
    W[:, 5] = 0.0                                   # a weight column of zeros: factor 1
    x, W = synth.to_bf16_bits(x), synth.to_bf16_bits(W)
    x[0, 7] = 0x8000                                # -0 counts as 0
    announce("smooth_factors", M, N, K)
    assert np.array_equal(_gpu_smooth(x, W), oracle.smooth_factors(x, W))


def test_smooth_factors_fullsize_mlp_up():
    cfg = synth.MLP_UP
    case = synth.linear_case(cfg)
    announce("smooth_factors fullsize", cfg.name)
    assert np.array_equal(_gpu_smooth(case["x"], case["W"]), oracle.smooth_factors(case["x"], case["W"]))


@pytest.mark.parametrize("prec,N,K,rank,smooth", [
    (0, 64, 256, 16, True), (0, 33, 4160, 32, True), (0, 130, 192, 0, False), (0, 96, 640, 48, True),
    (1, 64, 256, 16, True), (1, 33, 4160, 32, True), (1, 130, 192, 0, False), (1, 96, 640, 48, False),
])
def test_quantize_weight_matches_oracle_preparation(prec, N, K, rank, smooth):
    """The oracle prepares the layer (smoothing, exact SVD branch, residual
    quantization); the GPU redoes the residual and its quantization from the
    same smoothing factors and branch."""
    rng = np.random.default_rng(6000 + N + K + rank + prec)
    x = synth.to_bf16_bits(rng.standard_normal((64, K)) * np.exp(rng.standard_normal(K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    p = oracle.prepare_svdq_weight(prec, x, W, rank, smooth=smooth)
    announce("quantize_weight", "prec", prec, N, K, "rank", rank)
    codes, scales = _gpu_qweight(prec, W, p["smooth"], p["lora_up"], p["lora_down"])
    assert np.array_equal(scales, p["wgt_scales"]), f"scales differ at {np.argwhere(scales != p['wgt_scales'])[:5].tolist()}"
    assert np.array_equal(codes, p["wgt_codes"]), f"codes differ at {np.argwhere(codes != p['wgt_codes'])[:5].tolist()}"


@pytest.mark.parametrize("prec", [0, 1])
def test_quantize_weight_edge_groups(prec):
    """Exact rounding ties (scale 1), zero and tiny groups, E4M3 saturation."""
    K = 128
    rows = [np.tile([7.0, 0.5, 1.5, 2.5, -0.5, -3.5, 4.5, -6.5], K // 8),            # int4 ties, scale 1
            np.tile([6.0, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.25, 0.0, -0.0, 3.0, 1.5, -6.0, 4.0],
                    K // 16),                                                         # E2M1 ties, scale 1
            np.zeros(K), np.tile([1e-38, -3e-39, 2e-40, 0.0], K // 4),
            np.tile([6000.0, -3000.0, 1.0, 0.5], K // 4), np.linspace(-300.0, 300.0, K)]
    W = synth.to_bf16_bits(np.stack(rows))
    W[2, 9] = 0x8000
    announce("quantize_weight edges", "prec", prec)
    codes, scales = _gpu_qweight(prec, W, None, None, None)
    R = oracle.svdq_residual(W, np.full(K, 0x3F80, np.uint16), None, None)
    oc, os_ = oracle.quantize_int4(R) if prec == 0 else oracle.quantize_nvfp4(R)
    assert np.array_equal(scales, os_)
    assert np.array_equal(codes, oc)


def test_quantize_weight_fullsize_qkv():
    """The grouped QKV weight (9216 x 3072, rank 32) with a given branch."""
    N, K, r = 9216, 3072, 32
    rng = np.random.default_rng(77)
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    s = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.4))
    up = synth.to_bf16_bits(rng.standard_normal((N, r)) / np.sqrt(N))
    down = synth.to_bf16_bits(rng.standard_normal((r, K)) * 0.05)
    announce("quantize_weight fullsize qkv")
    codes, scales = _gpu_qweight(0, W, s, up, down)
    oc, os_ = oracle.quantize_int4(oracle.svdq_residual(W, s, up, down))
    assert np.array_equal(scales, os_)
    assert np.array_equal(codes, oc)
