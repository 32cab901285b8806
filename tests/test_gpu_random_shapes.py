"""Seeded random shapes through the whole layer on the GPU, against the
oracle: the activation step (plain or GELU-fed) with its codes, scales and
low-rank product checked, then the 4-bit GEMM fed with the GPU's own codes,
and the AWQ layer at random M (GEMV or GEMM regime).  The shapes are drawn
once from a fixed seed, so every run checks the same cases; each case prints
its parameters before its GPU calls."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import synth
from tests.fp6_layout import fp6_layout_from_nibbles
from tests.gpu_helpers import (announce, assert_bf16_close, assert_f32_close, gpu_gemm, gpu_gemv,
                               gpu_quantize)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _w4a4_cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        prec = int(rng.integers(0, 2))
        M = int(rng.integers(1, 261))
        N = int(rng.integers(1, 401))
        K = 64 * int(rng.integers(1, 71))
        rank = 16 * int(rng.integers(0, 9))
        out.append((i, prec, M, N, K, rank, bool(rng.integers(0, 2)), bool(rng.integers(0, 4) == 0)))
    return out


def _awq_cases(n=10, seed=20261204):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.choice([1, 2, 3, 5, 8, 13, 21, 32, 47, 96]))
        N = int(rng.integers(1, 300))
        K = 64 * int(rng.integers(1, 80))
        out.append((i, M, N, K, bool(rng.integers(0, 2))))
    return out


@pytest.mark.parametrize("i,prec,M,N,K,rank,with_bias,gelu", _w4a4_cases())
def test_random_layer_shapes(i, prec, M, N, K, rank, with_bias, gelu):
    rng = np.random.default_rng(5000 + i)
    x = rng.standard_normal((M, K))
    x[:, rng.choice(K, max(1, K // 100), replace=False)] *= 50.0
    if gelu:
        x *= 3.0                                   # pre-activations of a GELU MLP
    xb = synth.to_bf16_bits(x)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.5))
    w = synth.synthetic_w4a4_weights(6000 + i, N, K, rank, "int4" if prec == 0 else "nvfp4")
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    announce("random layer", i, "prec", prec, "M,N,K,r", M, N, K, rank, "bias", with_bias, "gelu", gelu)

    gc, gs, gt = gpu_quantize(prec, xb, smooth, w["lora_down"], K, gelu=gelu)
    if gelu:
        oc, os_, ot = oracle.gelu_quantize_act(prec, xb, smooth, w["lora_down"])
    else:
        oc, os_, ot = oracle.quantize_act(prec, xb, smooth, w["lora_down"])
    assert np.array_equal(gs, os_), f"case {i}: scales differ at {np.argwhere(gs != os_)[:5].tolist()}"
    assert np.array_equal(gc, oc), f"case {i}: codes differ at {np.argwhere(gc != oc)[:5].tolist()}"
    if rank:
        assert_f32_close(gt, ot, 1e-5, f"case {i} lora_act")

    y = gpu_gemm(prec, gc, gs, w["wgt_codes"], w["wgt_scales"], gt if rank else None,
                 w["lora_up"], bias)
    ref = oracle.gemm_w4a4(prec, oc, os_, w["wgt_codes"], w["wgt_scales"], ot if rank else None,
                           w["lora_up"], bias)
    assert_bf16_close(y, ref, f"case {i} out")
    if prec == 0:
        yp = gpu_gemm(prec, gc, gs, w["wgt_codes"], w["wgt_scales"], gt if rank else None, w["lora_up"], bias,
                      packed=True)
        assert_bf16_close(yp, ref, f"case {i} packed out")
        # the FP6 chain: the activation step's FP6 output into the FP6 GEMM
        fc, fs, ft = gpu_quantize(3, xb, smooth, w["lora_down"], K, gelu=gelu)
        assert np.array_equal(fs, os_), f"case {i} fp6: scales differ"
        assert np.array_equal(fc, fp6_layout_from_nibbles(oc, K)), f"case {i} fp6: code bytes differ"
        yf = gpu_gemm(prec, gc, gs, w["wgt_codes"], w["wgt_scales"], ft if rank else None, w["lora_up"], bias,
                      fp6=True, act_fp6=fc)
        assert_bf16_close(yf, ref, f"case {i} fp6 out")


@pytest.mark.parametrize("i,M,N,K,with_bias", _awq_cases())
def test_random_awq_shapes(i, M, N, K, with_bias):
    rng = np.random.default_rng(7000 + i)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    codes, scales, zeros = oracle.awq_quantize_weight(W)
    assert np.count_nonzero(scales) == scales.size, "degenerate AWQ layer (zero scales)"
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    announce("random awq", i, "M,N,K", M, N, K, "bias", with_bias)
    y = gpu_gemv(x, codes, scales, zeros, bias)
    ref = oracle.awq_gemv(x, codes, scales, zeros, bias)
    assert_bf16_close(y, ref, f"awq case {i}")
