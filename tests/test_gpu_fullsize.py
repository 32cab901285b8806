"""Parity at the full DiT-shaped sizes (the configurations the benchmark
times, same kernels and launch shapes): codes and scales over the whole
tensor, lora_act over the whole tensor, GEMM outputs on sampled rows that
the oracle computes one by one, and the weight-only GEMV in full.

Workloads (seeded, synthetic; weights prepared offline by the oracle):
  QKV    M=4096 K=3072 N=9216  int4 g64 rank 32
  MLP    up 4096x3072->12288, down 4096x12288->3072 (GELU-tanh input), int4, rank 32
  NVFP4  attention out 4096x3072->3072, rank 32
  AWQ    adaptive-norm modulation, M in {1,2,8}, K=3072, N=18432; and the same
         weights applied to all 4096 tokens (the GEMM regime), sampled rows"""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import synth
from tests.fp6_layout import fp6_layout_from_nibbles
from tests.gpu_helpers import announce, assert_bf16_close, assert_f32_close, gpu_gemm, gpu_gemv, gpu_quantize, svdq_case

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]

SAMPLE_ROWS = 24

# Row positions inside a 128-row GEMM tile that fall in different classes of
# the kernels' row handling (the 8-row LDS swizzle, the 32-row MFMA blocks,
# the two 64-row wave halves, first/last rows of each).
TILE_POSITIONS = np.array([0, 1, 7, 8, 30, 31, 33, 62, 63, 64, 66, 95, 96, 101, 126, 127])


def _rows(M, seed):
    rng = np.random.default_rng(seed)
    extra = rng.choice(np.arange(2, M - 1), SAMPLE_ROWS - 3, replace=False)
    return np.concatenate([[0, 1, M - 1], np.sort(extra)])


def _tile_rows(M, per_tile=4):
    """per_tile rows in every 128-row tile, the position classes taken in
    turn so that every class is checked every 16/per_tile tiles, plus the
    first and last rows."""
    rows = [0, 1, M - 1]
    for t, base in enumerate(range(0, M, 128)):
        for j in range(per_tile):
            r = base + TILE_POSITIONS[(per_tile * t + j) % len(TILE_POSITIONS)]
            if r < M:
                rows.append(r)
    return np.unique(np.array(rows))


def _layer_parity(cfg, case, prec):
    K = cfg.K
    announce("fullsize quantize_act", cfg.name)
    gc, gs, gt = gpu_quantize(prec, case["x"], case["smooth"], case["lora_down"], K)
    oc, os_, ot = oracle.quantize_act(prec, case["x"], case["smooth"], case["lora_down"])
    assert np.array_equal(gs, os_), f"{cfg.name}: scales differ ({int((gs != os_).sum())} elements)"
    assert np.array_equal(gc, oc), f"{cfg.name}: codes differ ({int((gc != oc).sum())} bytes)"
    assert_f32_close(gt, ot, 1e-5, cfg.name + " lora_act")
    announce("fullsize gemm_w4a4", cfg.name)
    y = gpu_gemm(prec, oc, os_, case["wgt_codes"], case["wgt_scales"], ot, case["lora_up"], case["bias"])
    rows = _tile_rows(cfg.M)
    ref = oracle.gemm_w4a4(prec, oc, os_, case["wgt_codes"], case["wgt_scales"], ot, case["lora_up"],
                           case["bias"], rows=rows)
    stats = assert_bf16_close(y[rows], ref, cfg.name)
    assert np.isfinite(synth.bf16_bits_to_f32(y)).all()
    if prec == oracle.INT4:
        # the packed weight (fp8 matrix-core formulation)
        announce("fullsize gemm_w4a4 packed", cfg.name)
        yp = gpu_gemm(prec, oc, os_, case["wgt_codes"], case["wgt_scales"], ot, case["lora_up"], case["bias"],
                      packed=True)
        stats = assert_bf16_close(yp[rows], ref, cfg.name + " packed")
        assert np.isfinite(synth.bf16_bits_to_f32(yp)).all()
        # the production path: the activation step's FP6 output (whole tensor
        # against the oracle's codes in that layout) into the FP6 GEMM
        announce("fullsize quantize_act fp6", cfg.name)
        fc, fs, ft = gpu_quantize(3, case["x"], case["smooth"], case["lora_down"], K)
        assert np.array_equal(fs, os_), f"{cfg.name} fp6: scales differ"
        assert np.array_equal(fc, fp6_layout_from_nibbles(oc, K)), f"{cfg.name} fp6: code bytes differ"
        assert np.array_equal(ft, gt), f"{cfg.name} fp6: lora_act differs from the nibble output's"
        announce("fullsize gemm_w4a4 fp6", cfg.name)
        yf = gpu_gemm(prec, oc, os_, case["wgt_codes"], case["wgt_scales"], ft, case["lora_up"], case["bias"],
                      fp6=True, act_fp6=fc)
        stats = assert_bf16_close(yf[rows], ref, cfg.name + " fp6")
        assert np.isfinite(synth.bf16_bits_to_f32(yf)).all()
    return stats


def test_fullsize_qkv_int4():
    _layer_parity(synth.QKV, svdq_case(synth.QKV), oracle.INT4)


def test_fullsize_mlp_up_int4():
    _layer_parity(synth.MLP_UP, svdq_case(synth.MLP_UP), oracle.INT4)


def test_fullsize_mlp_down_int4():
    h = synth.gelu_activations(synth.MLP_UP, synth.MLP_DOWN)
    case = {"x": h["x"], "W": h["W"], "bias": None}
    case.update(oracle.prepare_svdq_weight(oracle.INT4, h["x"], h["W"], synth.MLP_DOWN.rank))
    _layer_parity(synth.MLP_DOWN, case, oracle.INT4)


def test_fullsize_attn_out_nvfp4():
    _layer_parity(synth.ATTN_OUT_NVFP4, svdq_case(synth.ATTN_OUT_NVFP4), oracle.NVFP4)


@pytest.mark.parametrize("M", [1, 2, 8])
def test_fullsize_adaln_awq(M):
    cfg = synth.ADALN_AWQ
    case = synth.linear_case(cfg, M=8)
    codes, scales, zeros = oracle.awq_quantize_weight(case["W"])
    x = case["x"][:M]
    announce("fullsize awq_gemv", cfg.name, "M", M)
    y = gpu_gemv(x, codes, scales, zeros, None)
    ref = oracle.awq_gemv(x, codes, scales, zeros, None)
    assert_bf16_close(y, ref, f"{cfg.name} M={M}")


def test_fullsize_awq_gemm_regime():
    """The AWQ weights of the adaptive-norm shape (N=18432, K=3072) applied to
    4096 rows of x: the GEMM path, checked on sampled rows."""
    cfg = synth.ADALN_AWQ
    case = synth.linear_case(cfg, M=8)
    codes, scales, zeros = oracle.awq_quantize_weight(case["W"])
    rng = np.random.default_rng(4711)
    M = 4096
    x = synth.to_bf16_bits(rng.standard_normal((M, cfg.K)))
    announce("fullsize awq gemm regime", cfg.name, "M", M)
    y = gpu_gemv(x, codes, scales, zeros, None)
    rows = _rows(M, 4711)
    ref = oracle.awq_gemv(x[rows], codes, scales, zeros, None)
    assert_bf16_close(y[rows], ref, f"{cfg.name} M={M}")
    assert np.isfinite(synth.bf16_bits_to_f32(y)).all()
