"""The grouped QKV GEMM with per-head RMSNorm + rotary embedding of Q and K in
its epilogue (svdq_gemm_w4a4_qk_norm_rope) against the oracle.

Two comparisons: the whole output against the oracle's GEMM followed by its
norm/rotary step (the layer's bf16 tolerance), and the epilogue alone -- the
oracle's norm/rotary step applied to the plain GEMM's own bf16 output from
the GPU, where only fp32-vs-fp64 rounding separates the two.  V columns are
the plain GEMM's output bit for bit."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.fp6_layout import fp6_layout_from_nibbles
from tests.gpu_helpers import (announce, assert_bf16_close, empty, gpu_gemm, gpu_pack_weight, gpu_pack_weight_fp6,
                               poison, to_dev, to_host)

pytestmark = pytest.mark.gpu


def _norm_rope_inputs(rng, M):
    qw = synth.to_bf16_bits(rng.uniform(0.5, 1.5, 128))
    kw = synth.to_bf16_bits(rng.uniform(0.5, 1.5, 128))
    th = rng.uniform(-np.pi, np.pi, (M, 64))
    return qw, kw, np.cos(th).astype(np.float32), np.sin(th).astype(np.float32)


def _gpu_qk(ac, asc, w, t, bias, qw, kw, eps, cs, sn, alpha=1.0, prec=0, packed=False, fp6=False):
    M, N = ac.shape[0], w["wgt_codes"].shape[0]
    out = poison(empty((M, N), "bf16"))
    sk = "bf16" if prec == 0 else "u8"
    wc, ws = to_dev(w["wgt_codes"], "u8"), to_dev(w["wgt_scales"], sk)
    if packed:
        wc, prec = gpu_pack_weight(wc, ws), capi.SVDQ_INT4_PACKED
    if fp6:
        wc, prec = gpu_pack_weight_fp6(wc), capi.SVDQ_INT4_FP6
        ac = fp6_layout_from_nibbles(ac, 2 * ac.shape[1])
    capi.svdq_gemm_w4a4_qk_norm_rope(prec, to_dev(ac, "u8"), to_dev(asc, sk), wc, ws, alpha, to_dev(t, "f32"),
                                     to_dev(w["lora_up"], "bf16"), to_dev(bias, "bf16"), to_dev(qw, "bf16"),
                                     to_dev(kw, "bf16"), eps, to_dev(cs, "f32"), to_dev(sn, "f32"), out)
    torch.cuda.synchronize()
    return to_host(out, "bf16")


def _case(M, H, K, rank, with_bias, seed, prec=0):
    rng = np.random.default_rng(seed)
    N = 3 * H * 128
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.5))
    w = synth.synthetic_w4a4_weights(seed + 1, N, K, rank, "int4" if prec == 0 else "nvfp4")
    ac, asc, t = oracle.quantize_act(prec, x, smooth, w["lora_down"])
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    return ac, asc, t, w, bias, rng


@pytest.mark.parametrize("prec,M,H,K,rank,with_bias,alpha", [
    (0, 64, 1, 256, 16, True, 1.0), (0, 200, 2, 512, 32, False, 1.0), (0, 33, 3, 4160, 0, True, 1.0),
    (0, 130, 1, 192, 48, False, 0.5), (0, 1, 2, 128, 16, True, 1.0), (0, 257, 2, 640, 32, True, 1.0),
    # NVFP4: the three staging paths (K % 512 == 0, K % 256 == 0, neither)
    (1, 200, 2, 1024, 32, True, 1.0), (1, 33, 1, 768, 16, False, 0.5), (1, 130, 2, 4160, 0, True, 1.0),
])
def test_qk_norm_rope_shapes(prec, M, H, K, rank, with_bias, alpha):
    ac, asc, t, w, bias, rng = _case(M, H, K, rank, with_bias, 3000 + M + H + K, prec)
    qw, kw, cs, sn = _norm_rope_inputs(rng, M)
    eps = 1e-6
    announce("gemm qk_norm_rope", "prec", prec, "M,H,K,r", M, H, K, rank, "bias", with_bias)
    y = _gpu_qk(ac, asc, w, t, bias, qw, kw, eps, cs, sn, alpha, prec)
    plain = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha)
    HD = H * 128
    assert np.array_equal(y[:, 2 * HD:], plain[:, 2 * HD:]), "V columns differ from the plain GEMM"
    # the epilogue alone: the oracle's norm/rotary on the GPU's own bf16 y
    ep = oracle.qk_norm_rope(plain, qw, kw, eps, cs, sn)
    assert_bf16_close(y, ep, f"epilogue {M}x{H}x{K}")
    ulp = np.abs(y.view(np.int16).astype(np.int32) - ep.view(np.int16).astype(np.int32))
    assert np.mean(ulp <= 1) >= 0.999, f"epilogue: {np.mean(ulp <= 1):.5f} within 1 ulp"
    ref = oracle.gemm_w4a4_qk_norm_rope(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias,
                                        qw, kw, eps, cs, sn, alpha=alpha)
    assert_bf16_close(y, ref, f"qkv p{prec} {M}x{H}x{K} r{rank}")
    if prec == 0:
        announce("gemm qk_norm_rope packed", "M,H,K,r", M, H, K, rank)
        yp = _gpu_qk(ac, asc, w, t, bias, qw, kw, eps, cs, sn, alpha, prec, packed=True)
        plain_p = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha,
                           packed=True)
        assert np.array_equal(yp[:, 2 * HD:], plain_p[:, 2 * HD:]), "packed: V columns differ from its plain GEMM"
        ep_p = oracle.qk_norm_rope(plain_p, qw, kw, eps, cs, sn)
        ulp = np.abs(yp.view(np.int16).astype(np.int32) - ep_p.view(np.int16).astype(np.int32))
        assert np.mean(ulp <= 1) >= 0.999, f"packed epilogue: {np.mean(ulp <= 1):.5f} within 1 ulp"
        assert_bf16_close(yp, ref, f"qkv packed {M}x{H}x{K} r{rank}")
        announce("gemm qk_norm_rope fp6", "M,H,K,r", M, H, K, rank)
        yf = _gpu_qk(ac, asc, w, t, bias, qw, kw, eps, cs, sn, alpha, prec, fp6=True)
        plain_f = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha, fp6=True)
        assert np.array_equal(yf[:, 2 * HD:], plain_f[:, 2 * HD:]), "fp6: V columns differ from its plain GEMM"
        ep_f = oracle.qk_norm_rope(plain_f, qw, kw, eps, cs, sn)
        ulp = np.abs(yf.view(np.int16).astype(np.int32) - ep_f.view(np.int16).astype(np.int32))
        assert np.mean(ulp <= 1) >= 0.999, f"fp6 epilogue: {np.mean(ulp <= 1):.5f} within 1 ulp"
        assert_bf16_close(yf, ref, f"qkv fp6 {M}x{H}x{K} r{rank}")


def test_qk_norm_rope_zero_and_tiny_heads():
    """A row of zeros (eps keeps it finite) and heads whose mean square is
    far below eps."""
    ac, asc, t, w, bias, rng = _case(8, 1, 256, 16, False, 77)
    ac[0] = 0                                     # row 0: codes and low-rank input zero -> y = 0
    t[0] = 0.0
    qw, kw, cs, sn = _norm_rope_inputs(rng, 8)
    for eps in (1e-6, 10.0):
        y = _gpu_qk(ac, asc, w, t, None, qw, kw, eps, cs, sn)
        plain = gpu_gemm(0, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], None)
        ep = oracle.qk_norm_rope(plain, qw, kw, eps, cs, sn)
        assert_bf16_close(y, ep, f"eps {eps}")
        assert np.isfinite(synth.bf16_bits_to_f32(y)).all()


def test_qk_norm_rope_fullsize_qkv():
    """The grouped QKV layer of the DiT block (4096 x 3072 -> 9216, 24 heads,
    rank 32), sampled rows."""
    cfg = synth.QKV
    ac, asc, t, w, bias, rng = _case(cfg.M, 24, cfg.K, cfg.rank, False, cfg.seed + 500)
    qw, kw, cs, sn = _norm_rope_inputs(rng, cfg.M)
    announce("fullsize qkv qk_norm_rope")
    y = _gpu_qk(ac, asc, w, t, None, qw, kw, 1e-6, cs, sn)
    rows = np.concatenate([[0, 1, cfg.M - 1], rng.choice(np.arange(2, cfg.M - 1), 21, replace=False)])
    ref = oracle.gemm_w4a4_qk_norm_rope(0, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], None,
                                        qw, kw, 1e-6, cs, sn, rows=rows)
    assert_bf16_close(y[rows], ref, "fullsize qkv")
    assert np.isfinite(synth.bf16_bits_to_f32(y)).all()
    announce("fullsize qkv qk_norm_rope packed")
    yp = _gpu_qk(ac, asc, w, t, None, qw, kw, 1e-6, cs, sn, packed=True)
    assert_bf16_close(yp[rows], ref, "fullsize qkv packed")
    assert np.isfinite(synth.bf16_bits_to_f32(yp)).all()
    announce("fullsize qkv qk_norm_rope fp6")
    yf = _gpu_qk(ac, asc, w, t, None, qw, kw, 1e-6, cs, sn, fp6=True)
    assert_bf16_close(yf[rows], ref, "fullsize qkv fp6")
    assert np.isfinite(synth.bf16_bits_to_f32(yf)).all()
