"""Pins for the oracle's 4-bit GEMM step, the offline SVD step and the AWQ
weight-only layer.

Method (blog "Hugging Face integrates Nunchaku 4-bit diffusion inference into
Diffusers", "SVDQuant and the Nunchaku engine"; Thai blog "Bringing Nunchaku
4-bit diffusion inference to Diffusers", "Background: SVDQuant and
Nunchaku"): outliers migrate from activations into weights, the hardest part
of each weight is a 16-bit low-rank branch, the residual is 4-bit, and the
engine adds the low-rank up-projection to the 4-bit product.

Pins: brute-force fp64 matmuls of the dequantized tensors (a different
summation than the oracle's per-group integer sums), library integer
matmuls for the group sums, the Eckart-Young identity, the zero-residual
invariant (a weight that is exactly its low-rank branch), power-of-two
scaling of alpha, and the method's stated purpose as an ordering property
(SVDQuant beats smoothing only, which beats plain W4A4, on outlier data).
"""
import numpy as np
import pytest

from bit_w4a4_quantized_svdq_amd import synth


def f32(h):
    return synth.bf16_bits_to_f32(h).astype(np.float64)


def ulp_dist(a, b):
    """bf16 ulp distance on the monotone integer line (+0 == -0)."""
    def ordv(h):
        h = np.asarray(h, np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    return np.abs(ordv(a) - ordv(b))


def _layer(oracle, cfg, precision, rank, with_bias=False, smooth=True):
    case = synth.linear_case(cfg, with_bias=with_bias)
    prep = oracle.prepare_svdq_weight(precision, case["x"], case["W"], rank, smooth=smooth)
    return case, prep


# -------------------------------------------------------------- group sums

def test_group_sums_match_integer_matmul(oracle):
    rng = np.random.default_rng(31)
    M, N, K = 7, 9, 256
    qa = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (N, K))
    G = oracle.group_sums_int4(synth.pack_nibbles(qa), synth.pack_nibbles(qw), K)
    for g in range(K // 64):
        ref = qa[:, 64 * g:64 * g + 64] @ qw[:, 64 * g:64 * g + 64].T
        assert np.array_equal(G[:, :, g], ref)
    # extremes: -8*-8*64 = 4096 and 7*-8*64 = -3584
    G = oracle.group_sums_int4(synth.pack_nibbles(np.full((1, 64), -8)),
                               synth.pack_nibbles(np.full((2, 64), -8)), 64)
    assert G.ravel().tolist() == [4096, 4096]


def test_unpack_inverts_pack(oracle):
    rng = np.random.default_rng(32)
    q = rng.integers(-8, 8, (5, 128))
    assert np.array_equal(oracle.unpack_int4(synth.pack_nibbles(q), 5, 128), q)
    u = rng.integers(0, 16, (5, 128))
    assert np.array_equal(oracle.unpack_u4(synth.pack_nibbles(u), 5, 128), u)


# ------------------------------------------------------------ int4 GEMM

def _dequant_int4(oracle, codes, scales, rows, K):
    return oracle.unpack_int4(codes, rows, K).astype(np.float64) * f32(scales).repeat(64, 1)


@pytest.mark.parametrize("with_bias", [False, True])
def test_int4_gemm_brute_force_tiny(oracle, with_bias):
    cfg = synth.TINY
    case, prep = _layer(oracle, cfg, oracle.INT4, cfg.rank, with_bias=with_bias)
    ac, asc, t = oracle.quantize_act(oracle.INT4, case["x"], prep["smooth"], prep["lora_down"])
    y = oracle.gemm_w4a4(oracle.INT4, ac, asc, prep["wgt_codes"], prep["wgt_scales"], t,
                         prep["lora_up"], case["bias"])
    A = _dequant_int4(oracle, ac, asc, cfg.M, cfg.K)
    B = _dequant_int4(oracle, prep["wgt_codes"], prep["wgt_scales"], cfg.N, cfg.K)
    ref = A @ B.T + t.astype(np.float64) @ f32(prep["lora_up"]).T
    if with_bias:
        ref += f32(case["bias"])[None, :]
    d = ulp_dist(y, oracle.f64_to_bf16(ref))
    assert d.max() <= 1 and (d == 0).mean() >= 0.999


def test_int4_gemm_rows_subset(oracle):
    cfg = synth.TINY
    case, prep = _layer(oracle, cfg, oracle.INT4, cfg.rank)
    ac, asc, t = oracle.quantize_act(oracle.INT4, case["x"], prep["smooth"], prep["lora_down"])
    full = oracle.gemm_w4a4(oracle.INT4, ac, asc, prep["wgt_codes"], prep["wgt_scales"], t, prep["lora_up"])
    rows = np.array([63, 0, 17])
    sub = oracle.gemm_w4a4(oracle.INT4, ac, asc, prep["wgt_codes"], prep["wgt_scales"], t,
                           prep["lora_up"], rows=rows)
    assert np.array_equal(sub, full[rows])


def test_alpha_scales_the_4bit_term_only(oracle):
    rng = np.random.default_rng(33)
    M, N, K = 4, 8, 128
    ac = synth.pack_nibbles(rng.integers(-7, 8, (M, K)))
    wc = synth.pack_nibbles(rng.integers(-7, 8, (N, K)))
    asc = synth.to_bf16_bits(rng.uniform(0.1, 1, (M, K // 64)))
    wsc = synth.to_bf16_bits(rng.uniform(0.1, 1, (N, K // 64)))
    y1 = oracle.gemm_w4a4(oracle.INT4, ac, asc, wc, wsc, None, None, alpha=1.0)
    y2 = oracle.gemm_w4a4(oracle.INT4, ac, asc, wc, wsc, None, None, alpha=2.0)
    assert np.array_equal(f32(y2), 2 * f32(y1))


@pytest.mark.parametrize("precision", [0, 1])
def test_zero_residual_invariant(oracle, precision):
    """A weight that is exactly its own low-rank branch: the residual is 0,
    every weight code and scale is 0, and y = RNE_bf16(t . up + bias) with
    t = fp32(x_hat . down^T).

    W = up . down is made exactly representable in bf16: up holds powers of
    two and each column k of down is non-zero in one rank slot only (k % r),
    so every W[n,k] is one bf16 times a power of two."""
    rng = np.random.default_rng(34 + precision)
    M, N, K, r = 24, 48, 256, 16
    up_f = np.where(rng.random((N, r)) < 0.5, -1.0, 1.0) * 2.0 ** rng.integers(-2, 2, (N, r))
    down_f = synth.bf16_bits_to_f32(synth.to_bf16_bits(rng.standard_normal((r, K)) * 0.3)).astype(np.float64)
    down_f[np.arange(r)[:, None] != (np.arange(K) % r)[None, :]] = 0.0
    up, down = synth.to_bf16_bits(up_f), synth.to_bf16_bits(down_f)
    W = synth.to_bf16_bits(up_f @ down_f)
    assert np.array_equal(f32(W), up_f @ down_f)              # exact in bf16
    s = np.full(K, 0x3F80, np.uint16)
    R = oracle.svdq_residual(W, s, up, down)
    assert not R.any()
    wc, wsc = (oracle.quantize_int4 if precision == 0 else oracle.quantize_nvfp4)(R)
    assert not wc.any() and not wsc.any()
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    bias = synth.to_bf16_bits(rng.standard_normal(N))
    ac, asc, t = oracle.quantize_act(precision, x, s, down)
    y = oracle.gemm_w4a4(precision, ac, asc, wc, wsc, t, up, bias)
    t_ref = (f32(x) @ down_f.T).astype(np.float32)            # x_hat = x when s = 1
    ref = oracle.f64_to_bf16(t_ref.astype(np.float64) @ up_f.T + f32(bias)[None, :])
    d = ulp_dist(y, ref)
    assert d.max() <= 1 and (d == 0).mean() >= 0.99


# ----------------------------------------------------------- NVFP4 GEMM

def test_nvfp4_gemm_brute_force(oracle):
    cfg = synth.LinearConfig("tiny_nvfp4", 32, 256, 64, 16, "nvfp4", 7, 4, 30.0)
    case, prep = _layer(oracle, cfg, oracle.NVFP4, cfg.rank, with_bias=True)
    ac, asc, t = oracle.quantize_act(oracle.NVFP4, case["x"], prep["smooth"], prep["lora_down"])
    y = oracle.gemm_w4a4(oracle.NVFP4, ac, asc, prep["wgt_codes"], prep["wgt_scales"], t,
                         prep["lora_up"], case["bias"], alpha=0.5)

    def deq(codes, scales, rows):
        c = oracle.e2m1_to_f32(oracle.unpack_u4(codes, rows, cfg.K)).astype(np.float64)
        return c * oracle.e4m3_to_f32(scales).astype(np.float64).repeat(16, 1)

    A = deq(ac, asc, cfg.M)
    B = deq(prep["wgt_codes"], prep["wgt_scales"], cfg.N)
    ref = 0.5 * (A @ B.T) + t.astype(np.float64) @ f32(prep["lora_up"]).T + f32(case["bias"])[None, :]
    d = ulp_dist(y, oracle.f64_to_bf16(ref))
    assert d.max() <= 1 and (d == 0).mean() >= 0.999


# ------------------------------------------------------ offline low rank

def test_eckart_young_and_factor_rounding(oracle):
    rng = np.random.default_rng(35)
    N, K, r = 96, 160, 16
    A = rng.standard_normal((N, K)) * np.exp(rng.uniform(-2, 2, K))[None, :]
    U, S, VT = oracle.top_singular_triplets(A, r)
    full = np.linalg.svd(A, compute_uv=False)
    assert np.allclose(S, full[:r], rtol=1e-12)
    trunc = U @ np.diag(S) @ VT
    assert np.isclose(np.linalg.norm(A - trunc) ** 2, np.sum(full[r:] ** 2), rtol=1e-10)
    # canonical signs: each left vector's largest |entry| is positive
    assert (U[np.abs(U).argmax(0), np.arange(r)] > 0).all()
    up, down = oracle.lowrank_factors(A, r)
    assert np.array_equal(up, oracle.f64_to_bf16(U))
    assert np.array_equal(down, oracle.f64_to_bf16(S[:, None] * VT))
    rounded = f32(up) @ f32(down)
    assert np.linalg.norm(A - rounded) <= np.linalg.norm(A - trunc) + 2 ** -7 * np.linalg.norm(trunc)


def test_truncated_svd_large_path_matches_dense(oracle):
    """Matrices wider than 1024 use a Lanczos solver; its leading triplets
    must match the dense LAPACK SVD."""
    rng = np.random.default_rng(36)
    A = rng.standard_normal((1100, 1030)) + 5 * np.outer(rng.standard_normal(1100), rng.standard_normal(1030))
    U, S, VT = oracle.top_singular_triplets(A, 8)
    Ud, Sd, VTd = np.linalg.svd(A, full_matrices=False)
    assert np.allclose(S, Sd[:8], rtol=1e-9)
    assert np.allclose(np.abs(np.sum(U * Ud[:, :8], 0)), 1, atol=1e-6)


def test_svdquant_error_ordering_on_outliers(oracle):
    """The method's purpose (outliers moved to the weights, hardest part kept
    16-bit): on outlier-heavy inputs the SVDQuant layer's error against the
    unquantized fp64 product is below smoothing-only, which is below plain
    W4A4.  Only the ordering is pinned; the pages print no magnitudes."""
    cfg = synth.LinearConfig("outlier_case", 128, 512, 256, 32, "int4", 5, 8, 50.0)
    case = synth.linear_case(cfg)
    exact = f32(case["x"]) @ f32(case["W"]).T
    errs = {}
    for name, smooth, rank in (("naive", False, 0), ("smooth", True, 0), ("svdq", True, 32)):
        prep = oracle.prepare_svdq_weight(oracle.INT4, case["x"], case["W"], rank, smooth=smooth)
        ac, asc, t = oracle.quantize_act(oracle.INT4, case["x"], prep["smooth"], prep["lora_down"])
        y = oracle.gemm_w4a4(oracle.INT4, ac, asc, prep["wgt_codes"], prep["wgt_scales"], t, prep["lora_up"])
        errs[name] = np.linalg.norm(f32(y) - exact) / np.linalg.norm(exact)
    assert errs["svdq"] < errs["smooth"] < errs["naive"], errs


# ------------------------------------------------------------------ AWQ

def test_awq_quantizer_invariants(oracle):
    rng = np.random.default_rng(37)
    W = synth.to_bf16_bits(rng.standard_normal((64, 512)) * 0.02)
    codes, scales, zeros = oracle.awq_quantize_weight(W)
    q = oracle.unpack_u4(codes, 64, 512).astype(np.float64)
    z = f32(zeros)
    assert np.array_equal(z, np.round(z)) and z.min() >= 0 and z.max() <= 15
    s = f32(scales).repeat(64, 1)
    w_deq = (q - z.repeat(64, 1)) * s
    # (q - z) * s is exact in fp32: 5-bit integer times an 8-bit significand
    assert np.array_equal(w_deq.astype(np.float32).astype(np.float64), w_deq)
    # Round trip: <= s/2 unless the code clipped at 15.  s = bf16((hi-lo)/15)
    # can sit 2^-8 below the exact step, so (hi-lo)/s <= 15/(1-2^-8), and z is
    # within 1/2 of -lo/s: a clipped element is off by at most
    # (1/2 + 15*2^-8/(1-2^-8)) * s.  Clipping is rare.
    err = np.abs(f32(W) - w_deq)
    assert (err <= (0.5 + 15 * 2 ** -8 / (1 - 2 ** -8)) * s).all()
    assert (err > s / 2).mean() < 1e-3


def test_awq_gemv_brute_force(oracle):
    cfg = synth.ADALN_AWQ
    rng = np.random.default_rng(38)
    K, N = 512, 200
    x = synth.to_bf16_bits(rng.standard_normal((8, K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    bias = synth.to_bf16_bits(rng.standard_normal(N))
    codes, scales, zeros = oracle.awq_quantize_weight(W)
    w = (oracle.unpack_u4(codes, N, K).astype(np.float64) - f32(zeros).repeat(64, 1)) * f32(scales).repeat(64, 1)
    for b in (None, bias):
        y = oracle.awq_gemv(x, codes, scales, zeros, b)
        ref = f32(x) @ w.T + (0 if b is None else f32(b)[None, :])
        d = ulp_dist(y, oracle.f64_to_bf16(ref))
        assert d.max() <= 1 and (d == 0).mean() >= 0.999
    assert cfg.K == 3072 and cfg.N == 6 * 3072
