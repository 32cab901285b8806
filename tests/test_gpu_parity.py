"""GPU parity of the HIP path against the CPU oracle, element by element, at
sizes the oracle finishes in seconds (several tiles plus ragged tails) and
at the degenerate and edge cases of the method.  All calls go through the
C ABI (libsvdq.so) via its Python binding."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.fp6_layout import fp6_layout_from_nibbles, fp6_layout_from_q
from tests.gpu_helpers import (announce, assert_bf16_close, assert_f32_close, gpu_gemm, gpu_gemv,
                               gpu_pack_weight_fp6, gpu_quantize, svdq_case, to_dev, to_host, empty, poison)

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _heavy_x(rng, M, K, n_out=None, scale=50.0):
    x = rng.standard_normal((M, K))
    n_out = max(1, K // 100) if n_out is None else n_out
    x[:, rng.choice(K, n_out, replace=False)] *= scale
    return synth.to_bf16_bits(x)


def _check_quantize(prec, x, smooth, down, what):
    K = x.shape[1]
    announce("quantize_act", what, "prec", prec, "shape", x.shape, "rank", 0 if down is None else down.shape[0])
    gc, gs, gt = gpu_quantize(prec, x, smooth, down, K)
    oc, os_, ot = oracle.quantize_act(prec, x, smooth, down)
    assert np.array_equal(gs, os_), f"{what}: scales differ at {np.argwhere(gs != os_)[:5].tolist()}"
    assert np.array_equal(gc, oc), f"{what}: codes differ at {np.argwhere(gc != oc)[:5].tolist()}"
    if down is not None:
        assert_f32_close(gt, ot, 1e-5, what)
    if prec == 0:
        _check_fp6_codes(x, smooth, down, oc, os_, gt, what)
    return oc, os_, ot


def _check_fp6_codes(x, smooth, down, oc, os_, gt_int4, what, gelu=False):
    """The SVDQ_INT4_FP6 activation step: the oracle's int4 codes in the FP6
    layout (host reference encoder), int4's scales, and the same lora_act as
    the nibble output."""
    K = x.shape[1]
    announce("quantize_act fp6", what, "shape", x.shape, "gelu", gelu)
    fc, fs, ft = gpu_quantize(3, x, smooth, down, K, gelu=gelu)
    assert np.array_equal(fs, os_), f"{what} fp6: scales differ"
    want = fp6_layout_from_nibbles(oc, K)
    assert np.array_equal(fc, want), f"{what} fp6: code bytes differ at {np.argwhere(fc != want)[:5].tolist()}"
    if down is not None:
        assert np.array_equal(ft, gt_int4), f"{what} fp6: lora_act differs from the nibble output's"


# ------------------------------------------------------------ quantize_act

@pytest.mark.parametrize("prec", [0, 1])
def test_quantize_act_tiny_config(prec):
    cfg = synth.TINY if prec == 0 else synth.LinearConfig("tiny_nvfp4", 64, 256, 256, 16, "nvfp4", 0, 4, 30.0)
    c = svdq_case(cfg)
    _check_quantize(prec, c["x"], c["smooth"], c["lora_down"], cfg.name)


@pytest.mark.parametrize("prec,M,K,rank", [
    (0, 1, 64, 0), (0, 17, 192, 48), (0, 200, 512, 32), (0, 33, 4160, 16), (0, 40, 1024, 128),
    (1, 1, 64, 0), (1, 17, 192, 16), (1, 200, 512, 32), (1, 33, 4160, 128), (1, 40, 1024, 64),
])
def test_quantize_act_shapes(prec, M, K, rank):
    rng = np.random.default_rng(1000 + 7 * M + K + rank + prec)
    x = _heavy_x(rng, M, K)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.7))
    down = synth.to_bf16_bits(rng.standard_normal((rank, K)) * 0.05) if rank else None
    _check_quantize(prec, x, smooth, down, f"M{M}_K{K}_r{rank}")


def _edge_rows(K):
    """Rows that hit the method's degenerate and tie cases (bf16 bits)."""
    rows = []
    f = np.zeros(K)
    rows.append(f.copy())                                   # all-zero row
    rows.append(np.full(K, -1.75))                          # constant groups
    t = np.tile(np.arange(-13, 14) / 2.0, K)[:K]            # int4 ties: absmax 7 -> scale 1
    t[::64] = 7.0
    rows.append(t)
    e = np.tile([6.0, -0.25, 0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, -5.0, -0.75, 0.0, -0.0, 3.0, 1.5, -6.0],
                K // 16)                                    # nvfp4 ties: absmax 6 -> scale 1
    rows.append(e)
    rows.append(np.tile(np.arange(1, 17), K // 16) * 2.0 ** -133)   # bf16 subnormal inputs
    rows.append(np.tile([5000.0, -3000.0, 1.0, 0.5], K // 4))       # E4M3 saturation (absmax/6 > 448)
    rows.append(np.tile([1e-30, -3e-31, 2e-32, 0.0], K // 4))       # tiny groups
    rows.append(np.linspace(-3.0e4, 3.0e4, K))
    x = synth.to_bf16_bits(np.stack(rows))
    x[1, 5] = 0x8000                                        # a -0
    return x


@pytest.mark.parametrize("prec", [0, 1])
@pytest.mark.parametrize("smooth_kind", ["none", "ones", "twos_threes", "tiny_channels", "random"])
def test_quantize_act_edge_values(prec, smooth_kind):
    K = 256
    x = _edge_rows(K)
    rng = np.random.default_rng(77)
    if smooth_kind == "none":
        smooth = None
    elif smooth_kind == "ones":
        smooth = np.full(K, 0x3F80, np.uint16)
    elif smooth_kind == "twos_threes":                      # halves subnormal inputs -> exact bf16 ties
        smooth = synth.to_bf16_bits(np.where(np.arange(K) % 2 == 0, 2.0, 3.0))
    elif smooth_kind == "tiny_channels":                    # 1/s outside fp32's normal range -> IEEE path
        s = np.exp(rng.standard_normal(K) * 0.3)
        s[::37] = 2.0 ** -70
        smooth = synth.to_bf16_bits(s)
        x = x.copy()
        x[:, ::37] = synth.to_bf16_bits(np.full((x.shape[0], len(range(0, K, 37))), 2.0 ** -80))
    else:
        smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K)))
    down = synth.to_bf16_bits(rng.standard_normal((16, K)) * 0.05)
    _check_quantize(prec, x, smooth, down, f"edge_{smooth_kind}")


def test_quantize_act_ragged_large_M():
    rng = np.random.default_rng(5)
    x = _heavy_x(rng, 4095, 256)
    _check_quantize(0, x, None, synth.to_bf16_bits(rng.standard_normal((32, 256)) * 0.05), "M4095")


# ------------------------------------------------------------------ GEMM

@pytest.mark.parametrize("with_bias", [False, True])
def test_gemm_int4_tiny_config(with_bias):
    cfg = synth.TINY
    c = svdq_case(cfg, with_bias=with_bias)
    ac, asc, t = oracle.quantize_act(0, c["x"], c["smooth"], c["lora_down"])
    announce("gemm_w4a4 int4", cfg.name, "bias", with_bias)
    y = gpu_gemm(0, ac, asc, c["wgt_codes"], c["wgt_scales"], t, c["lora_up"], c["bias"])
    ref = oracle.gemm_w4a4(0, ac, asc, c["wgt_codes"], c["wgt_scales"], t, c["lora_up"], c["bias"])
    assert_bf16_close(y, ref, cfg.name)


def _random_gemm_case(prec, M, N, K, rank, with_bias, seed):
    rng = np.random.default_rng(seed)
    x = _heavy_x(rng, M, K)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.5))
    w = synth.synthetic_w4a4_weights(seed + 1, N, K, rank, "int4" if prec == 0 else "nvfp4")
    ac, asc, t = oracle.quantize_act(prec, x, smooth, w["lora_down"])
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    return ac, asc, t, w, bias


@pytest.mark.parametrize("prec,M,N,K,rank,with_bias,alpha", [
    (0, 200, 320, 512, 32, True, 1.0), (0, 1, 64, 64, 0, False, 1.0), (0, 130, 96, 4160, 16, True, 1.0),
    (0, 257, 129, 192, 128, False, 0.5), (0, 64, 1000, 640, 48, True, 1.0),
    (1, 200, 320, 512, 32, True, 1.0), (1, 1, 64, 64, 0, False, 1.0), (1, 130, 96, 4160, 16, True, 0.5),
    (1, 257, 129, 192, 128, False, 2.0),
    # NVFP4 staging paths: K % 512 == 0 (two-slice stages, several 8-slice scale
    # chunks, ragged M and N) and K % 512 == 256 (single-slice ring, 4-slice scales)
    (1, 67, 200, 1024, 32, True, 1.0), (1, 130, 192, 2560, 16, False, 0.5), (1, 200, 320, 768, 32, True, 1.0),
    # FP6 main loops: K/64 = 3 (odd: a last stage with one group), 6 (pairs, 2-byte scales),
    # 12 and 48 (4-group scale loads), ragged M and N
    (0, 70, 200, 192, 16, True, 1.0), (0, 129, 130, 384, 32, False, 1.0), (0, 200, 256, 768, 32, True, 2.0),
    (0, 131, 384, 3072, 32, True, 1.0),
])
def test_gemm_shapes(prec, M, N, K, rank, with_bias, alpha):
    ac, asc, t, w, bias = _random_gemm_case(prec, M, N, K, rank, with_bias, 2000 + M + N + K + prec)
    announce("gemm_w4a4", "prec", prec, "M,N,K,r", M, N, K, rank, "alpha", alpha)
    y = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha)
    ref = oracle.gemm_w4a4(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha=alpha)
    assert_bf16_close(y, ref, f"gemm p{prec} {M}x{N}x{K} r{rank}")
    if prec == 0:
        announce("gemm_w4a4 packed", "M,N,K,r", M, N, K, rank, "alpha", alpha)
        yp = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha, packed=True)
        assert_bf16_close(yp, ref, f"gemm packed {M}x{N}x{K} r{rank}")
        announce("gemm_w4a4 fp6", "M,N,K,r", M, N, K, rank, "alpha", alpha)
        yf = gpu_gemm(prec, ac, asc, w["wgt_codes"], w["wgt_scales"], t, w["lora_up"], bias, alpha, fp6=True)
        assert_bf16_close(yf, ref, f"gemm fp6 {M}x{N}x{K} r{rank}")


# ------------------------------------------------------- packed int4 weights

def expected_packed_blob(codes, scales, N, K):
    """The blob of svdq_pack_weight_int4 computed on the host from the plain
    codes by the documented layout (codes in sign-magnitude form: per dword
    (h, i) of a group and byte e, k = 64g + 32h + 8i + 2e, bits 0-2 |q[k]|,
    bit 7 its sign, bits 4-6 |q[k+1]|, its sign in bit 3 of byte (e+1) mod 4;
    then bf16 [N][2][K/64] with hi + lo = -8 * scale * group code sum).
    Returns (packed code bytes [N, K/2], corr hi [N, K/64], corr lo, -8 count)."""
    NG = K // 64
    q = oracle.unpack_int4(codes, N, K).astype(np.int64).reshape(N, NG, 2, 4, 4, 2)
    qe, qo = q[..., 0], q[..., 1]
    mag_e, mag_o = np.abs(qe) & 7, np.abs(qo) & 7
    sgn_e, sgn_o = (qe < 0).astype(np.int64), (qo < 0).astype(np.int64)
    byte = mag_e | sgn_e << 7 | mag_o << 4 | np.roll(sgn_o, 1, axis=-1) << 3
    packed = byte.reshape(N, K // 2).astype(np.uint8)
    sums = q.reshape(N, NG, 64).sum(axis=2)
    c = -8.0 * sums * synth.bf16_bits_to_f32(scales).astype(np.float64)
    hi = oracle.f64_to_bf16(c)
    lo = oracle.f64_to_bf16(c - synth.bf16_bits_to_f32(hi).astype(np.float64))
    return packed, hi, lo, int((q == -8).sum())


@pytest.mark.parametrize("N,K,with_minus8", [(64, 64, False), (130, 192, False), (257, 4160, False),
                                             (1000, 3072, False), (40, 512, True)])
def test_pack_weight_layout_exact(N, K, with_minus8):
    from tests.gpu_helpers import gpu_pack_weight
    rng = np.random.default_rng(6100 + N + K)
    q = rng.integers(-7, 8, (N, K))
    if with_minus8:
        q[3, 5] = q[7, 64] = q[39, K - 1] = -8
    codes = synth.pack_nibbles(q)
    scales = synth.to_bf16_bits(rng.uniform(0.001, 0.02, (N, K // 64)))
    announce("pack_weight_int4", N, K, "minus8", with_minus8)
    wc, ws = to_dev(codes, "u8"), to_dev(scales, "bf16")
    blob = poison(empty((capi.svdq_packed_weight_bytes(N, K),), "u8"))
    bad = poison(empty((1,), "i32"))
    capi.svdq_pack_weight_int4(wc, ws, blob, bad)
    torch.cuda.synchronize()
    got = to_host(blob, "u8")
    packed, hi, lo, n8 = expected_packed_blob(codes, scales, N, K)
    assert int(to_host(bad, "i32")[0]) == n8
    nb = N * K // 2
    assert np.array_equal(got[:nb].reshape(N, K // 2), packed), "packed codes differ"
    corr = got[nb:].view(np.uint16).reshape(N, 2, K // 64)
    assert np.array_equal(corr[:, 0], hi) and np.array_equal(corr[:, 1], lo), "correction planes differ"


@pytest.mark.parametrize("M,N,K", [
    (64, 64, 64), (33, 130, 4160), (1, 1, 128),
    (200, 320, 512), (130, 384, 3072), (130, 384, 12288), (257, 129, 1024),
])
def test_debug_group_sums_packed_exact(M, N, K):
    """Exact int32 group sums from the main loop of the packed (fp8) GEMM:
    activation codes anywhere in [-8, 7], weight codes in [-7, 7]."""
    from tests.gpu_helpers import gpu_pack_weight
    rng = np.random.default_rng(3500 + M + N + K)
    qa = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-7, 8, (N, K))
    qa[0, :64] = -8
    qw[0, :64] = -7                                           # extreme group: 64 * 56
    ac, wc = synth.pack_nibbles(qa), synth.pack_nibbles(qw)
    ws = synth.to_bf16_bits(np.full((N, K // 64), 0.01))
    announce("debug_group_sums_packed", M, N, K)
    blob = gpu_pack_weight(to_dev(wc, "u8"), to_dev(ws, "bf16"))
    G = poison(empty((M, N, K // 64), "i32"))
    capi.svdq_debug_group_sums_packed(to_dev(ac, "u8"), blob, N, G)
    torch.cuda.synchronize()
    got = to_host(G, "i32")
    ref = oracle.group_sums_int4(ac, wc, K)
    assert np.array_equal(got, ref), f"group sums differ at {np.argwhere(got != ref)[:5].tolist()}"


# ------------------------------------------------------ FP6 layout of int4

@pytest.mark.parametrize("N,K", [(64, 64), (130, 192), (257, 4160), (1000, 3072), (40, 512)])
def test_pack_weight_fp6_layout_exact(N, K):
    """svdq_pack_weight_fp6 against the host encoder of the documented layout;
    every code in [-8, 7] (the FP6 form holds -8 too)."""
    rng = np.random.default_rng(6300 + N + K)
    q = rng.integers(-8, 8, (N, K))
    q[0, :16] = np.arange(-8, 8)
    codes = synth.pack_nibbles(q)
    announce("pack_weight_fp6", N, K)
    got = to_host(gpu_pack_weight_fp6(to_dev(codes, "u8")), "u8")
    assert np.array_equal(got, fp6_layout_from_q(q)), "FP6 weight bytes differ"


@pytest.mark.parametrize("M,N,K", [
    (64, 64, 64), (33, 130, 4160), (1, 1, 128), (65, 200, 192),
    # K/64 a multiple of 4: the chunked loop with 4-group scale loads that the
    # DiT shapes run (K = 3072, 12288); odd K/64 (4160, 192): a one-group last stage
    (200, 320, 512), (130, 384, 3072), (130, 384, 12288), (257, 129, 1024),
])
def test_debug_group_sums_fp6_exact(M, N, K):
    """Exact int32 group sums from the main loop of the FP6 GEMM, codes
    anywhere in [-8, 7] on both sides."""
    rng = np.random.default_rng(3700 + M + N + K)
    qa = rng.integers(-8, 8, (M, K))
    qw = rng.integers(-8, 8, (N, K))
    qa[0, :64] = -8
    qw[0, :64] = -8                                          # extreme group: 64 * 64 = 4096
    ac, wc = synth.pack_nibbles(qa), synth.pack_nibbles(qw)
    announce("debug_group_sums_fp6", M, N, K)
    wf = gpu_pack_weight_fp6(to_dev(wc, "u8"))
    G = poison(empty((M, N, K // 64), "i32"))
    capi.svdq_debug_group_sums_fp6(to_dev(fp6_layout_from_q(qa), "u8"), wf, M, N, K, G)
    torch.cuda.synchronize()
    got = to_host(G, "i32")
    ref = oracle.group_sums_int4(ac, wc, K)
    assert np.array_equal(got, ref), f"group sums differ at {np.argwhere(got != ref)[:5].tolist()}"


@pytest.mark.parametrize("M,N,K", [
    (64, 64, 64), (33, 130, 4160), (1, 1, 128), (65, 200, 4160),
    # K/64 a multiple of 8: the chunked main loop that every DiT-shaped GEMM
    # launch runs (QKV / MLP-up K = 3072, MLP-down K = 12288), ragged M and N
    (200, 320, 512), (130, 384, 3072), (130, 384, 12288), (257, 129, 1024),
])
def test_debug_group_sums_exact(M, N, K):
    rng = np.random.default_rng(3000 + M + N + K)
    qa = rng.integers(-8, 8, (M, K))                        # includes foreign -8 codes
    qw = rng.integers(-8, 8, (N, K))
    qa[0, :64] = -8
    qw[0, :64] = -8                                          # extreme group: 64 * 64 = 4096
    ac, wc = synth.pack_nibbles(qa), synth.pack_nibbles(qw)
    announce("debug_group_sums", M, N, K)
    G = poison(empty((M, N, K // 64), "i32"))
    capi.svdq_debug_group_sums(to_dev(ac, "u8"), to_dev(wc, "u8"), G)
    torch.cuda.synchronize()
    got = to_host(G, "i32")
    ref = oracle.group_sums_int4(ac, wc, K)
    assert np.array_equal(got, ref), f"group sums differ at {np.argwhere(got != ref)[:5].tolist()}"


def test_zero_residual_layer_on_gpu():
    """Weight == its low-rank branch: the 4-bit term vanishes and the GPU
    output is the fp32 low-rank product plus bias."""
    rng = np.random.default_rng(41)
    M, N, K, r = 96, 192, 256, 16
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    up = synth.to_bf16_bits(rng.standard_normal((N, r)) * 0.3)
    down = synth.to_bf16_bits(rng.standard_normal((r, K)) * 0.3)
    bias = synth.to_bf16_bits(rng.standard_normal(N))
    zc = np.zeros((N, K // 2), np.uint8)
    zs = np.zeros((N, K // 64), np.uint16)
    announce("zero residual layer")
    gc, gs, gt = gpu_quantize(0, x, None, down, K)
    y = gpu_gemm(0, gc, gs, zc, zs, gt, up, bias, zero_weight_ok=True)
    yp = gpu_gemm(0, gc, gs, zc, zs, gt, up, bias, zero_weight_ok=True, packed=True)
    yf = gpu_gemm(0, gc, gs, zc, zs, gt, up, bias, zero_weight_ok=True, fp6=True)
    assert np.array_equal(y, yp) and np.array_equal(y, yf)
    ref_t = (synth.bf16_bits_to_f32(x).astype(np.float64) @ synth.bf16_bits_to_f32(down).astype(np.float64).T)
    ref = oracle.f64_to_bf16(ref_t @ synth.bf16_bits_to_f32(up).astype(np.float64).T +
                             synth.bf16_bits_to_f32(bias).astype(np.float64)[None, :])
    assert_bf16_close(y, ref, "zero residual")


def test_layer_end_to_end_and_determinism():
    """GPU quantize -> GPU GEMM through the layer object equals the oracle's
    chain within the bar, and two runs give identical bits."""
    from bit_w4a4_quantized_svdq_amd.layer import SVDQW4A4Linear
    cfg = synth.TINY
    c = svdq_case(cfg, with_bias=True)
    layer = SVDQW4A4Linear("int4", c["wgt_codes"], c["wgt_scales"], c["lora_down"], c["lora_up"],
                           c["smooth"], c["bias"])
    xd = to_dev(c["x"], "bf16")
    announce("layer end to end", cfg.name)
    y1 = to_host(layer(xd).clone(), "bf16")
    y2 = to_host(layer(xd).clone(), "bf16")
    own = torch.empty((xd.shape[0], layer.N), dtype=torch.bfloat16, device="cuda")
    y3 = to_host(layer(xd, out=own), "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(y1, y2)
    assert np.array_equal(y1, y3)                 # a caller's output buffer: the same bits
    ac, asc, t = oracle.quantize_act(0, c["x"], c["smooth"], c["lora_down"])
    ref = oracle.gemm_w4a4(0, ac, asc, c["wgt_codes"], c["wgt_scales"], t, c["lora_up"], c["bias"])
    assert_bf16_close(y1, ref, "layer")


# ------------------------------------------------------------------ GEMV

@pytest.mark.parametrize("M,N,K,with_bias", [
    (1, 1024, 3072, False), (2, 512, 3072, True), (8, 256, 3072, False), (17, 100, 128, True),
    (70, 96, 64, True), (3, 5, 64, False), (16, 48, 4160, True),
    # small M with ragged N and K that is not a multiple of the 6-way K split
    # or of 4 groups (the 2-byte scale path), and large K (several x chunks)
    (1, 5, 64, True), (2, 33, 192, False), (1, 100, 4160, True), (2, 40, 8192, True), (1, 64, 8256, False),
    # K a multiple of 24 groups: 21 rows still take 8-byte scale loads, from 22
    # rows on (and every multi-tile M up to the GEMM's range) the 2-byte loads
    (21, 64, 1536, True), (22, 96, 3072, False), (32, 70, 1536, True), (64, 100, 3072, True),
    (255, 40, 3072, False),
    # tiles of 17..31 rows on the 2-byte path with several x copies per row
    (20, 64, 4096, True), (40, 50, 4160, False), (23, 33, 2240, True),
    # 8-byte scale loads with several x chunks (the first code loads go out
    # behind each chunk's x copy): 16-row tiles take 24 groups per chunk,
    # 2-row tiles 48
    (12, 96, 3072, True), (2, 64, 4608, False), (1, 32, 4608, True),
    # one or two rows with K a multiple of 512 up to 4096: the whole-line
    # stream (8 rows per wave, 24 per block), ragged N, every chunk count
    (1, 5, 512, True), (2, 33, 1024, False), (1, 25, 1536, False), (2, 48, 2048, True),
    (1, 71, 2560, True), (2, 24, 3584, False), (1, 49, 4096, True), (2, 100, 4096, True),
    # two to eight rows with K a multiple of 512 up to 4096: the whole-line
    # matrix-core stream (8 weight rows per wave; 4 waves per block up to 4
    # rows of x, 8 beyond), ragged N, every line count; the last two need more
    # than its LDS budget and take the one-row-per-lane GEMV
    (3, 7, 512, True), (4, 33, 1024, False), (5, 65, 1536, True), (6, 24, 2048, False),
    (7, 100, 2560, True), (8, 57, 3072, True), (3, 40, 3584, False), (4, 64, 4096, True),
    (5, 70, 4096, False), (2, 1, 512, False), (8, 200, 512, False),
    (8, 33, 4096, True), (8, 40, 3584, False),
])
def test_awq_gemv_shapes(M, N, K, with_bias):
    rng = np.random.default_rng(4000 + M + N + K)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    codes, scales, zeros = oracle.awq_quantize_weight(W)
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    announce("awq_gemv", M, N, K, "bias", with_bias)
    y = gpu_gemv(x, codes, scales, zeros, bias)
    ref = oracle.awq_gemv(x, codes, scales, zeros, bias)
    assert_bf16_close(y, ref, f"gemv {M}x{N}x{K}")


def awq_runs_as_gemm(M, N, K):
    """The library's choice between its AWQ GEMV and GEMM kernels (K a
    multiple of 512, at least 32 rows, at least 576 output tiles of 32 x 32)."""
    return K % 512 == 0 and M >= 32 and -(-M // 32) * -(-N // 32) >= 576


def gemm_tile_rows(M):
    """Rows of x that cover, in every 128-row GEMM tile, each position class
    of the kernel's row handling (the 8-row LDS swizzle, the 32-row MFMA
    blocks, the two 64-row wave halves), plus the ragged tail."""
    inner = np.array([0, 1, 7, 8, 30, 31, 33, 62, 63, 64, 66, 95, 96, 101, 126, 127])
    rows = np.concatenate([t + inner for t in range(0, M, 128)] + [np.arange(max(M - 3, 0), M)])
    return np.unique(rows[rows < M])


@pytest.mark.parametrize("M,N,K,with_bias,sampled", [
    # shapes in the GEMM regime: the smallest (one 128-row tile with 32 real
    # rows, 576 tiles exactly), ragged M and N, several scale chunks, the
    # smallest K; the larger K (3 and 8 scale chunks) on sampled rows
    (32, 18432, 512, False, False), (256, 2304, 512, True, False), (300, 2000, 1024, False, False),
    (513, 1200, 512, True, False), (1000, 600, 3072, False, True), (257, 2300, 4096, True, True),
])
def test_awq_gemm_regime_shapes(M, N, K, with_bias, sampled):
    assert awq_runs_as_gemm(M, N, K)
    rng = np.random.default_rng(4500 + M + N + K)
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    codes, scales, zeros = oracle.awq_quantize_weight(W)
    bias = synth.to_bf16_bits(rng.standard_normal(N)) if with_bias else None
    announce("awq gemm regime", M, N, K, "bias", with_bias)
    y = gpu_gemv(x, codes, scales, zeros, bias)
    rows = gemm_tile_rows(M) if sampled else np.arange(M)
    ref = oracle.awq_gemv(x[rows], codes, scales, zeros, bias)
    assert_bf16_close(y[rows], ref, f"awq gemm {M}x{N}x{K}")
    assert np.isfinite(synth.bf16_bits_to_f32(y)).all()


@pytest.mark.parametrize("M", [1, 4])
def test_awq_gemv_extreme_codes(M):
    """Codes 0 and 15 with zero points 0 and 15 (the (q - z) range ends)."""
    rng = np.random.default_rng(43)
    N, K = 64, 256
    x = synth.to_bf16_bits(rng.standard_normal((M, K)))
    q = np.where(rng.random((N, K)) < 0.5, 0, 15)
    codes = synth.pack_nibbles(q)
    scales = synth.to_bf16_bits(rng.uniform(0.001, 0.01, (N, K // 64)))
    zeros = synth.to_bf16_bits(np.where(rng.random((N, K // 64)) < 0.5, 0.0, 15.0))
    announce("awq_gemv extreme codes")
    y = gpu_gemv(x, codes, scales, zeros, None)
    ref = oracle.awq_gemv(x, codes, scales, zeros, None)
    assert_bf16_close(y, ref, "gemv extremes")


@pytest.mark.gpu
@pytest.mark.parametrize("nbytes", [16, 12288, 49152 * 3 + 4096 + 16, 1 << 22])
@pytest.mark.parametrize("pattern", [0, 1])
def test_stream_read_covers_every_chunk(nbytes, pattern):
    """The plain-read measurement kernel reads each whole 16-byte chunk of the
    range exactly once: the xor of every 12288-byte span's 32-bit words, in
    both access patterns, and nothing is written past the last span."""
    rng = np.random.default_rng(nbytes + pattern)
    host = rng.integers(0, 2 ** 32, nbytes // 4 + 16, dtype=np.uint32)
    dev = torch.from_numpy(host.view(np.int32)).cuda()
    spans = (nbytes + 12287) // 12288
    acc = torch.full((spans + 64,), 0x5A5A5A5A, dtype=torch.int32, device="cuda")
    announce("stream_read", nbytes, pattern)
    capi.svdq_debug_stream_read(dev, acc, pattern, nbytes)
    torch.cuda.synchronize()
    words = host[: (nbytes // 16) * 4]
    want = [np.bitwise_xor.reduce(words[i * 3072:(i + 1) * 3072]) for i in range(spans)]
    got = acc.cpu().numpy().view(np.uint32)
    assert [int(v) for v in got[:spans]] == [int(v) for v in want]
    assert (got[spans:] == 0x5A5A5A5A).all()
