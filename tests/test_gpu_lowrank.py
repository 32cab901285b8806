"""The GPU's low-rank branch (randomized SVD) against the oracle's exact
truncated SVD, by the properties a correct branch has: its residual norm is
close to the Eckart-Young optimum, its row norms are the leading singular
values, its left factor is orthonormal (to bf16), and it is repeatable for a
seed.  The whole GPU preparation (smoothing, branch, 4-bit residual) is
compared with the oracle's on the reconstructed weight."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.gpu_helpers import announce, empty, poison, to_dev, to_host

pytestmark = pytest.mark.gpu


def _gpu_lowrank(W, smooth, rank, seed=1):
    N, K = W.shape
    ws = torch.empty(capi.svdq_lowrank_workspace_bytes(N, K, rank), dtype=torch.uint8, device="cuda")
    up, down = poison(empty((N, rank), "bf16")), poison(empty((rank, K), "bf16"))
    capi.svdq_lowrank_factors(to_dev(W, "bf16"), to_dev(smooth, "bf16"), rank, seed, ws, up, down)
    torch.cuda.synchronize()
    return to_host(up, "bf16"), to_host(down, "bf16")


def _f(b):
    return oracle.bf16_to_f32(b).astype(np.float64)


def _what(W, s):
    return _f(W) if s is None else _f(W) * _f(s)[None, :]


def _low_rank_plus_noise(rng, N, K, r0, noise):
    """A spectrum decaying geometrically from 0.5 to 5e-4 over r0 values, so
    that even its tail stays well above the bf16 rounding noise of W
    (~1e-4 in singular value at these sizes), plus Gaussian noise."""
    U, _ = np.linalg.qr(rng.standard_normal((N, r0)))
    V, _ = np.linalg.qr(rng.standard_normal((K, r0)))
    sig = 0.5 * (1e-3 ** (1.0 / r0)) ** np.arange(r0)
    return synth.to_bf16_bits(U @ np.diag(sig) @ V.T + noise * rng.standard_normal((N, K)))


@pytest.mark.parametrize("N,K,rank", [
    # l = rank + 8: Cholesky and Jacobi in LDS (24, 40), Cholesky in global
    # memory (56), both in global memory (72), and the largest l (136)
    (256, 512, 32), (200, 640, 16), (448, 192, 48), (320, 576, 64), (384, 640, 128),
])
def test_lowrank_decaying_spectrum(N, K, rank):
    rng = np.random.default_rng(7000 + N + K + rank)
    # noise far below the rank-th singular value (bf16 rounding of W dominates it)
    W = _low_rank_plus_noise(rng, N, K, rank + 24, 1e-6)
    s = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.3))
    announce("lowrank decaying", N, K, rank)
    up, down = _gpu_lowrank(W, s, rank)
    ou, od = oracle.lowrank_factors(_what(W, s), rank)
    A = _what(W, s)
    res_g = np.linalg.norm(A - _f(up) @ _f(down))
    res_o = np.linalg.norm(A - _f(ou) @ _f(od))
    assert res_g <= 1.01 * res_o, (res_g, res_o)
    sv = np.linalg.svd(A, compute_uv=False)[:rank]
    # Ritz estimates from a projection: never above the true values (beyond
    # rounding), within 1 % for all but the last 8, whose error grows as
    # sigma_j approaches sigma_{l+1}; within 5 % there
    got = np.linalg.norm(_f(down), axis=1)
    assert np.all(got <= sv * (1 + 3e-3)), np.stack([got, sv])[:, got > sv * (1 + 3e-3)]
    assert np.allclose(got[:-8], sv[:-8], rtol=1e-2), np.stack([got, sv])[:, :-8][:, np.abs(got[:-8] / sv[:-8] - 1) > 1e-2]
    assert np.all(got >= sv * 0.95), np.stack([got, sv])[:, got < sv * 0.95]
    # well-separated leading vectors: the same vectors and signs as the oracle
    cos = np.sum(_f(up) * _f(ou), axis=0) / (np.linalg.norm(_f(up), axis=0) * np.linalg.norm(_f(ou), axis=0))
    assert np.all(cos[:8] > 0.99), cos[:8]
    G = _f(up).T @ _f(up)
    assert np.abs(G - np.eye(rank)).max() < 2e-2


def test_lowrank_flat_spectrum_near_optimal():
    rng = np.random.default_rng(71)
    N, K, rank = 192, 640, 16
    W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02)
    announce("lowrank flat")
    up, down = _gpu_lowrank(W, None, rank)
    A = _what(W, None)
    sv = np.linalg.svd(A, compute_uv=False)
    optimal = np.sqrt(np.sum(sv[rank:] ** 2))
    res_g = np.linalg.norm(A - _f(up) @ _f(down))
    assert res_g <= 1.05 * optimal, (res_g, optimal)
    assert res_g >= optimal * (1 - 1e-3)   # no better than the optimum (up to bf16 rounding)


def test_lowrank_repeatable_for_a_seed():
    rng = np.random.default_rng(72)
    W = _low_rank_plus_noise(rng, 256, 256, 48, 1e-3)
    announce("lowrank repeatable")
    a = _gpu_lowrank(W, None, 32, seed=5)
    b = _gpu_lowrank(W, None, 32, seed=5)
    c = _gpu_lowrank(W, None, 32, seed=6)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    A = _what(W, None)
    optimal = np.sqrt(np.sum(np.linalg.svd(A, compute_uv=False)[32:] ** 2))
    for up, down in (a, c):   # both seeds near the optimum (a flat spectrum around rank 32 here)
        assert np.linalg.norm(A - _f(up) @ _f(down)) <= 1.03 * optimal


def test_gpu_preparation_end_to_end():
    """Smoothing factors, branch and 4-bit residual all on the GPU, against the
    oracle's preparation: the reconstructed smoothed weight up.down + deq(R)
    is as close to W diag(s) as the oracle's."""
    cfg = synth.LinearConfig("prep_e2e", 128, 512, 384, 32, "int4", 9, 5, 40.0)
    case = synth.linear_case(cfg)
    x, W = case["x"], case["W"]
    s = poison(empty((cfg.K,), "bf16"))
    capi.svdq_smooth_factors(to_dev(x, "bf16"), to_dev(W, "bf16"), s)
    torch.cuda.synchronize()
    s = to_host(s, "bf16")
    up, down = _gpu_lowrank(W, s, cfg.rank)
    codes, scales = poison(empty((cfg.N, cfg.K // 2), "u8")), poison(empty((cfg.N, cfg.K // 64), "bf16"))
    capi.svdq_quantize_weight(0, to_dev(W, "bf16"), to_dev(s, "bf16"), to_dev(up, "bf16"), to_dev(down, "bf16"),
                              codes, scales)
    torch.cuda.synchronize()
    codes, scales = to_host(codes, "u8"), to_host(scales, "bf16")
    p = oracle.prepare_svdq_weight(0, x, W, cfg.rank)
    assert np.array_equal(s, p["smooth"])
    announce("gpu preparation end to end")

    def recon(up_, down_, c_, sc_):
        q = oracle.unpack_int4(c_, cfg.N, cfg.K).astype(np.float64)
        return _f(up_) @ _f(down_) + q * np.repeat(_f(sc_), 64, axis=1)

    A = _what(W, s)
    err_g = np.linalg.norm(A - recon(up, down, codes, scales))
    err_o = np.linalg.norm(A - recon(p["lora_up"], p["lora_down"], p["wgt_codes"], p["wgt_scales"]))
    assert err_g <= 1.05 * err_o, (err_g, err_o)
