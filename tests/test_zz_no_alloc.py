"""The allocation-free low-rank entry point (svdq_lowrank_factors_noalloc)
against svdq_lowrank_factors with a caller workspace: the same kernels, so
the factors must agree bit for bit, on two calls in a row (the second with a
smaller layer, on the scratch the first one left behind)."""
import numpy as np
import pytest
import torch

from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.gpu_helpers import announce, empty, poison, to_dev, to_host

pytestmark = [pytest.mark.gpu,
              pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")]


def _factors(W, s, rank, seed, noalloc):
    N, K = W.shape
    up, down = poison(empty((N, rank), "bf16")), poison(empty((rank, K), "bf16"))
    Wd, sd = to_dev(W, "bf16"), to_dev(s, "bf16")
    if noalloc:
        capi.svdq_lowrank_factors_noalloc(Wd, sd, rank, seed, up, down)
    else:
        ws = torch.empty(capi.svdq_lowrank_workspace_bytes(N, K, rank), dtype=torch.uint8, device="cuda")
        ws.fill_(0xFF)
        capi.svdq_lowrank_factors(Wd, sd, rank, seed, ws, up, down)
    torch.cuda.synchronize()
    return to_host(up, "bf16"), to_host(down, "bf16")


def test_lowrank_noalloc_matches_workspace_version():
    rng = np.random.default_rng(909)
    cases = [(12288, 3072, 32, 11), (1000, 640, 16, 12)]     # the second call is smaller
    for N, K, rank, seed in cases:
        W = synth.to_bf16_bits(rng.standard_normal((N, K)) * 0.02 +
                               np.outer(rng.standard_normal(N), rng.standard_normal(K)) * 0.01)
        s = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.3))
        announce("lowrank noalloc", N, K, rank, "seed", seed)
        up_n, down_n = _factors(W, s, rank, seed, noalloc=True)
        up_w, down_w = _factors(W, s, rank, seed, noalloc=False)
        assert np.array_equal(up_n, up_w), f"{N}x{K} r{rank}: lora_up differs"
        assert np.array_equal(down_n, down_w), f"{N}x{K} r{rank}: lora_down differs"
        assert np.isfinite(synth.bf16_bits_to_f32(down_n)).all() and np.any(down_n != 0)


def test_lowrank_noalloc_rejects_beyond_scratch():
    """65536 x 65536 at rank 128 needs far more than the fixed scratch: the
    host check refuses it and nothing is launched."""
    W = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    p = W.data_ptr()
    st = capi.lib().svdq_lowrank_factors_noalloc(65536, 65536, 128, p, None, 1, p, p, None)
    assert st == capi.SVDQ_ERR_INVALID_ARG
    assert "scratch" in capi.lib().svdq_last_error().decode()
    torch.cuda.synchronize()
