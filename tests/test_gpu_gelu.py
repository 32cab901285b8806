"""The GELU-fed activation step (svdq_gelu_quantize_act) against the oracle.

GELU (tanh form) of bf16 to bf16 is bit-exact for every input; codes and
scales of the step are bit-exact; lora_act within 1e-5 relative (fp32
summation order)."""
import numpy as np
import pytest
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import capi, synth
from tests.fp6_layout import fp6_layout_from_nibbles
from tests.gpu_helpers import announce, assert_f32_close, gpu_quantize

pytestmark = pytest.mark.gpu


def _check(prec, x, smooth, down, what):
    K = x.shape[1]
    announce("gelu_quantize_act", what, "prec", prec, "shape", x.shape, "rank", 0 if down is None else down.shape[0])
    gc, gs, gt = gpu_quantize(prec, x, smooth, down, K, gelu=True)
    oc, os_, ot = oracle.gelu_quantize_act(prec, x, smooth, down)
    assert np.array_equal(gs, os_), f"{what}: scales differ at {np.argwhere(gs != os_)[:5].tolist()}"
    assert np.array_equal(gc, oc), f"{what}: codes differ at {np.argwhere(gc != oc)[:5].tolist()}"
    if down is not None:
        assert_f32_close(gt, ot, 1e-5, what)
    if prec == 0:
        # the same step with the codes in the FP6 layout
        fc, fs, ft = gpu_quantize(3, x, smooth, down, K, gelu=True)
        assert np.array_equal(fs, os_), f"{what} fp6: scales differ"
        assert np.array_equal(fc, fp6_layout_from_nibbles(oc, K)), f"{what} fp6: code bytes differ"
        if down is not None:
            assert np.array_equal(ft, gt), f"{what} fp6: lora_act differs from the nibble output's"


def test_gelu_every_bf16():
    """All 65536 bf16 inputs (zeros, subnormals, both table edges, +-inf,
    NaNs) through the step's own GELU code."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    announce("gelu every bf16")
    x = torch.from_numpy(bits.view(np.int16)).cuda()
    out = torch.full_like(x, 0x5555)
    capi.svdq_debug_gelu_bf16(x, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    want = oracle.gelu_tanh_bf16(bits)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(hex(int(bits[i])), hex(int(got[i])), hex(int(want[i]))) for i in bad[:8]]


@pytest.mark.parametrize("prec,M,K,rank", [
    (0, 1, 64, 0), (0, 17, 192, 48), (0, 200, 512, 32), (0, 33, 4160, 16), (0, 40, 1024, 128),
    (1, 1, 64, 0), (1, 17, 192, 16), (1, 200, 512, 32), (1, 33, 4160, 128), (1, 40, 1024, 64),
])
def test_gelu_quantize_act_shapes(prec, M, K, rank):
    rng = np.random.default_rng(2000 + 7 * M + K + rank + prec)
    # pre-activations of an MLP up projection, some channels much larger
    u = rng.standard_normal((M, K)) * 2.0
    u[:, rng.choice(K, max(1, K // 100), replace=False)] *= 20.0
    x = synth.to_bf16_bits(u)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.7))
    down = synth.to_bf16_bits(rng.standard_normal((rank, K)) * 0.05) if rank else None
    _check(prec, x, smooth, down, f"M{M}_K{K}_r{rank}")


@pytest.mark.parametrize("prec", [0, 1])
def test_gelu_quantize_act_range_edges(prec):
    """Inputs at every boundary of the GELU's table and rules: just below and
    above 2^-14 and 128 in magnitude (the table's edges), 32 (where the
    |y| >= 32 rule starts inside the table), 2^-10 and 16, the two lowest
    binades (subnormal and least-normal ties), negative values whose GELU
    underflows, +-0, and large magnitudes (kept finite after the smoothing:
    an overflowing value is outside the step's contract)."""
    K = 256
    edges = [2.0 ** -10, 2.0 ** -10 * (1 - 2 ** -8), 16.0, 16.0 * (1 - 2 ** -8), 8.0, 2.0 ** -126,
             3 * 2.0 ** -133, 2.0 ** -133, 10.3, 10.5, 13.0, 21.5, 1.0e36, 0.75, 0.5234, 1.0,
             2.0 ** -14, 2.0 ** -14 * (1 - 2 ** -8), 32.0, 32.0 * (1 - 2 ** -8), 128.0, 128.0 * (1 - 2 ** -8),
             100.0]
    vals = np.array(edges + [-e for e in edges])
    x = synth.to_bf16_bits(np.resize(vals, (6, K)) * np.array([[1.0], [1.0], [-1.0], [0.5], [2.0], [1.0]]))
    x[5, :] = 0
    x[5, 1::2] = 0x8000                                   # -0
    rng = np.random.default_rng(11)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(K) * 0.3))
    down = synth.to_bf16_bits(rng.standard_normal((32, K)) * 0.05)
    _check(prec, x, smooth, down, "range edges")


def test_gelu_quantize_act_fullsize_mlp_down():
    """The MLP down layer's activation step (4096 x 12288, rank 32, int4) fed
    with the up layer's pre-activation output."""
    cfg = synth.MLP_DOWN
    h = synth.gelu_activations(synth.MLP_UP, cfg)
    rng = np.random.default_rng(cfg.seed + 300)
    smooth = synth.to_bf16_bits(np.exp(rng.standard_normal(cfg.K) * 0.25))
    down = synth.to_bf16_bits(rng.standard_normal((cfg.rank, cfg.K)) * 0.05)
    _check(oracle.INT4, h["u"], smooth, down, cfg.name)
