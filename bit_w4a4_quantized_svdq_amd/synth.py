"""Seeded synthetic inputs for the W4A4 / W4A16 layers.

This module only draws random numbers and converts them to the storage
formats the layers take (bf16 bit patterns, packed nibbles).  It holds none
of the method's arithmetic (no smoothing, no SVD, no quantization rule):
those steps live in the kernels and in the independent CPU checker.

The workloads are DiT-shaped stand-ins for the image transformers the pages
benchmark (ERNIE-Image-Turbo and Flux at 1024x1024, blog "Hugging Face
integrates Nunchaku 4-bit diffusion inference into Diffusers", "Benchmarks"):
a 1024x1024 image is a 64x64 latent patch grid, i.e. 4096 tokens, hidden
size 3072, fused QKV width 9216 (the Q/K/V -> to_qkv rewrite of the
"Structural rewrite" section), MLP width 12288, and a 6x3072 adaptive-norm
modulation projection for the weight-only layer ("memory-bound,
precision-sensitive layers such as adaptive normalization").

Recipe (numpy PCG64 ``default_rng(seed)``, fixed draw order):
  x  = N(0,1) [M,K] drawn in fp64; ``n_outliers`` channels chosen with
       ``rng.choice(K, n_outliers, replace=False)`` are multiplied by
       ``outlier_scale``;
  W  = N(0, 0.02) [N,K] drawn in fp64;
  bias (when asked) = N(0,1) [N];
every fp64 draw is cast to fp32 and then rounded to bf16 by torch (RNE).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np
import torch


def to_bf16_bits(a) -> np.ndarray:
    """fp64/fp32 numpy array -> bf16 bit patterns (uint16), via torch RNE."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(h) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << 16).view(np.float32)


@dataclasses.dataclass(frozen=True)
class LinearConfig:
    name: str
    M: int
    K: int
    N: int
    rank: int
    precision: str          # "int4" | "nvfp4" | "awq"
    seed: int
    n_outliers: int
    outlier_scale: float
    w_std: float = 0.02


TINY = LinearConfig("tiny_w4a4_int4", 64, 256, 256, 16, "int4", 0, 4, 30.0)
QKV = LinearConfig("dit_qkv_w4a4_int4", 4096, 3072, 9216, 32, "int4", 1, 31, 50.0)
MLP_UP = LinearConfig("dit_mlp_up_w4a4_int4", 4096, 3072, 12288, 32, "int4", 2, 31, 50.0)
MLP_DOWN = LinearConfig("dit_mlp_down_w4a4_int4", 4096, 12288, 3072, 32, "int4", 2, 0, 1.0)
ATTN_OUT_NVFP4 = LinearConfig("dit_attn_out_w4a4_nvfp4", 4096, 3072, 3072, 32, "nvfp4", 3, 31, 50.0)
ADALN_AWQ = LinearConfig("dit_adaln_w4a16_awq", 8, 3072, 18432, 0, "awq", 4, 0, 1.0)

CONFIGS = {c.name: c for c in (TINY, QKV, MLP_UP, MLP_DOWN, ATTN_OUT_NVFP4, ADALN_AWQ)}


def draw_activations(rng, M, K, n_outliers, outlier_scale):
    x = rng.standard_normal((M, K))
    idx = np.sort(rng.choice(K, n_outliers, replace=False)) if n_outliers else np.zeros(0, np.int64)
    x[:, idx] *= outlier_scale
    return x, idx


def linear_case(cfg: LinearConfig, M: int | None = None, with_bias: bool = False):
    """Activations, weight and optional bias of one layer (bf16 bits).

    The MLP down layer's input is drawn by :func:`gelu_activations` instead."""
    rng = np.random.default_rng(cfg.seed)
    M = cfg.M if M is None else M
    x, idx = draw_activations(rng, M, cfg.K, cfg.n_outliers, cfg.outlier_scale)
    W = rng.standard_normal((cfg.N, cfg.K)) * cfg.w_std
    out = {"x": to_bf16_bits(x), "W": to_bf16_bits(W), "outliers": idx}
    out["bias"] = to_bf16_bits(rng.standard_normal(cfg.N)) if with_bias else None
    return out


def gelu_tanh(u):
    """GELU, tanh form -- the MLP activation between the two layers (not part
    of the quantized layer itself)."""
    return 0.5 * u * (1.0 + np.tanh(math.sqrt(2.0 / math.pi) * (u + 0.044715 * u ** 3)))


def gelu_activations(cfg_up: LinearConfig, cfg_down: LinearConfig, M: int | None = None):
    """Input of the MLP down layer: bf16(gelu_tanh(u)), u ~ N(0, sigma^2);
    also bf16(u) itself ("u", the up layer's output before the activation).

    sigma is the standard deviation of the up layer's output for the up
    layer's own input distribution: sqrt(w_std^2 * (K - n + n*scale^2)).
    The draw uses seed ``cfg_down.seed + 100`` so it does not repeat the up
    layer's stream."""
    M = cfg_down.M if M is None else M
    rng = np.random.default_rng(cfg_down.seed + 100)
    n, s = cfg_up.n_outliers, cfg_up.outlier_scale
    sigma = cfg_up.w_std * math.sqrt(cfg_up.K - n + n * s * s)
    u = rng.standard_normal((M, cfg_down.K)) * sigma
    W = rng.standard_normal((cfg_down.N, cfg_down.K)) * cfg_down.w_std
    return {"x": to_bf16_bits(gelu_tanh(u)), "u": to_bf16_bits(u), "W": to_bf16_bits(W), "sigma": sigma}


def pack_nibbles(vals) -> np.ndarray:
    """int array [R,K] with values in [-8,15] -> packed bytes [R,K/2]
    (element k in byte k/2, even k in the low nibble)."""
    v = np.asarray(vals).astype(np.int64) & 0xF
    return (v[:, 0::2] | (v[:, 1::2] << 4)).astype(np.uint8)


def synthetic_w4a4_weights(seed: int, N: int, K: int, rank: int, precision: str):
    """Random already-quantized weight-side tensors of a W4A4 layer, for
    timing runs that must not depend on the CPU checker.

    int4: codes uniform in [-7,7], bf16 scales 0.02*(2+|N(0,1)|)/7.
    nvfp4: E2M1 codes uniform over the 16 nibbles, E4M3 scale bytes drawn
    from the normal range (exponent field 1..10).  lora_up ~ N(0,1/N),
    lora_down ~ N(0, 0.05), smooth = exp(N(0, 0.25)); all bf16."""
    rng = np.random.default_rng(seed)
    if precision == "int4":
        codes = pack_nibbles(rng.integers(-7, 8, size=(N, K)))
        scales = to_bf16_bits(0.02 * (2.0 + np.abs(rng.standard_normal((N, K // 64)))) / 7.0)
    else:
        codes = pack_nibbles(rng.integers(0, 16, size=(N, K)))
        scales = ((rng.integers(1, 11, size=(N, K // 16)) << 3) |
                  rng.integers(0, 8, size=(N, K // 16))).astype(np.uint8)
    lora_up = to_bf16_bits(rng.standard_normal((N, rank)) / math.sqrt(N)) if rank else None
    lora_down = to_bf16_bits(rng.standard_normal((rank, K)) * 0.05) if rank else None
    smooth = to_bf16_bits(np.exp(rng.standard_normal(K) * 0.25))
    return {"wgt_codes": codes, "wgt_scales": scales, "lora_up": lora_up,
            "lora_down": lora_down, "smooth": smooth}


def synthetic_awq_weights(seed: int, N: int, K: int):
    """Random AWQ weight tensors: unsigned codes uniform in [0,15], bf16
    scales 0.02*(2+|N(0,1)|)/15, bf16 integer zero points uniform in [4,11].
    Scales and zero points are [N, K/64]."""
    rng = np.random.default_rng(seed)
    codes = pack_nibbles(rng.integers(0, 16, size=(N, K)))
    scales = to_bf16_bits(0.02 * (2.0 + np.abs(rng.standard_normal((N, K // 64)))) / 15.0)
    zeros = to_bf16_bits(rng.integers(4, 12, size=(N, K // 64)).astype(np.float64))
    return {"wgt_codes": codes, "wgt_scales": scales, "wgt_zeros": zeros}
