"""Layer objects over the C ABI: an SVDQuant W4A4 linear layer and an
AWQ-style W4A16 linear layer whose weights live on the GPU.

A W4A4 forward is the two fused kernels of the method (blog "Hugging Face
integrates Nunchaku 4-bit diffusion inference into Diffusers", "SVDQuant and
the Nunchaku engine"): ``svdq_quantize_act`` (smooth + low-rank down-
projection + 4-bit group quantization) and ``svdq_gemm_w4a4`` (4-bit GEMM
with the low-rank up-projection and bias).  Buffers for the intermediate
codes, scales and low-rank activations are allocated once per batch size
and reused, so steady-state forwards allocate nothing.
"""
from __future__ import annotations

import numpy as np
import torch

from . import capi


def _dev(a, dtype, device):
    """numpy array (bf16 bits as uint16) -> device tensor of the storage dtype."""
    if a is None:
        return None
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is torch.bfloat16:
        t = t.view(torch.int16).view(torch.bfloat16)
    return t.to(device)


class SVDQW4A4Linear:
    """y = alpha * Q(x/s) . Q(R)^T + (x/s . L1^T) . L2^T + bias  (bf16 out).

    precision: "int4" (group 64, bf16 scales) or "nvfp4" (group 16, E4M3)."""

    def __init__(self, precision, wgt_codes, wgt_scales, lora_down, lora_up, smooth=None,
                 bias=None, alpha=1.0, device="cuda"):
        self.prec = capi.SVDQ_INT4 if precision == "int4" else capi.SVDQ_NVFP4
        self.group = 64 if self.prec == capi.SVDQ_INT4 else 16
        self.wgt_codes = _dev(wgt_codes, torch.uint8, device)
        sdt = torch.bfloat16 if self.prec == capi.SVDQ_INT4 else torch.uint8
        self.wgt_scales = _dev(wgt_scales, sdt, device)
        self.lora_down = _dev(lora_down, torch.bfloat16, device)
        self.lora_up = _dev(lora_up, torch.bfloat16, device)
        self.smooth = _dev(smooth, torch.bfloat16, device)
        self.bias = _dev(bias, torch.bfloat16, device)
        self.alpha = float(alpha)
        self.N, Kh = self.wgt_codes.shape
        self.K = 2 * Kh
        self.rank = 0 if self.lora_up is None else self.lora_up.shape[1]
        self.device = device
        self._bufs = {}

    def buffers(self, M):
        b = self._bufs.get(M)
        if b is None:
            d = self.device
            sdt = torch.bfloat16 if self.prec == capi.SVDQ_INT4 else torch.uint8
            b = {"codes": torch.empty((M, self.K // 2), dtype=torch.uint8, device=d),
                 "scales": torch.empty((M, self.K // self.group), dtype=sdt, device=d),
                 "lora_act": torch.empty((M, max(self.rank, 1)), dtype=torch.float32, device=d),
                 "out": torch.empty((M, self.N), dtype=torch.bfloat16, device=d)}
            self._bufs[M] = b
        return b

    def quantize(self, x, b, gelu=False):
        """The activation step into the buffers ``b``; with ``gelu`` x is the
        preceding GELU MLP up projection's output and GELU runs inside the step."""
        fn = capi.svdq_gelu_quantize_act if gelu else capi.svdq_quantize_act
        fn(self.prec, x, self.smooth, self.lora_down, b["codes"], b["scales"],
           b["lora_act"] if self.rank else None)

    def gemm(self, b):
        capi.svdq_gemm_w4a4(self.prec, b["codes"], b["scales"], self.wgt_codes, self.wgt_scales,
                            self.alpha, b["lora_act"] if self.rank else None, self.lora_up,
                            self.bias, b["out"])

    def gemm_qk_norm_rope(self, b, q_norm_weight, k_norm_weight, eps, rope_cos, rope_sin):
        """The GEMM step of a grouped QKV layer (N = 3 * heads * 128) with
        per-head RMSNorm and rotary embedding of Q and K in its epilogue."""
        capi.svdq_gemm_w4a4_qk_norm_rope(self.prec, b["codes"], b["scales"], self.wgt_codes,
                                         self.wgt_scales, self.alpha,
                                         b["lora_act"] if self.rank else None, self.lora_up, self.bias,
                                         q_norm_weight, k_norm_weight, eps, rope_cos, rope_sin, b["out"])

    def forward(self, x):
        """x: bf16 [M,K] device tensor -> bf16 [M,N] (a reused buffer)."""
        b = self.buffers(x.shape[0])
        self.quantize(x, b)
        self.gemm(b)
        return b["out"]

    __call__ = forward


class AWQW4A16Linear:
    """y = x . ((q - z) * s)^T + bias with int4 weights in groups of 64.

    wgt_codes [N, K/2]; wgt_scales and wgt_zeros [N, K/64]."""

    def __init__(self, wgt_codes, wgt_scales, wgt_zeros, bias=None, device="cuda"):
        self.wgt_codes = _dev(wgt_codes, torch.uint8, device)
        self.wgt_scales = _dev(wgt_scales, torch.bfloat16, device)
        self.wgt_zeros = _dev(wgt_zeros, torch.bfloat16, device)
        self.bias = _dev(bias, torch.bfloat16, device)
        self.N, Kh = self.wgt_codes.shape
        self.K = 2 * Kh
        self.device = device
        self._out = {}

    def forward(self, x):
        M = x.shape[0]
        out = self._out.get(M)
        if out is None:
            out = self._out[M] = torch.empty((M, self.N), dtype=torch.bfloat16, device=self.device)
        capi.awq_gemv_w4a16(x, self.wgt_codes, self.wgt_scales, self.wgt_zeros, self.bias, out)
        return out

    __call__ = forward
