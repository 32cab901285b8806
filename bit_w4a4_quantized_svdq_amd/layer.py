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


def pack_weight_int4(wgt_codes, wgt_scales):
    """Device int4 codes [N, K/2] + bf16 scales -> the packed weight blob of the
    SVDQ_INT4_PACKED GEMM (raises if a code is -8)."""
    N, Kh = wgt_codes.shape
    blob = torch.empty((capi.svdq_packed_weight_bytes(N, 2 * Kh),), dtype=torch.uint8, device=wgt_codes.device)
    bad = torch.empty((1,), dtype=torch.int32, device=wgt_codes.device)
    capi.svdq_pack_weight_int4(wgt_codes, wgt_scales, blob, bad)
    if int(bad.item()) != 0:
        raise ValueError(f"{int(bad.item())} weight codes of -8 cannot be packed")
    return blob


def pack_weight_fp6(wgt_codes):
    """Device int4 codes [N, K/2] -> their FP6 tiled layout (the weight
    operand of the SVDQ_INT4_FP6 GEMM)."""
    N, Kh = wgt_codes.shape
    out = torch.empty((capi.svdq_fp6_codes_bytes(N, 2 * Kh),), dtype=torch.uint8, device=wgt_codes.device)
    capi.svdq_pack_weight_fp6(wgt_codes, out)
    return out


class SVDQW4A4Linear:
    """y = alpha * Q(x/s) . Q(R)^T + (x/s . L1^T) . L2^T + bias  (bf16 out).

    precision: "int4" (group 64, bf16 scales) or "nvfp4" (group 16, E4M3).
    int4_layout (int4 only), how the codes reach the GEMM (same codes, scales
    and results within the output tolerance):
      "fp6"    both operands in the FP6 layout (SVDQ_INT4_FP6; the weight is
               re-encoded once, at construction) -- the fastest path;
      "packed" the weight re-encoded by svdq_pack_weight_int4
               (SVDQ_INT4_PACKED; codes of -8, which the group quantizer
               never produces, are refused);
      "plain"  packed nibbles on both sides (SVDQ_INT4)."""

    def __init__(self, precision, wgt_codes, wgt_scales, lora_down, lora_up, smooth=None,
                 bias=None, alpha=1.0, device="cuda", int4_layout="fp6"):
        self.prec = capi.SVDQ_INT4 if precision == "int4" else capi.SVDQ_NVFP4
        self.group = 64 if self.prec == capi.SVDQ_INT4 else 16
        self.wgt_codes = _dev(wgt_codes, torch.uint8, device)
        sdt = torch.bfloat16 if self.prec == capi.SVDQ_INT4 else torch.uint8
        self.wgt_scales = _dev(wgt_scales, sdt, device)
        self.gemm_prec = self.act_prec = self.prec
        if self.prec == capi.SVDQ_INT4:
            if int4_layout == "fp6":
                self.wgt_codes = pack_weight_fp6(self.wgt_codes)
                self.gemm_prec = self.act_prec = capi.SVDQ_INT4_FP6
            elif int4_layout == "packed":
                self.wgt_codes = pack_weight_int4(self.wgt_codes, self.wgt_scales)
                self.gemm_prec = capi.SVDQ_INT4_PACKED
            elif int4_layout != "plain":
                raise ValueError(f"int4_layout must be 'fp6', 'packed' or 'plain' (got {int4_layout!r})")
        self.lora_down = _dev(lora_down, torch.bfloat16, device)
        self.lora_up = _dev(lora_up, torch.bfloat16, device)
        self.smooth = _dev(smooth, torch.bfloat16, device)
        self.bias = _dev(bias, torch.bfloat16, device)
        self.alpha = float(alpha)
        self.N, G = self.wgt_scales.shape
        self.K = G * self.group
        self.rank = 0 if self.lora_up is None else self.lora_up.shape[1]
        self.device = device
        self._bufs = {}

    def buffers(self, M):
        b = self._bufs.get(M)
        if b is None:
            d = self.device
            sdt = torch.bfloat16 if self.prec == capi.SVDQ_INT4 else torch.uint8
            shape = ((capi.svdq_fp6_codes_bytes(M, self.K),) if self.act_prec == capi.SVDQ_INT4_FP6
                     else (M, self.K // 2))
            b = {"codes": torch.empty(shape, dtype=torch.uint8, device=d),
                 "scales": torch.empty((M, self.K // self.group), dtype=sdt, device=d),
                 "lora_act": torch.empty((M, max(self.rank, 1)), dtype=torch.float32, device=d),
                 "out": torch.empty((M, self.N), dtype=torch.bfloat16, device=d)}
            self._bufs[M] = b
        return b

    def quantize(self, x, b, gelu=False):
        """The activation step into the buffers ``b``; with ``gelu`` x is the
        preceding GELU MLP up projection's output and GELU runs inside the step."""
        fn = capi.svdq_gelu_quantize_act if gelu else capi.svdq_quantize_act
        fn(self.act_prec, x, self.smooth, self.lora_down, b["codes"], b["scales"],
           b["lora_act"] if self.rank else None)

    def gemm(self, b, out=None):
        capi.svdq_gemm_w4a4(self.gemm_prec, b["codes"], b["scales"], self.wgt_codes, self.wgt_scales,
                            self.alpha, b["lora_act"] if self.rank else None, self.lora_up,
                            self.bias, b["out"] if out is None else out)

    def gemm_qk_norm_rope(self, b, q_norm_weight, k_norm_weight, eps, rope_cos, rope_sin):
        """The GEMM step of a grouped QKV layer (N = 3 * heads * 128) with
        per-head RMSNorm and rotary embedding of Q and K in its epilogue."""
        capi.svdq_gemm_w4a4_qk_norm_rope(self.gemm_prec, b["codes"], b["scales"], self.wgt_codes,
                                         self.wgt_scales, self.alpha,
                                         b["lora_act"] if self.rank else None, self.lora_up, self.bias,
                                         q_norm_weight, k_norm_weight, eps, rope_cos, rope_sin, b["out"])

    def gemm_gelu_quantize(self, b, nxt, nb, out=None):
        """The GEMM step of a GELU MLP's up projection with the down layer
        ``nxt``'s activation step in its epilogue: writes nxt's codes, scales
        and lora_act into its buffers ``nb`` (and this layer's output into
        ``out`` when given).  Both layers int4 in the FP6 layout."""
        if self.gemm_prec != capi.SVDQ_INT4_FP6 or nxt.act_prec != capi.SVDQ_INT4_FP6 or nxt.K != self.N:
            raise ValueError("gemm_gelu_quantize: both layers int4 in the FP6 layout, nxt.K == N")
        M = nb["scales"].shape[0]
        ws = b.get("gq_workspace")
        need = capi.svdq_gelu_quantize_workspace_bytes(M, self.N, nxt.rank)
        if need > 0 and (ws is None or ws.numel() < need):
            ws = b["gq_workspace"] = torch.empty((need,), dtype=torch.uint8, device=self.device)
        if need == 0:
            ws = None
        capi.svdq_gemm_w4a4_gelu_quantize(b["codes"], b["scales"], self.wgt_codes, self.wgt_scales, self.alpha,
                                          b["lora_act"] if self.rank else None, self.lora_up, self.bias,
                                          nxt.smooth, nxt.lora_down, nb["codes"], nb["scales"],
                                          nb["lora_act"] if nxt.rank else None, ws, out)

    def forward(self, x, out=None):
        """x: bf16 [M,K] device tensor -> bf16 [M,N].  Without ``out`` the
        result is the layer's own buffer for this M, which the next call with
        the same M overwrites; pass ``out`` (bf16 [M,N], contiguous, on the
        device) to keep results apart."""
        b = self.buffers(x.shape[0])
        self.quantize(x, b)
        self.gemm(b, out)
        return b["out"] if out is None else out

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

    def forward(self, x, out=None):
        """x: bf16 [M,K] -> bf16 [M,N]; without ``out`` the result is a buffer
        of the layer's own, reused by the next call with the same M."""
        M = x.shape[0]
        if out is None:
            out = self._out.get(M)
            if out is None:
                out = self._out[M] = torch.empty((M, self.N), dtype=torch.bfloat16, device=self.device)
        capi.awq_gemv_w4a16(x, self.wgt_codes, self.wgt_scales, self.wgt_zeros, self.bias, out)
        return out

    __call__ = forward
