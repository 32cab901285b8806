"""Thin Python binding of libsvdq's C ABI (include/svdq.h).

The functions carry the C names and only marshal arguments: sizes are read
from the tensor shapes, device pointers from ``tensor.data_ptr()``, and the
stream is torch's current HIP stream unless one is given.  Every step of the
layer runs in the HIP kernels of libsvdq.so; there is no fallback: if the
library is missing, importing the entry points raises.

Tensors use torch dtypes as storage: bf16 tensors are ``torch.bfloat16``
(or ``torch.int16`` / ``uint16`` views of the bits), packed codes and E4M3
scales are ``torch.uint8``, lora_act is ``torch.float32``.
"""
from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "_lib", "libsvdq.so")

SVDQ_OK, SVDQ_ERR_INVALID_ARG, SVDQ_ERR_UNSUPPORTED, SVDQ_ERR_HIP = 0, 1, 2, 3
SVDQ_INT4, SVDQ_NVFP4 = 0, 1

EXPORTED = ("svdq_quantize_act", "svdq_gelu_quantize_act", "svdq_gemm_w4a4", "svdq_gemm_w4a4_qk_norm_rope",
            "awq_gemv_w4a16",
            "svdq_smooth_factors", "svdq_quantize_weight", "svdq_lowrank_workspace_bytes",
            "svdq_lowrank_factors",
            "svdq_debug_group_sums", "svdq_debug_gelu_bf16", "svdq_status_string", "svdq_last_error",
            "svdq_abi_version")


class SvdqError(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        self.status = status
        super().__init__(f"{func}: {_status_text(status)} ({detail})")


_lib = None
_P, _I64, _I32, _F32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_float


def lib() -> ctypes.CDLL:
    """The loaded libsvdq.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m bit_w4a4_quantized_svdq_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        L.svdq_quantize_act.argtypes = [_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_gelu_quantize_act.argtypes = [_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_gemm_w4a4.argtypes = [_I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _F32, _P, _P, _P,
                                     _P, _P]
        L.svdq_gemm_w4a4_qk_norm_rope.argtypes = [_I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _F32, _P, _P,
                                                  _P, _P, _P, _F32, _P, _P, _P, _P]
        L.awq_gemv_w4a16.argtypes = [_I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_debug_group_sums.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_debug_gelu_bf16.argtypes = [_I64, _P, _P, _P]
        L.svdq_smooth_factors.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_quantize_weight.argtypes = [_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_lowrank_workspace_bytes.argtypes = [_I64, _I64, _I32]
        L.svdq_lowrank_workspace_bytes.restype = _I64
        L.svdq_lowrank_factors.argtypes = [_I64, _I64, _I32, _P, _P, ctypes.c_uint64, _P, _I64, _P, _P, _P]
        for f in ("svdq_quantize_act", "svdq_gelu_quantize_act", "svdq_gemm_w4a4",
                  "svdq_gemm_w4a4_qk_norm_rope", "awq_gemv_w4a16",
                  "svdq_debug_group_sums", "svdq_debug_gelu_bf16", "svdq_smooth_factors",
                  "svdq_quantize_weight", "svdq_lowrank_factors"):
            getattr(L, f).restype = ctypes.c_int
        L.svdq_status_string.argtypes = [ctypes.c_int]
        L.svdq_status_string.restype = ctypes.c_char_p
        L.svdq_last_error.argtypes = []
        L.svdq_last_error.restype = ctypes.c_char_p
        L.svdq_abi_version.argtypes = []
        L.svdq_abi_version.restype = ctypes.c_int32
        _lib = L
    return _lib


def _status_text(status: int) -> str:
    return lib().svdq_status_string(status).decode()


def svdq_status_string(status: int) -> str:
    return _status_text(status)


def svdq_last_error() -> str:
    return lib().svdq_last_error().decode()


def svdq_abi_version() -> int:
    return int(lib().svdq_abi_version())


def _check(status: int, func: str):
    if status != SVDQ_OK:
        raise SvdqError(status, func, svdq_last_error())


def _ptr(t):
    return None if t is None else t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def svdq_quantize_act(precision, x, smooth, lora_down, act_codes, act_scales, lora_act,
                      stream=None):
    """Smooth, low-rank down-projection and group quantization of x [M,K]."""
    M, K = x.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    _check(lib().svdq_quantize_act(precision, M, K, rank, _ptr(x), _ptr(smooth), _ptr(lora_down),
                                   _ptr(act_codes), _ptr(act_scales), _ptr(lora_act),
                                   _stream(stream)), "svdq_quantize_act")


def svdq_gelu_quantize_act(precision, x, smooth, lora_down, act_codes, act_scales, lora_act,
                           stream=None):
    """svdq_quantize_act of GELU(x) (tanh form), x being a GELU MLP's up-projection output."""
    M, K = x.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    _check(lib().svdq_gelu_quantize_act(precision, M, K, rank, _ptr(x), _ptr(smooth), _ptr(lora_down),
                                        _ptr(act_codes), _ptr(act_scales), _ptr(lora_act),
                                        _stream(stream)), "svdq_gelu_quantize_act")


def svdq_gemm_w4a4(precision, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                   lora_up, bias, out, stream=None):
    """4-bit GEMM with the low-rank up-projection and bias; out is [M,N] bf16."""
    M = act_codes.shape[0]
    N, Kh = wgt_codes.shape
    rank = 0 if lora_up is None else lora_up.shape[1]
    _check(lib().svdq_gemm_w4a4(precision, M, N, 2 * Kh, rank, _ptr(act_codes), _ptr(act_scales),
                                _ptr(wgt_codes), _ptr(wgt_scales), float(alpha), _ptr(lora_act),
                                _ptr(lora_up), _ptr(bias), _ptr(out), _stream(stream)),
           "svdq_gemm_w4a4")


def svdq_gemm_w4a4_qk_norm_rope(precision, act_codes, act_scales, wgt_codes, wgt_scales, alpha,
                                lora_act, lora_up, bias, q_norm_weight, k_norm_weight, eps, rope_cos,
                                rope_sin, out, stream=None):
    """4-bit GEMM of a grouped QKV layer with per-head RMSNorm + rotary embedding
    of Q and K in the epilogue; out is [M, 3*H*128] bf16."""
    M = act_codes.shape[0]
    N, Kh = wgt_codes.shape
    rank = 0 if lora_up is None else lora_up.shape[1]
    _check(lib().svdq_gemm_w4a4_qk_norm_rope(precision, M, N, 2 * Kh, rank, _ptr(act_codes),
                                             _ptr(act_scales), _ptr(wgt_codes), _ptr(wgt_scales),
                                             float(alpha), _ptr(lora_act), _ptr(lora_up), _ptr(bias),
                                             _ptr(q_norm_weight), _ptr(k_norm_weight), float(eps),
                                             _ptr(rope_cos), _ptr(rope_sin), _ptr(out), _stream(stream)),
           "svdq_gemm_w4a4_qk_norm_rope")


def awq_gemv_w4a16(x, wgt_codes, wgt_scales, wgt_zeros, bias, out, group_size=64, stream=None):
    """int4 weight-only layer: out[M,N] = x . dequant(W)^T + bias."""
    M, K = x.shape
    N = wgt_codes.shape[0]
    _check(lib().awq_gemv_w4a16(M, N, K, group_size, _ptr(x), _ptr(wgt_codes), _ptr(wgt_scales),
                                _ptr(wgt_zeros), _ptr(bias), _ptr(out), _stream(stream)),
           "awq_gemv_w4a16")


def svdq_smooth_factors(x, W, smooth, stream=None):
    """Smoothing factors [K] from calibration activations x [M,K] and the weight W [N,K]."""
    M, K = x.shape
    _check(lib().svdq_smooth_factors(M, W.shape[0], K, _ptr(x), _ptr(W), _ptr(smooth), _stream(stream)),
           "svdq_smooth_factors")


def svdq_lowrank_workspace_bytes(N, K, rank) -> int:
    return int(lib().svdq_lowrank_workspace_bytes(N, K, rank))


def svdq_lowrank_factors(W, smooth, rank, seed, workspace, lora_up, lora_down, stream=None):
    """Low-rank branch (randomized SVD) of W diag(smooth); workspace: a uint8 device tensor."""
    N, K = W.shape
    _check(lib().svdq_lowrank_factors(N, K, rank, _ptr(W), _ptr(smooth), int(seed), _ptr(workspace),
                                      workspace.numel(), _ptr(lora_up), _ptr(lora_down), _stream(stream)),
           "svdq_lowrank_factors")


def svdq_quantize_weight(precision, W, smooth, lora_up, lora_down, wgt_codes, wgt_scales, stream=None):
    """4-bit residual of the smoothed weight after the low-rank branch, group-quantized."""
    N, K = W.shape
    rank = 0 if lora_up is None else lora_up.shape[1]
    _check(lib().svdq_quantize_weight(precision, N, K, rank, _ptr(W), _ptr(smooth), _ptr(lora_up),
                                      _ptr(lora_down), _ptr(wgt_codes), _ptr(wgt_scales), _stream(stream)),
           "svdq_quantize_weight")


def svdq_debug_gelu_bf16(x, out, stream=None):
    """GELU of bf16 values on the GELU-quantize step's own device code."""
    _check(lib().svdq_debug_gelu_bf16(x.numel(), _ptr(x), _ptr(out), _stream(stream)),
           "svdq_debug_gelu_bf16")


def svdq_debug_group_sums(act_codes, wgt_codes, G, stream=None):
    """Exact int32 group sums [M,N,K/64] on the int4 GEMM's device path."""
    M, Kh = act_codes.shape
    N = wgt_codes.shape[0]
    _check(lib().svdq_debug_group_sums(M, N, 2 * Kh, _ptr(act_codes), _ptr(wgt_codes), _ptr(G),
                                       _stream(stream)), "svdq_debug_group_sums")
