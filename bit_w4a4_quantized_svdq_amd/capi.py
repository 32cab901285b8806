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
SVDQ_INT4, SVDQ_NVFP4, SVDQ_INT4_PACKED, SVDQ_INT4_FP6 = 0, 1, 2, 3

EXPORTED = ("svdq_quantize_act", "svdq_gelu_quantize_act", "svdq_gemm_w4a4", "svdq_gemm_w4a4_qk_norm_rope",
            "svdq_gelu_quantize_workspace_bytes", "svdq_gemm_w4a4_gelu_quantize",
            "awq_gemv_w4a16",
            "svdq_smooth_factors", "svdq_quantize_weight", "svdq_lowrank_workspace_bytes",
            "svdq_lowrank_factors", "svdq_lowrank_factors_noalloc",
            "svdq_packed_weight_bytes", "svdq_pack_weight_int4", "svdq_debug_group_sums_packed",
            "svdq_fp6_codes_bytes", "svdq_pack_weight_fp6", "svdq_debug_group_sums_fp6",
            "svdq_debug_group_sums", "svdq_debug_gelu_bf16", "svdq_debug_stream_read",
            "svdq_status_string", "svdq_last_error",
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
        L.svdq_gelu_quantize_workspace_bytes.argtypes = [_I64, _I64, _I32]
        L.svdq_gelu_quantize_workspace_bytes.restype = _I64
        L.svdq_gemm_w4a4_gelu_quantize.argtypes = [_I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _F32, _P, _P, _P,
                                                   _I32, _P, _P, _P, _P, _P, _P, _I64, _P, _P]
        L.awq_gemv_w4a16.argtypes = [_I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_debug_group_sums.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_debug_group_sums_packed.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_packed_weight_bytes.argtypes = [_I64, _I64]
        L.svdq_packed_weight_bytes.restype = _I64
        L.svdq_pack_weight_int4.argtypes = [_I64, _I64, _P, _P, _P, _P, _P]
        L.svdq_debug_group_sums_fp6.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_fp6_codes_bytes.argtypes = [_I64, _I64]
        L.svdq_fp6_codes_bytes.restype = _I64
        L.svdq_pack_weight_fp6.argtypes = [_I64, _I64, _P, _P, _P]
        L.svdq_debug_gelu_bf16.argtypes = [_I64, _P, _P, _P]
        L.svdq_debug_stream_read.argtypes = [_P, _I64, _I32, _P, _P]
        L.svdq_smooth_factors.argtypes = [_I64, _I64, _I64, _P, _P, _P, _P]
        L.svdq_quantize_weight.argtypes = [_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P]
        L.svdq_lowrank_workspace_bytes.argtypes = [_I64, _I64, _I32]
        L.svdq_lowrank_workspace_bytes.restype = _I64
        L.svdq_lowrank_factors.argtypes = [_I64, _I64, _I32, _P, _P, ctypes.c_uint64, _P, _I64, _P, _P, _P]
        L.svdq_lowrank_factors_noalloc.argtypes = [_I64, _I64, _I32, _P, _P, ctypes.c_uint64, _P, _P, _P]
        for f in ("svdq_quantize_act", "svdq_gelu_quantize_act", "svdq_gemm_w4a4",
                  "svdq_gemm_w4a4_qk_norm_rope", "svdq_gemm_w4a4_gelu_quantize", "awq_gemv_w4a16",
                  "svdq_debug_group_sums", "svdq_debug_group_sums_packed", "svdq_pack_weight_int4",
                  "svdq_debug_group_sums_fp6", "svdq_pack_weight_fp6",
                  "svdq_debug_gelu_bf16", "svdq_debug_stream_read", "svdq_smooth_factors",
                  "svdq_quantize_weight", "svdq_lowrank_factors", "svdq_lowrank_factors_noalloc"):
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


_gpu = None


def _gpu_present() -> bool:
    global _gpu
    if _gpu is None:
        import torch
        _gpu = bool(torch.cuda.is_available())
    return _gpu


def _ptr(t):
    """Device pointer of a tensor handed to the library: it must be
    contiguous (the C ABI takes flat buffers) and, where a GPU is present,
    in device memory (a host pointer would reach the kernels)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("libsvdq takes contiguous tensors")
    if not t.is_cuda and _gpu_present():
        raise ValueError("libsvdq takes device tensors")
    return t.data_ptr()


def _need(t, nbytes, what, func):
    """Raise unless tensor t (if given) holds at least nbytes."""
    if t is not None and t.numel() * t.element_size() < nbytes:
        raise ValueError(f"{func}: {what} holds {t.numel() * t.element_size()} bytes, "
                         f"{int(nbytes)} are needed")


def _code_bytes(precision, rows, K, weight=False):
    """Bytes of a [rows, K] operand's codes in the given precision's layout."""
    if precision == SVDQ_INT4_FP6:
        return svdq_fp6_codes_bytes(rows, K)
    if precision == SVDQ_INT4_PACKED and weight:
        return svdq_packed_weight_bytes(rows, K)
    return rows * K // 2


def _scale_bytes(precision, rows, K):
    return rows * K // 16 if precision == SVDQ_NVFP4 else rows * (K // 64) * 2


def _check_layer_buffers(func, precision, M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales,
                         lora_act, lora_up, bias, out):
    _need(act_codes, _code_bytes(precision, M, K), "act_codes", func)
    _need(act_scales, _scale_bytes(precision, M, K), "act_scales", func)
    _need(wgt_codes, _code_bytes(precision, N, K, weight=True), "wgt_codes", func)
    _need(wgt_scales, _scale_bytes(precision, N, K), "wgt_scales", func)
    _need(lora_act, 4 * M * rank, "lora_act", func)
    _need(lora_up, 2 * N * rank, "lora_up", func)
    _need(bias, 2 * N, "bias", func)
    _need(out, 2 * M * N, "out", func)


def _stream(stream):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _check_act_buffers(func, precision, M, K, rank, smooth, lora_down, act_codes, act_scales, lora_act):
    _need(smooth, 2 * K, "smooth", func)
    _need(lora_down, 2 * rank * K, "lora_down", func)
    _need(act_codes, _code_bytes(precision, M, K), "act_codes", func)
    _need(act_scales, _scale_bytes(precision, M, K), "act_scales", func)
    _need(lora_act, 4 * M * rank, "lora_act", func)


def svdq_quantize_act(precision, x, smooth, lora_down, act_codes, act_scales, lora_act,
                      stream=None):
    """Smooth, low-rank down-projection and group quantization of x [M,K]."""
    M, K = x.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    _check_act_buffers("svdq_quantize_act", precision, M, K, rank, smooth, lora_down, act_codes, act_scales,
                       lora_act)
    _check(lib().svdq_quantize_act(precision, M, K, rank, _ptr(x), _ptr(smooth), _ptr(lora_down),
                                   _ptr(act_codes), _ptr(act_scales), _ptr(lora_act),
                                   _stream(stream)), "svdq_quantize_act")


def svdq_gelu_quantize_act(precision, x, smooth, lora_down, act_codes, act_scales, lora_act,
                           stream=None):
    """svdq_quantize_act of GELU(x) (tanh form), x being a GELU MLP's up-projection output."""
    M, K = x.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    _check_act_buffers("svdq_gelu_quantize_act", precision, M, K, rank, smooth, lora_down, act_codes,
                       act_scales, lora_act)
    _check(lib().svdq_gelu_quantize_act(precision, M, K, rank, _ptr(x), _ptr(smooth), _ptr(lora_down),
                                        _ptr(act_codes), _ptr(act_scales), _ptr(lora_act),
                                        _stream(stream)), "svdq_gelu_quantize_act")


def _weight_shape(precision, wgt_codes, wgt_scales):
    """(N, K) of a layer's weight: from the codes [N, K/2], or for a packed
    blob or an FP6-layout weight from the int4 scales [N, K/64]."""
    if precision in (SVDQ_INT4_PACKED, SVDQ_INT4_FP6):
        N, G = wgt_scales.shape
        return N, 64 * G
    N, Kh = wgt_codes.shape
    return N, 2 * Kh


def svdq_packed_weight_bytes(N, K) -> int:
    return int(lib().svdq_packed_weight_bytes(N, K))


def svdq_pack_weight_int4(wgt_codes, wgt_scales, packed_weight, invalid_codes=None, stream=None):
    """Offline re-encoding of int4 weight codes [N, K/2] (+ bf16 scales) into the
    packed blob of the SVDQ_INT4_PACKED GEMM; invalid_codes: optional int32 [1]."""
    N, Kh = wgt_codes.shape
    _check(lib().svdq_pack_weight_int4(N, 2 * Kh, _ptr(wgt_codes), _ptr(wgt_scales), _ptr(packed_weight),
                                       _ptr(invalid_codes), _stream(stream)), "svdq_pack_weight_int4")


def svdq_debug_group_sums_packed(act_codes, packed_weight, N, G, stream=None):
    """Exact int32 group sums [M,N,K/64] on the packed int4 GEMM's device path."""
    M, Kh = act_codes.shape
    _check(lib().svdq_debug_group_sums_packed(M, N, 2 * Kh, _ptr(act_codes), _ptr(packed_weight), _ptr(G),
                                              _stream(stream)), "svdq_debug_group_sums_packed")


def svdq_fp6_codes_bytes(rows, K) -> int:
    """Bytes of int4 codes of [rows, K] in the FP6 tiled layout (activations
    of the SVDQ_INT4_FP6 path, or its weight)."""
    return int(lib().svdq_fp6_codes_bytes(rows, K))


def svdq_pack_weight_fp6(wgt_codes, fp6_weight, stream=None):
    """Offline re-encoding of int4 weight codes [N, K/2] into the FP6 tiled
    layout (svdq_fp6_codes_bytes(N, K) bytes) of the SVDQ_INT4_FP6 GEMM."""
    N, Kh = wgt_codes.shape
    _check(lib().svdq_pack_weight_fp6(N, 2 * Kh, _ptr(wgt_codes), _ptr(fp6_weight), _stream(stream)),
           "svdq_pack_weight_fp6")


def svdq_debug_group_sums_fp6(act_codes, fp6_weight, M, N, K, G, stream=None):
    """Exact int32 group sums [M,N,K/64] on the FP6 GEMM's device path
    (both operands in the FP6 tiled layout)."""
    _check(lib().svdq_debug_group_sums_fp6(M, N, K, _ptr(act_codes), _ptr(fp6_weight), _ptr(G), _stream(stream)),
           "svdq_debug_group_sums_fp6")


def svdq_gemm_w4a4(precision, act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act,
                   lora_up, bias, out, stream=None):
    """4-bit GEMM with the low-rank up-projection and bias; out is [M,N] bf16
    (M from out: the FP6 layout is one-dimensional)."""
    M = out.shape[0]
    N, K = _weight_shape(precision, wgt_codes, wgt_scales)
    rank = 0 if lora_up is None else lora_up.shape[1]
    _check_layer_buffers("svdq_gemm_w4a4", precision, M, N, K, rank, act_codes, act_scales, wgt_codes,
                         wgt_scales, lora_act, lora_up, bias, out)
    _check(lib().svdq_gemm_w4a4(precision, M, N, K, rank, _ptr(act_codes), _ptr(act_scales),
                                _ptr(wgt_codes), _ptr(wgt_scales), float(alpha), _ptr(lora_act),
                                _ptr(lora_up), _ptr(bias), _ptr(out), _stream(stream)),
           "svdq_gemm_w4a4")


def svdq_gemm_w4a4_qk_norm_rope(precision, act_codes, act_scales, wgt_codes, wgt_scales, alpha,
                                lora_act, lora_up, bias, q_norm_weight, k_norm_weight, eps, rope_cos,
                                rope_sin, out, stream=None):
    """4-bit GEMM of a grouped QKV layer with per-head RMSNorm + rotary embedding
    of Q and K in the epilogue; out is [M, 3*H*128] bf16."""
    M = out.shape[0]
    N, K = _weight_shape(precision, wgt_codes, wgt_scales)
    rank = 0 if lora_up is None else lora_up.shape[1]
    _check_layer_buffers("svdq_gemm_w4a4_qk_norm_rope", precision, M, N, K, rank, act_codes, act_scales,
                         wgt_codes, wgt_scales, lora_act, lora_up, bias, out)
    _need(rope_cos, 4 * M * 64, "rope_cos", "svdq_gemm_w4a4_qk_norm_rope")
    _need(rope_sin, 4 * M * 64, "rope_sin", "svdq_gemm_w4a4_qk_norm_rope")
    _check(lib().svdq_gemm_w4a4_qk_norm_rope(precision, M, N, K, rank, _ptr(act_codes),
                                             _ptr(act_scales), _ptr(wgt_codes), _ptr(wgt_scales),
                                             float(alpha), _ptr(lora_act), _ptr(lora_up), _ptr(bias),
                                             _ptr(q_norm_weight), _ptr(k_norm_weight), float(eps),
                                             _ptr(rope_cos), _ptr(rope_sin), _ptr(out), _stream(stream)),
           "svdq_gemm_w4a4_qk_norm_rope")


def svdq_gelu_quantize_workspace_bytes(M, N, rank_next) -> int:
    """Workspace bytes of svdq_gemm_w4a4_gelu_quantize (-1 if the sizes are invalid)."""
    return int(lib().svdq_gelu_quantize_workspace_bytes(M, N, rank_next))


def svdq_gemm_w4a4_gelu_quantize(act_codes, act_scales, wgt_codes, wgt_scales, alpha, lora_act, lora_up,
                                 bias, smooth_next, lora_down_next, next_codes, next_scales, next_lora_act,
                                 workspace, out=None, stream=None):
    """Up projection of a GELU MLP (int4, FP6 layout) with the down layer's
    activation step in its epilogue: writes the down layer's FP6 codes,
    scales [M, N/64] and lora_act [M, rank_next] (M from next_scales), and
    the up layer's output into out [M, N] when given; workspace: a uint8
    device tensor of svdq_gelu_quantize_workspace_bytes(M, N, rank_next)
    bytes (None when that is 0, i.e. rank_next == 0)."""
    func = "svdq_gemm_w4a4_gelu_quantize"
    prec = SVDQ_INT4_FP6
    M = next_scales.shape[0]
    N, K = _weight_shape(prec, wgt_codes, wgt_scales)
    rank = 0 if lora_up is None else lora_up.shape[1]
    rank_next = 0 if lora_down_next is None else lora_down_next.shape[0]
    _check_layer_buffers(func, prec, M, N, K, rank, act_codes, act_scales, wgt_codes, wgt_scales, lora_act,
                         lora_up, bias, out)
    _check_act_buffers(func, prec, M, N, rank_next, smooth_next, lora_down_next, next_codes, next_scales,
                       next_lora_act)
    _check(lib().svdq_gemm_w4a4_gelu_quantize(prec, M, N, K, rank, _ptr(act_codes), _ptr(act_scales),
                                              _ptr(wgt_codes), _ptr(wgt_scales), float(alpha), _ptr(lora_act),
                                              _ptr(lora_up), _ptr(bias), rank_next, _ptr(smooth_next),
                                              _ptr(lora_down_next), _ptr(next_codes), _ptr(next_scales),
                                              _ptr(next_lora_act), _ptr(workspace),
                                              0 if workspace is None else workspace.numel() * workspace.element_size(),
                                              _ptr(out), _stream(stream)), func)


def awq_gemv_w4a16(x, wgt_codes, wgt_scales, wgt_zeros, bias, out, group_size=64, stream=None):
    """int4 weight-only layer: out[M,N] = x . dequant(W)^T + bias."""
    M, K = x.shape
    N = wgt_codes.shape[0]
    if group_size == 64:
        for t, nb, what in ((wgt_codes, N * K // 2, "wgt_codes"), (wgt_scales, 2 * N * (K // 64), "wgt_scales"),
                            (wgt_zeros, 2 * N * (K // 64), "wgt_zeros"), (bias, 2 * N, "bias"),
                            (out, 2 * M * N, "out")):
            _need(t, nb, what, "awq_gemv_w4a16")
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


def svdq_lowrank_factors_noalloc(W, smooth, rank, seed, lora_up, lora_down, stream=None):
    """svdq_lowrank_factors on the library's fixed per-device scratch (no workspace, no allocation)."""
    N, K = W.shape
    _check(lib().svdq_lowrank_factors_noalloc(N, K, rank, _ptr(W), _ptr(smooth), int(seed), _ptr(lora_up),
                                              _ptr(lora_down), _stream(stream)),
           "svdq_lowrank_factors_noalloc")


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


STREAM_READ_SPAN = 12288


def svdq_debug_stream_read(src, out, pattern=0, nbytes=None, stream=None):
    """Plain read of a device tensor (pattern 0 contiguous, 1 the AWQ GEMV's
    row pattern); out (int32, at least ceil(nbytes / 12288) entries) receives
    the xor of each 12288-byte span's 16-byte chunks."""
    n = src.numel() * src.element_size() if nbytes is None else int(nbytes)
    if out.numel() * out.element_size() < 4 * ((n + STREAM_READ_SPAN - 1) // STREAM_READ_SPAN):
        raise ValueError("svdq_debug_stream_read: out holds fewer than ceil(nbytes / 12288) words")
    _check(lib().svdq_debug_stream_read(_ptr(src), n, int(pattern), _ptr(out), _stream(stream)),
           "svdq_debug_stream_read")
