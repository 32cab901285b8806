"""Python face of the CPU oracle.

TEST INFRASTRUCTURE ONLY: the product package never imports this module.
Only the tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` use it.

The arithmetic lives in ``svdq_oracle.c`` (plain C, fp64 where the method is
exact, one IEEE rounding per fp32 step).  This module only marshals numpy
arrays and adds the one offline step that is a library primitive: the
truncated SVD that yields the 16-bit low-rank branch ("the hardest part of
each weight matrix is kept in a small 16-bit low-rank branch" -- blog
"Hugging Face integrates Nunchaku 4-bit diffusion inference into Diffusers",
section "SVDQuant and the Nunchaku engine").

bf16 tensors are numpy ``uint16`` bit patterns; E4M3 scales and packed
nibbles are ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "svdq_oracle.c")
_LIB_PATH = os.path.join(_HERE, "_build", "liboracle.so")

INT4 = 0
NVFP4 = 1

GCC_FLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off",
             "-fno-fast-math", "-shared", "-fPIC"]


def build(force: bool = True) -> str:
    """Compile the oracle with gcc into ``oracle/_build/liboracle.so``."""
    if force or not os.path.exists(_LIB_PATH):
        os.makedirs(os.path.dirname(_LIB_PATH), exist_ok=True)
        tmp = _LIB_PATH + ".tmp"
        subprocess.run(["gcc", *GCC_FLAGS, "-o", tmp, _SRC, "-lm"], check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F32 = ctypes.c_float

_SIGS = {
    "oracle_bf16_to_f32": ([ctypes.c_uint16], ctypes.c_float),
    "oracle_f32_to_bf16": ([ctypes.c_float], ctypes.c_uint16),
    "oracle_f64_to_bf16": ([ctypes.c_double], ctypes.c_uint16),
    "oracle_e4m3_to_f32": ([ctypes.c_uint8], ctypes.c_float),
    "oracle_f32_to_e4m3": ([ctypes.c_float], ctypes.c_uint8),
    "oracle_e2m1_to_f32": ([ctypes.c_uint8], ctypes.c_float),
    "oracle_f32_to_e2m1": ([ctypes.c_float], ctypes.c_uint8),
    "oracle_bf16_to_f32_array": ([_I64, _P, _P], None),
    "oracle_f32_to_bf16_array": ([_I64, _P, _P], None),
    "oracle_f64_to_bf16_array": ([_I64, _P, _P], None),
    "oracle_e4m3_to_f32_array": ([_I64, _P, _P], None),
    "oracle_f32_to_e4m3_array": ([_I64, _P, _P], None),
    "oracle_e2m1_to_f32_array": ([_I64, _P, _P], None),
    "oracle_f32_to_e2m1_array": ([_I64, _P, _P], None),
    "oracle_unpack_int4": ([_I64, _I64, _P, _P], None),
    "oracle_unpack_u4": ([_I64, _I64, _P, _P], None),
    "oracle_smooth_factors": ([_I64, _I64, _I64, _P, _P, _P], None),
    "oracle_svdq_residual": ([_I64, _I64, _I32, _P, _P, _P, _P, _P], None),
    "oracle_quantize_int4": ([_I64, _I64, _P, _P, _P], None),
    "oracle_quantize_nvfp4": ([_I64, _I64, _P, _P, _P], None),
    "oracle_smooth_act": ([_I64, _I64, _P, _P, _P], None),
    "oracle_lowrank_down": ([_I64, _I64, _I32, _P, _P, _P], None),
    "oracle_svdq_quantize_act": ([_I32, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P, _P, _P], None),
    "oracle_group_sums_int4": ([_I64, _I64, _I64, _P, _P, _P], None),
    "oracle_svdq_gemm_w4a4": ([_I32, _I64, _I64, _I64, _I32, _P, _P, _P, _P, _F32, _P, _P, _P, _P],
                              None),
    "oracle_awq_quantize_weight": ([_I64, _I64, _P, _P, _P, _P], None),
    "oracle_awq_gemv_w4a16": ([_I64, _I64, _I64, _I32, _P, _P, _P, _P, _P, _P], None),
    "oracle_gelu_tanh_bf16": ([ctypes.c_uint16], ctypes.c_uint16),
    "oracle_gelu_tanh_bf16_array": ([_I64, _P, _P], None),
    "oracle_qk_norm_rope": ([_I64, _I64, _P, _P, _P, ctypes.c_double, _P, _P, _P], None),
}


def lib():
    """Load (building on first use) the oracle shared library."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=False)
        L = ctypes.CDLL(_LIB_PATH)
        for name, (args, res) in _SIGS.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    """Contiguous array of ``dtype``.  Integer storage (bf16 / E4M3 bit
    patterns, packed nibbles) is never produced by casting floating-point
    values: that would silently turn, e.g., weights of magnitude 0.02 into
    the bf16 pattern 0x0000."""
    src = np.asarray(a)
    if np.issubdtype(np.dtype(dtype), np.integer) and np.issubdtype(src.dtype, np.floating):
        raise TypeError(f"oracle: float array ({src.dtype}) where {np.dtype(dtype)} bit patterns "
                        "are expected; convert the values first (e.g. to bf16 bits)")
    return np.ascontiguousarray(src, dtype=dtype)


# --------------------------------------------------------------------------
# codecs
# --------------------------------------------------------------------------

def bf16_to_f32(h):
    h = _c(h, np.uint16)
    out = np.empty(h.shape, np.float32)
    lib().oracle_bf16_to_f32_array(h.size, _ptr(h), _ptr(out))
    return out


def f32_to_bf16(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f32_to_bf16_array(v.size, _ptr(v), _ptr(out))
    return out


def f64_to_bf16(v):
    v = _c(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().oracle_f64_to_bf16_array(v.size, _ptr(v), _ptr(out))
    return out


def e4m3_to_f32(b):
    b = _c(b, np.uint8)
    out = np.empty(b.shape, np.float32)
    lib().oracle_e4m3_to_f32_array(b.size, _ptr(b), _ptr(out))
    return out


def f32_to_e4m3(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_f32_to_e4m3_array(v.size, _ptr(v), _ptr(out))
    return out


def e2m1_to_f32(c):
    c = _c(c, np.uint8)
    out = np.empty(c.shape, np.float32)
    lib().oracle_e2m1_to_f32_array(c.size, _ptr(c), _ptr(out))
    return out


def f32_to_e2m1(v):
    v = _c(v, np.float32)
    out = np.empty(v.shape, np.uint8)
    lib().oracle_f32_to_e2m1_array(v.size, _ptr(v), _ptr(out))
    return out


def unpack_int4(codes, rows, K):
    """Packed two's-complement nibbles [rows, K/2] -> int8 [rows, K]."""
    codes = _c(codes, np.uint8)
    out = np.empty((rows, K), np.int8)
    lib().oracle_unpack_int4(rows, K, _ptr(codes), _ptr(out))
    return out


def unpack_u4(codes, rows, K):
    """Packed unsigned nibbles [rows, K/2] -> uint8 [rows, K]."""
    codes = _c(codes, np.uint8)
    out = np.empty((rows, K), np.uint8)
    lib().oracle_unpack_u4(rows, K, _ptr(codes), _ptr(out))
    return out


# --------------------------------------------------------------------------
# quantizers and runtime steps
# --------------------------------------------------------------------------

def quantize_int4(v):
    """int4 group-64 quantizer on fp32 rows -> (codes u8 [R,K/2], scales bf16 [R,K/64])."""
    v = _c(v, np.float32)
    R, K = v.shape
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.empty((R, K // 64), np.uint16)
    lib().oracle_quantize_int4(R, K, _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def quantize_nvfp4(v):
    """NVFP4 group-16 quantizer on fp32 rows -> (codes u8 [R,K/2], E4M3 scales u8 [R,K/16])."""
    v = _c(v, np.float32)
    R, K = v.shape
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.empty((R, K // 16), np.uint8)
    lib().oracle_quantize_nvfp4(R, K, _ptr(v), _ptr(codes), _ptr(scales))
    return codes, scales


def smooth_act(x, smooth):
    x = _c(x, np.uint16)
    M, K = x.shape
    out = np.empty((M, K), np.uint16)
    lib().oracle_smooth_act(M, K, _ptr(x), _ptr(None if smooth is None else _c(smooth, np.uint16)),
                            _ptr(out))
    return out


def lowrank_down(xhat, lora_down):
    xhat = _c(xhat, np.uint16)
    lora_down = _c(lora_down, np.uint16)
    M, K = xhat.shape
    r = lora_down.shape[0]
    t = np.empty((M, r), np.float32)
    lib().oracle_lowrank_down(M, K, r, _ptr(xhat), _ptr(lora_down), _ptr(t))
    return t


def quantize_act(precision, x, smooth, lora_down):
    """The activation step: smooth, low-rank down-projection, group quantize.

    Returns (act_codes u8 [M,K/2], act_scales, lora_act f32 [M,rank])."""
    x = _c(x, np.uint16)
    M, K = x.shape
    rank = 0 if lora_down is None else lora_down.shape[0]
    codes = np.zeros((M, K // 2), np.uint8)
    if precision == INT4:
        scales = np.empty((M, K // 64), np.uint16)
    else:
        scales = np.empty((M, K // 16), np.uint8)
    t = np.empty((M, max(rank, 1)), np.float32)
    xhat = np.empty((M, K), np.uint16)
    vals = np.empty((M, K), np.float32)
    sm = None if smooth is None else _c(smooth, np.uint16)
    ld = None if lora_down is None else _c(lora_down, np.uint16)
    lib().oracle_svdq_quantize_act(precision, M, K, rank, _ptr(x), _ptr(sm), _ptr(ld),
                                   _ptr(codes), _ptr(scales), _ptr(t), _ptr(xhat), _ptr(vals))
    return codes, scales, t[:, :rank].copy()


def gelu_tanh_bf16(x):
    """GELU (tanh form) of bf16 values, rounded once to bf16.  x: uint16 bits."""
    x = _c(x, np.uint16)
    out = np.empty(x.shape, np.uint16)
    lib().oracle_gelu_tanh_bf16_array(x.size, _ptr(x), _ptr(out))
    return out


def gelu_quantize_act(precision, x, smooth, lora_down):
    """The activation step of a layer that consumes GELU(x): x is the
    preceding layer's bf16 output; GELU is applied before the smoothing.
    Returns what ``quantize_act`` returns for gelu_tanh_bf16(x)."""
    return quantize_act(precision, gelu_tanh_bf16(x), smooth, lora_down)


def qk_norm_rope(y, q_w, k_w, eps, rope_cos, rope_sin):
    """Per-head RMSNorm + rotary embedding of the Q and K columns of a grouped
    QKV output y (bf16 [M, 3*H*128]); V columns unchanged.  q_w, k_w: bf16
    [128]; rope_cos, rope_sin: fp32 [M, 64].  Returns bf16 [M, N]."""
    y = _c(y, np.uint16)
    M, N = y.shape
    assert N % 384 == 0
    out = np.empty((M, N), np.uint16)
    lib().oracle_qk_norm_rope(M, N, _ptr(y), _ptr(_c(q_w, np.uint16)), _ptr(_c(k_w, np.uint16)),
                              float(eps), _ptr(_c(rope_cos, np.float32)), _ptr(_c(rope_sin, np.float32)),
                              _ptr(out))
    return out


def gemm_w4a4_qk_norm_rope(precision, act_codes, act_scales, wgt_codes, wgt_scales, lora_act,
                           lora_up, bias, q_w, k_w, eps, rope_cos, rope_sin, alpha=1.0, rows=None):
    """The grouped QKV layer's GEMM step followed by per-head RMSNorm and
    rotary embedding of Q and K (``qk_norm_rope`` of the ``gemm_w4a4`` output);
    ``rows`` as in ``gemm_w4a4`` (the angles of those rows are used)."""
    y = gemm_w4a4(precision, act_codes, act_scales, wgt_codes, wgt_scales, lora_act, lora_up, bias,
                  alpha=alpha, rows=rows)
    if rows is not None:
        rope_cos, rope_sin = np.asarray(rope_cos)[rows], np.asarray(rope_sin)[rows]
    return qk_norm_rope(y, q_w, k_w, eps, rope_cos, rope_sin)


def group_sums_int4(act_codes, wgt_codes, K):
    act_codes = _c(act_codes, np.uint8)
    wgt_codes = _c(wgt_codes, np.uint8)
    M = act_codes.shape[0]
    N = wgt_codes.shape[0]
    G = np.empty((M, N, K // 64), np.int32)
    lib().oracle_group_sums_int4(M, N, K, _ptr(act_codes), _ptr(wgt_codes), _ptr(G))
    return G


def gemm_w4a4(precision, act_codes, act_scales, wgt_codes, wgt_scales, lora_act, lora_up,
              bias=None, alpha=1.0, rows=None):
    """The 4-bit GEMM step with the fused low-rank up-projection and bias.

    ``rows`` (optional index array) restricts the computation to those output
    rows; the result then has ``len(rows)`` rows in that order."""
    wgt_codes = _c(wgt_codes, np.uint8)
    N, Kh = wgt_codes.shape
    K = 2 * Kh
    if rows is not None:
        rows = np.asarray(rows, np.int64)
        act_codes = act_codes[rows]
        act_scales = act_scales[rows]
        lora_act = None if lora_act is None else lora_act[rows]
    act_codes = _c(act_codes, np.uint8)
    M = act_codes.shape[0]
    if precision == INT4:
        act_scales = _c(act_scales, np.uint16)
        wgt_scales = _c(wgt_scales, np.uint16)
    else:
        act_scales = _c(act_scales, np.uint8)
        wgt_scales = _c(wgt_scales, np.uint8)
    rank = 0 if lora_up is None else lora_up.shape[1]
    la = None if rank == 0 else _c(lora_act, np.float32)
    lu = None if rank == 0 else _c(lora_up, np.uint16)
    b = None if bias is None else _c(bias, np.uint16)
    out = np.empty((M, N), np.uint16)
    lib().oracle_svdq_gemm_w4a4(precision, M, N, K, rank, _ptr(act_codes), _ptr(act_scales),
                                _ptr(wgt_codes), _ptr(wgt_scales), float(alpha), _ptr(la),
                                _ptr(lu), _ptr(b), _ptr(out))
    return out


def awq_quantize_weight(W):
    W = _c(W, np.uint16)
    N, K = W.shape
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.empty((N, K // 64), np.uint16)
    zeros = np.empty((N, K // 64), np.uint16)
    lib().oracle_awq_quantize_weight(N, K, _ptr(W), _ptr(codes), _ptr(scales), _ptr(zeros))
    return codes, scales, zeros


def awq_gemv(x, codes, scales, zeros, bias=None, group_size=64):
    x = _c(x, np.uint16)
    codes = _c(codes, np.uint8)
    M, K = x.shape
    N = codes.shape[0]
    out = np.empty((M, N), np.uint16)
    b = None if bias is None else _c(bias, np.uint16)
    lib().oracle_awq_gemv_w4a16(M, N, K, group_size, _ptr(x), _ptr(codes),
                                _ptr(_c(scales, np.uint16)), _ptr(_c(zeros, np.uint16)),
                                _ptr(b), _ptr(out))
    return out


# --------------------------------------------------------------------------
# offline weight preparation (SVDQuant: smoothing, low rank, 4-bit residual)
# --------------------------------------------------------------------------

def smooth_factors(x, W):
    """s[k] = RNE_bf16(sqrt(max|x[:,k]| / max|W[:,k]|)) (1 where either is 0)."""
    x = _c(x, np.uint16)
    W = _c(W, np.uint16)
    M, K = x.shape
    N = W.shape[0]
    s = np.empty((K,), np.uint16)
    lib().oracle_smooth_factors(M, N, K, _ptr(x), _ptr(W), _ptr(s))
    return s


def top_singular_triplets(A, r):
    """Leading r singular triplets of a fp64 matrix, largest first.

    Signs are made canonical: each left vector's largest-magnitude entry
    (first one on ties) is positive.  A library SVD is the primitive."""
    A = np.asarray(A, np.float64)
    if min(A.shape) <= 1024:
        U, S, VT = np.linalg.svd(A, full_matrices=False)
        U, S, VT = U[:, :r], S[:r], VT[:r]
    else:
        from scipy.sparse.linalg import svds
        v0 = np.ones(min(A.shape), np.float64) / np.sqrt(min(A.shape))
        U, S, VT = svds(A, k=r, tol=0, v0=v0)
        order = np.argsort(S)[::-1]
        U, S, VT = U[:, order], S[order], VT[order]
    for j in range(r):
        i = int(np.argmax(np.abs(U[:, j])))
        if U[i, j] < 0:
            U[:, j] = -U[:, j]
            VT[j] = -VT[j]
    return U, S, VT


def lowrank_factors(W_hat, r):
    """16-bit low-rank branch of the smoothed weight W_hat [N,K] (fp64).

    lora_up[n,j] = RNE_bf16(U[n,j]); lora_down[j,k] = RNE_bf16(sigma_j V[k,j]).
    The pages do not say how the singular values are split between the two
    factors; they are kept on the down factor."""
    U, S, VT = top_singular_triplets(W_hat, r)
    lora_up = f64_to_bf16(U)
    lora_down = f64_to_bf16(S[:, None] * VT)
    return lora_up, lora_down


def svdq_residual(W, smooth, lora_up, lora_down):
    """R = W*s - up.down in fp64, rounded once to fp32.  W bf16 [N,K]."""
    W = _c(W, np.uint16)
    N, K = W.shape
    r = 0 if lora_up is None else lora_up.shape[1]
    R = np.empty((N, K), np.float32)
    lib().oracle_svdq_residual(N, K, r, _ptr(W), _ptr(_c(smooth, np.uint16)),
                               _ptr(None if r == 0 else _c(lora_up, np.uint16)),
                               _ptr(None if r == 0 else _c(lora_down, np.uint16)), _ptr(R))
    return R


def prepare_svdq_weight(precision, x_calib, W, rank, smooth=True):
    """Offline SVDQuant preparation of one linear layer's weight.

    1. smoothing factors from the calibration activations (outliers migrate
       into the weight), 2. the rank-r 16-bit branch of the smoothed weight,
    3. 4-bit quantization of the residual.  ``smooth=False`` uses s = 1 and
    ``rank=0`` drops the branch (the ablations of the property tests).

    Returns a dict with smooth, lora_up, lora_down, wgt_codes, wgt_scales."""
    W = _c(W, np.uint16)
    N, K = W.shape
    s = smooth_factors(x_calib, W) if smooth else np.full((K,), 0x3F80, np.uint16)
    W_hat = bf16_to_f32(W).astype(np.float64) * bf16_to_f32(s).astype(np.float64)[None, :]
    if rank > 0:
        lora_up, lora_down = lowrank_factors(W_hat, rank)
    else:
        lora_up, lora_down = None, None
    R = svdq_residual(W, s, lora_up, lora_down)
    if precision == INT4:
        codes, scales = quantize_int4(R)
    else:
        codes, scales = quantize_nvfp4(R)
    return {"smooth": s, "lora_up": lora_up, "lora_down": lora_down,
            "wgt_codes": codes, "wgt_scales": scales, "residual": R}
