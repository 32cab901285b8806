"""Helpers for the GPU parity tests: host<->device transfer of bf16 bit
patterns, case builders (seeded inputs + the oracle's offline weight
preparation), and the comparison rules.

Pass bar (codes, scales and integer group sums bit-exact; bf16 outputs
within 1e-2 relative Frobenius error and within 2 bf16 ulp for at least
99.9% of elements) is the one stated for this layer; lora_act, an fp32
intermediate summed in a different order on each side, is held to 1e-5
relative Frobenius error."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
from bit_w4a4_quantized_svdq_amd import synth

DEV = "cuda"


def announce(*parts):
    """Name the case on stderr before a GPU step (bypasses pytest capture)."""
    sys.__stderr__.write("[gpu case] " + " ".join(str(p) for p in parts) + "\n")
    sys.__stderr__.flush()


def to_dev(a, kind):
    """numpy -> device tensor.  kind: 'bf16' (uint16 bits), 'u8', 'f32', 'i32'."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if kind == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(a).to(DEV)


GUARD_BYTES = 256     # poisoned canary bytes on each side of every output buffer


def check_guards(t):
    """The canaries around a buffer from empty() are intact: no kernel wrote
    before its start or past its end."""
    guard = getattr(t, "_svdq_guard", None)
    if guard is None:
        return
    flat, g, n = guard
    head = flat[:g].view(torch.uint8)
    tail = flat[g + n:].view(torch.uint8)
    bad_head = int((head != 0xFF).sum())
    bad_tail = int((tail != 0xFF).sum())
    assert bad_head == 0 and bad_tail == 0, \
        f"out-of-bounds write: {bad_head} canary bytes before and {bad_tail} after a {tuple(t.shape)} buffer"


def to_host(t, kind):
    check_guards(t)
    t = t.detach().cpu().contiguous()
    if kind == "bf16":
        return t.view(torch.int16).numpy().view(np.uint16).copy()
    return t.numpy().copy()


def empty(shape, kind):
    """A device buffer with GUARD_BYTES of 0xFF canaries before and after it
    (the buffer itself keeps 256-byte alignment); to_host() checks them."""
    dt = {"bf16": torch.bfloat16, "u8": torch.uint8, "f32": torch.float32, "i32": torch.int32}[kind]
    item = torch.empty((), dtype=dt).element_size()
    g = GUARD_BYTES // item
    n = int(np.prod(shape))
    flat = torch.empty(n + 2 * g, dtype=dt, device=DEV)
    flat.view(torch.uint8).fill_(0xFF)
    t = flat[g:g + n].view(shape)
    t._svdq_guard = (flat, g, n)
    return t


def poison(t):
    """Fill an output buffer with a NaN/0xFF pattern so unwritten elements show."""
    t.view(torch.uint8).fill_(0xFF)
    return t


def ulp_dist(a, b):
    def ordv(h):
        h = np.asarray(h, np.int64)
        return np.where(h & 0x8000, -(h & 0x7FFF), h)
    return np.abs(ordv(a) - ordv(b))


def bf16_f64(h):
    return synth.bf16_bits_to_f32(h).astype(np.float64)


def assert_bf16_close(got, ref, what=""):
    """The output bar: rel. Frobenius <= 1e-2 and <= 2 ulp for >= 99.9%."""
    assert got.shape == ref.shape, (got.shape, ref.shape)
    g, r = bf16_f64(got), bf16_f64(ref)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    d = ulp_dist(got, ref)
    frob = np.linalg.norm(g - r) / max(np.linalg.norm(r), 1e-300)
    within = (d <= 2).mean()
    assert frob <= 1e-2 and within >= 0.999, \
        f"{what}: rel_frob={frob:.3e} within2ulp={within:.5f} max_ulp={d.max()}"
    return {"rel_frob": frob, "within_2ulp": within, "max_ulp": int(d.max())}


def assert_f32_close(got, ref, tol=1e-5, what=""):
    frob = np.linalg.norm(got.astype(np.float64) - ref) / max(np.linalg.norm(ref), 1e-300)
    assert frob <= tol, f"{what}: rel_frob={frob:.3e}"


def svdq_case(cfg: synth.LinearConfig, with_bias=False, M=None, x=None):
    """Seeded layer of a config, prepared offline by the oracle."""
    prec = oracle.INT4 if cfg.precision == "int4" else oracle.NVFP4
    case = synth.linear_case(cfg, M=M, with_bias=with_bias)
    if x is not None:
        case["x"] = x
    prep = oracle.prepare_svdq_weight(prec, case["x"], case["W"], cfg.rank)
    case.update(prep)
    case["prec"] = prec
    return case


def gpu_quantize(prec, x, smooth, lora_down, K, gelu=False):
    """The activation step on the GPU.  prec 3 (SVDQ_INT4_FP6): int4 codes in
    the FP6 layout [M, 3K/4] with int4's bf16 scales."""
    from bit_w4a4_quantized_svdq_amd import capi
    M = x.shape[0]
    rank = 0 if lora_down is None else lora_down.shape[0]
    int4 = prec in (0, 3)
    codes = poison(empty((capi.svdq_fp6_codes_bytes(M, K),) if prec == 3 else (M, K // 2), "u8"))
    scales = poison(empty((M, K // 64), "bf16") if int4 else empty((M, K // 16), "u8"))
    lact = poison(empty((M, rank), "f32")) if rank else None
    fn = capi.svdq_gelu_quantize_act if gelu else capi.svdq_quantize_act
    fn(prec, to_dev(x, "bf16"), to_dev(smooth, "bf16"), to_dev(lora_down, "bf16"), codes, scales, lact)
    torch.cuda.synchronize()
    return (to_host(codes, "u8"), to_host(scales, "bf16" if int4 else "u8"),
            None if lact is None else to_host(lact, "f32"))


def gpu_pack_weight_fp6(wgt_codes_dev):
    """The FP6 tiled layout of device int4 codes (svdq_pack_weight_fp6), in a
    poisoned buffer: padding the packer must not write stays 0xFF."""
    from bit_w4a4_quantized_svdq_amd import capi
    N, Kh = wgt_codes_dev.shape
    out = poison(empty((capi.svdq_fp6_codes_bytes(N, 2 * Kh),), "u8"))
    capi.svdq_pack_weight_fp6(wgt_codes_dev, out)
    return out


def gpu_pack_weight(wgt_codes_dev, wgt_scales_dev):
    """The packed int4 weight blob (svdq_pack_weight_int4) of device codes and
    scales; asserts that no -8 code was met."""
    from bit_w4a4_quantized_svdq_amd import capi
    N, Kh = wgt_codes_dev.shape
    blob = poison(empty((capi.svdq_packed_weight_bytes(N, 2 * Kh),), "u8"))
    bad = poison(empty((1,), "i32"))
    capi.svdq_pack_weight_int4(wgt_codes_dev, wgt_scales_dev, blob, bad)
    torch.cuda.synchronize()
    assert int(to_host(bad, "i32")[0]) == 0, "weight codes of -8 cannot be packed"
    return blob


def gpu_gemm(prec, act_codes, act_scales, wgt_codes, wgt_scales, lora_act, lora_up, bias, alpha=1.0,
             zero_weight_ok=False, packed=False, fp6=False, act_fp6=None):
    """The W4A4 GEMM on the GPU (act_codes and wgt_codes: packed nibbles).
    int4 only: packed -- through the packed weight blob and the
    SVDQ_INT4_PACKED path; fp6 -- the SVDQ_INT4_FP6 path, the activation
    codes put in the FP6 layout on the host (tests/fp6_layout.py), the
    weight by svdq_pack_weight_fp6; act_fp6 (optional, with fp6): activation
    codes already in the FP6 layout (e.g. the GPU activation step's)."""
    from bit_w4a4_quantized_svdq_amd import capi
    M, N = act_codes.shape[0], wgt_codes.shape[0]
    # a layer whose weight scales are all zero tests only the bias and low-rank
    # terms; only a test that means to (the zero-residual invariant) may pass one
    assert zero_weight_ok or N == 0 or np.any(wgt_scales != 0), "degenerate layer: all weight scales zero"
    out = poison(empty((M, N), "bf16"))
    skind = "bf16" if prec == 0 else "u8"
    wc, ws = to_dev(wgt_codes, "u8"), to_dev(wgt_scales, skind)
    if packed:
        assert prec == 0
        wc, prec = gpu_pack_weight(wc, ws), capi.SVDQ_INT4_PACKED
    if fp6:
        from tests.fp6_layout import fp6_layout_from_nibbles
        assert prec == 0
        K = 2 * act_codes.shape[1]
        if act_fp6 is not None:
            act_codes = act_fp6
        else:
            act_codes = fp6_layout_from_nibbles(act_codes, K)
        wc, prec = gpu_pack_weight_fp6(wc), capi.SVDQ_INT4_FP6
    capi.svdq_gemm_w4a4(prec, to_dev(act_codes, "u8"), to_dev(act_scales, skind), wc, ws, alpha,
                        to_dev(lora_act, "f32"), to_dev(lora_up, "bf16"), to_dev(bias, "bf16"), out)
    torch.cuda.synchronize()
    return to_host(out, "bf16")


def gpu_gemv(x, codes, scales, zeros, bias):
    """scales, zeros [N, K/64], the oracle's and the library's layout."""
    from bit_w4a4_quantized_svdq_amd import capi
    M, N = x.shape[0], codes.shape[0]
    assert N == 0 or np.any(scales != 0), "degenerate AWQ layer: all scales zero"
    out = poison(empty((M, N), "bf16"))
    capi.awq_gemv_w4a16(to_dev(x, "bf16"), to_dev(codes, "u8"), to_dev(scales, "bf16"),
                        to_dev(zeros, "bf16"), to_dev(bias, "bf16"), out)
    torch.cuda.synchronize()
    return to_host(out, "bf16")
