"""C ABI checks that need no GPU: libsvdq.so loads, exports every function
declared in include/svdq.h, and rejects bad arguments on the host before any
HIP call (so these run on a CPU-only machine)."""
import ctypes
import os
import re

import pytest

from bit_w4a4_quantized_svdq_amd import capi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "svdq.h")

pytestmark = pytest.mark.skipif(not os.path.exists(capi.LIB_PATH),
                                reason="libsvdq.so not built (python -m bit_w4a4_quantized_svdq_amd.build)")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*([a-z_0-9]+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for f in ("svdq_quantize_act", "svdq_gemm_w4a4", "awq_gemv_w4a16"):
        assert f in names
    assert set(names) == set(capi.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(capi.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name
    assert capi.svdq_abi_version() == 11
    for s in range(4):
        assert capi.svdq_status_string(s).startswith(("SVDQ_OK", "SVDQ_ERR"))
    assert "unknown" in capi.svdq_status_string(99)


A = 1 << 20          # a 16-byte aligned fake device address (never dereferenced)
MIS = A + 2          # misaligned


def qa(prec=0, M=4, K=64, rank=16, x=A, smooth=A, down=A, codes=A, scales=A, lact=A):
    return capi.lib().svdq_quantize_act(prec, M, K, rank, x, smooth, down, codes, scales, lact, None)


def gm(prec=0, M=4, N=64, K=64, rank=16, ac=A, asc=A, wc=A, wsc=A, lact=A, up=A, bias=A, out=A):
    return capi.lib().svdq_gemm_w4a4(prec, M, N, K, rank, ac, asc, wc, wsc, 1.0, lact, up, bias, out,
                                     None)


def gv(M=1, N=64, K=64, gs=64, x=A, c=A, s=A, z=A, bias=A, out=A):
    return capi.lib().awq_gemv_w4a16(M, N, K, gs, x, c, s, z, bias, out, None)


INV, UNS = capi.SVDQ_ERR_INVALID_ARG, capi.SVDQ_ERR_UNSUPPORTED


@pytest.mark.parametrize("kw,want,msg", [
    (dict(prec=2), UNS, "precision"), (dict(prec=4), UNS, "precision"),
    (dict(K=0), INV, "K must"), (dict(K=96), INV, "K must"), (dict(K=1 << 17), INV, "K must"),
    (dict(M=-1), INV, "M and N"), (dict(M=(1 << 24) + 1), INV, "M and N"),
    (dict(rank=8), INV, "rank"), (dict(rank=144), INV, "rank"), (dict(rank=-16), INV, "rank"),
    (dict(x=None), INV, "x must not"), (dict(codes=None), INV, "act_codes"),
    (dict(scales=None), INV, "act_scales"), (dict(down=None), INV, "lora_down"),
    (dict(lact=None), INV, "lora_act"), (dict(x=MIS), INV, "aligned"),
    (dict(smooth=MIS), INV, "smooth"),
])
def test_quantize_act_rejects(kw, want, msg):
    assert qa(**kw) == want
    assert msg in capi.svdq_last_error()


def test_quantize_act_optional_pointers_and_empty():
    # rank 0: lora pointers may be NULL; M = 0 is a no-op that succeeds
    assert qa(M=0, rank=0, down=None, lact=None, smooth=None) == capi.SVDQ_OK


@pytest.mark.parametrize("kw,want,msg", [
    (dict(prec=-1), UNS, "precision"), (dict(N=-5), INV, "M and N"), (dict(K=32), INV, "K must"),
    (dict(rank=20), INV, "rank"), (dict(ac=None), INV, "act_codes"), (dict(wc=None), INV, "wgt_codes"),
    (dict(wsc=None), INV, "wgt_scales"), (dict(up=None), INV, "lora_up"), (dict(out=None), INV, "out"),
    (dict(bias=MIS), INV, "bias"), (dict(wc=MIS), INV, "wgt_codes"),
])
def test_gemm_rejects(kw, want, msg):
    assert gm(**kw) == want
    assert msg in capi.svdq_last_error()


def test_gemm_empty_is_noop():
    assert gm(M=0) == capi.SVDQ_OK
    assert gm(N=0, rank=0, lact=None, up=None, bias=None) == capi.SVDQ_OK


@pytest.mark.parametrize("kw,want,msg", [
    (dict(gs=128), UNS, "group_size"), (dict(gs=16), UNS, "group_size"), (dict(K=100), INV, "K must"),
    (dict(x=None), INV, "x must not"), (dict(z=None), INV, "wgt_zeros"), (dict(s=MIS), INV, "wgt_scales"),
])
def test_gemv_rejects(kw, want, msg):
    assert gv(**kw) == want
    assert msg in capi.svdq_last_error()


def test_gemv_empty_is_noop():
    assert gv(M=0, bias=None) == capi.SVDQ_OK


def test_group_sums_rejects():
    L = capi.lib()
    assert L.svdq_debug_group_sums(4, 4, 100, A, A, A, None) == INV
    assert L.svdq_debug_group_sums(4, 4, 64, A, A, None, None) == INV
    assert L.svdq_debug_group_sums(0, 4, 64, A, A, A, None) == capi.SVDQ_OK


def test_python_binding_raises_on_bad_status():
    import numpy as np
    import torch
    x = torch.zeros((4, 96), dtype=torch.bfloat16)       # K = 96: not a multiple of 64
    codes = torch.zeros((4, 48), dtype=torch.uint8)
    scales = torch.zeros((4, 2), dtype=torch.bfloat16)
    with pytest.raises(capi.SvdqError) as ei:
        capi.svdq_quantize_act(0, x, None, None, codes, scales, None, stream=0)
    assert ei.value.status == INV
    assert "K must" in str(ei.value)


def test_newer_entry_points_reject_bad_arguments_on_the_host():
    L = capi.lib()
    # GELU-fed activation step: same checks as svdq_quantize_act
    assert L.svdq_gelu_quantize_act(7, 4, 64, 16, A, A, A, A, A, A, None) == UNS
    assert L.svdq_gelu_quantize_act(0, 4, 65, 16, A, A, A, A, A, A, None) == INV
    assert L.svdq_gelu_quantize_act(0, 4, 64, 16, MIS, A, A, A, A, A, None) == INV
    assert L.svdq_gelu_quantize_act(0, 0, 64, 16, A, A, A, A, A, A, None) == capi.SVDQ_OK
    assert L.svdq_debug_gelu_bf16(-1, A, A, None) == INV
    assert L.svdq_debug_gelu_bf16(0, A, A, None) == capi.SVDQ_OK
    # QKV epilogue: int4 only, N = 3 * heads * 128, finite eps >= 0
    qk = lambda prec=0, N=384, eps=1e-6, cos=A: L.svdq_gemm_w4a4_qk_norm_rope(
        prec, 4, N, 64, 16, A, A, A, A, 1.0, A, A, A, A, A, eps, cos, A, A, None)
    assert qk(prec=4) == UNS
    assert qk(prec=capi.SVDQ_INT4_FP6, N=256) == INV
    assert qk(N=256) == INV
    assert qk(eps=-1.0) == INV
    assert qk(eps=float("inf")) == INV
    assert qk(cos=0) == INV
    # offline preparation
    assert L.svdq_smooth_factors(4, 8, 100, A, A, A, None) == INV
    assert L.svdq_quantize_weight(5, 8, 64, 16, A, A, A, A, A, A, None) == UNS
    assert L.svdq_quantize_weight(0, 8, 64, 16, A, A, 0, A, A, A, None) == INV
    assert L.svdq_quantize_weight(0, 0, 64, 0, A, 0, 0, 0, A, A, None) == capi.SVDQ_OK


def test_lowrank_workspace_query_and_checks():
    ws = capi.svdq_lowrank_workspace_bytes
    assert ws(256, 512, 32) > 0
    assert ws(512, 512, 32) >= ws(256, 512, 32)
    assert ws(256, 512, 8) == -1          # rank below 16
    assert ws(30, 512, 32) == -1          # N < rank + 8
    assert ws(256, 100, 32) == -1         # K not a multiple of 64
    L = capi.lib()
    need = ws(256, 512, 32)
    f = lambda rank=32, N=256, K=512, wb=need, work=A: L.svdq_lowrank_factors(N, K, rank, A, A, 1, work, wb, A, A, None)
    assert f(wb=need - 1) == INV
    assert f(rank=8) == INV
    assert f(N=39) == INV
    assert f(work=0) == INV


def test_lowrank_noalloc_host_checks():
    """The allocation-free low-rank entry point rejects, on the host, shapes
    whose workspace exceeds its fixed 32 MiB scratch, and the other bad
    arguments of svdq_lowrank_factors."""
    L = capi.lib()
    f = lambda rank=32, N=256, K=512, up=A, down=A: L.svdq_lowrank_factors_noalloc(N, K, rank, A, A, 1, up, down,
                                                                                    None)
    assert capi.svdq_lowrank_workspace_bytes(65536, 65536, 128) > 32 << 20
    assert f(rank=128, N=65536, K=65536) == INV
    assert "32" in capi.lib().svdq_last_error().decode() or "scratch" in capi.lib().svdq_last_error().decode()
    assert f(rank=8) == INV
    assert f(N=39) == INV
    assert f(up=0) == INV
    assert f(down=MIS) == INV
    # every layer of a 3072-wide DiT block at rank 32 fits
    for N, K in ((9216, 3072), (12288, 3072), (3072, 12288), (3072, 3072)):
        assert 0 < capi.svdq_lowrank_workspace_bytes(N, K, 32) <= 32 << 20


def test_packed_weight_entry_points_host_checks():
    """svdq_packed_weight_bytes and the host-side checks of the packed-weight
    entry points (no GPU needed: every rejection happens before a launch)."""
    L = capi.lib()
    # blob = codes [N, K/2] + bf16 [N][2][K/64]
    assert capi.svdq_packed_weight_bytes(12288, 3072) == 12288 * 1536 + 12288 * 2 * 48 * 2
    assert capi.svdq_packed_weight_bytes(1, 64) == 32 + 4
    assert capi.svdq_packed_weight_bytes(8, 100) == -1
    assert capi.svdq_packed_weight_bytes(-1, 64) == -1
    pk = lambda N=64, K=128, c=A, s=A, out=A, bad=A: L.svdq_pack_weight_int4(N, K, c, s, out, bad, None)
    assert pk(K=96) == INV
    assert pk(c=0) == INV
    assert pk(s=MIS) == INV
    assert pk(out=0) == INV
    assert pk(bad=A + 2) == INV                      # the counter must be 4-byte aligned
    assert pk(N=0) == capi.SVDQ_OK
    gs = lambda M=4, N=64, K=128, ac=A, w=A, G=A: L.svdq_debug_group_sums_packed(M, N, K, ac, w, G, None)
    assert gs(w=0) == INV
    assert gs(K=100) == INV
    assert gs(M=0) == capi.SVDQ_OK
    # the GEMM accepts precisions 2 and 3 (checks as for int4) and rejects 4
    assert gm(prec=4) == UNS
    assert gm(prec=capi.SVDQ_INT4_PACKED, wc=0) == INV
    assert gm(prec=capi.SVDQ_INT4_PACKED, M=0) == capi.SVDQ_OK


def test_fp6_entry_points_host_checks():
    """svdq_fp6_codes_bytes and the host-side checks of the FP6-layout entry
    points (every rejection happens before a launch)."""
    L = capi.lib()
    # tiles of 128 rows x pairs of groups, 12 KB each (padded)
    assert capi.svdq_fp6_codes_bytes(12288, 3072) == 12288 * 3072 * 3 // 4
    assert capi.svdq_fp6_codes_bytes(1, 64) == 12288
    assert capi.svdq_fp6_codes_bytes(130, 4160) == 2 * 33 * 12288
    assert capi.svdq_fp6_codes_bytes(8, 100) == -1
    assert capi.svdq_fp6_codes_bytes(-1, 64) == -1
    pk = lambda N=64, K=128, c=A, out=A: L.svdq_pack_weight_fp6(N, K, c, out, None)
    assert pk(K=96) == INV
    assert pk(c=0) == INV
    assert pk(out=MIS) == INV
    assert pk(N=0) == capi.SVDQ_OK
    gs = lambda M=4, N=64, K=128, ac=A, w=A, G=A: L.svdq_debug_group_sums_fp6(M, N, K, ac, w, G, None)
    assert gs(w=0) == INV
    assert gs(ac=MIS) == INV
    assert gs(K=100) == INV
    assert gs(N=0) == capi.SVDQ_OK
    # the activation steps and the GEMM take SVDQ_INT4_FP6 with int4's checks
    assert qa(prec=capi.SVDQ_INT4_FP6, K=96) == INV
    assert qa(prec=capi.SVDQ_INT4_FP6, M=0) == capi.SVDQ_OK
    assert L.svdq_gelu_quantize_act(capi.SVDQ_INT4_FP6, 4, 64, 8, A, A, A, A, A, A, None) == INV
    assert gm(prec=capi.SVDQ_INT4_FP6, wsc=0) == INV
    assert gm(prec=capi.SVDQ_INT4_FP6, rank=8) == INV
    assert gm(prec=capi.SVDQ_INT4_FP6, M=0) == capi.SVDQ_OK


def test_python_binding_checks_buffers_before_the_call():
    import torch
    x = torch.zeros((4, 128), dtype=torch.bfloat16)
    codes = torch.zeros((4, 64), dtype=torch.uint8)
    scales = torch.zeros((4, 2), dtype=torch.bfloat16)
    # a transposed view is not a flat buffer
    with pytest.raises(ValueError, match="contiguous"):
        capi.svdq_quantize_act(0, x, None, None, codes.t(), scales, None, stream=0)
    # codes too small for [4, 128] nibbles, scales too small for two groups per row
    with pytest.raises(ValueError, match="act_codes"):
        capi.svdq_quantize_act(0, x, None, None, codes[:3], scales, None, stream=0)
    with pytest.raises(ValueError, match="act_scales"):
        capi.svdq_quantize_act(0, x, None, None, codes, scales[:, :1].contiguous(), None, stream=0)
    # GEMM: an output smaller than [M, N] bf16
    out = torch.zeros((4, 63), dtype=torch.bfloat16)
    w = torch.zeros((64, 64), dtype=torch.uint8)
    ws = torch.zeros((64, 2), dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="out"):
        capi.svdq_gemm_w4a4(0, codes, scales, w, ws, 1.0, None, None, None, out, stream=0)


def test_gelu_quantize_entry_point_host_checks():
    """The up-GEMM with the next layer's activation step: FP6 layout only, N
    a multiple of 64 (the next layer's K), rank_next a multiple of 16 up to
    128, a workspace of at least the queried size; all checked on the host."""
    L = capi.lib()
    ws = capi.svdq_gelu_quantize_workspace_bytes
    # the fp32 low-rank partials [ceil(N/128)][M][rank_next]
    assert ws(4, 192, 32) == 2 * 4 * 32 * 4
    assert ws(4, 192, 0) == 0
    assert ws(4, 100, 32) == -1
    assert ws(4, 192, 8) == -1
    FP6 = capi.SVDQ_INT4_FP6

    def f(prec=FP6, M=4, N=192, K=64, rank=16, rank_next=32, smooth=A, down=A, codes=A, scales=A, lact=A,
          work=A, wb=None, out=A):
        wb = ws(M, N, rank_next) if wb is None else wb
        return L.svdq_gemm_w4a4_gelu_quantize(prec, M, N, K, rank, A, A, A, A, 1.0, A, A, A, rank_next, smooth,
                                              down, codes, scales, lact, work, wb, out, None)
    assert f(prec=capi.SVDQ_INT4) == UNS
    assert f(prec=capi.SVDQ_NVFP4) == UNS
    assert f(N=100) == INV
    assert f(N=0) == INV
    assert f(N=1 << 17) == INV
    assert f(K=100) == INV
    assert f(rank_next=8) == INV
    assert f(rank_next=144) == INV
    assert f(down=0) == INV
    assert f(lact=0) == INV
    assert f(codes=0) == INV
    assert f(scales=MIS) == INV
    assert f(work=0) == INV
    assert f(wb=ws(4, 192, 32) - 1) == INV
    assert f(M=0) == capi.SVDQ_OK
    assert f(M=0, rank_next=0, down=0, lact=0, smooth=0, out=0) == capi.SVDQ_OK
    assert f(M=0, rank_next=0, down=0, lact=0, work=0) == capi.SVDQ_OK      # nothing to hold

