"""A hot-path step captured into one HIP graph (torch.cuda.CUDAGraph on ROCm)
gives, on every replay, exactly the outputs of the same step run eagerly --
the form in which bench.py times the step.  Replays are interleaved with
eager work and synchronizations, and each is compared bit for bit."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

from bit_w4a4_quantized_svdq_amd import synth  # noqa: E402
from tests.gpu_helpers import announce  # noqa: E402

pytestmark = pytest.mark.gpu


def _layers():
    from bit_w4a4_quantized_svdq_amd.layer import AWQW4A16Linear, SVDQW4A4Linear
    out = []
    for i, (prec, M, K, N) in enumerate((("int4", 200, 512, 320), ("nvfp4", 130, 256, 192))):
        w = synth.synthetic_w4a4_weights(100 + i, N, K, 32, prec)
        L = SVDQW4A4Linear(prec, w["wgt_codes"], w["wgt_scales"], w["lora_down"], w["lora_up"], w["smooth"],
                           synth.to_bf16_bits(np.random.default_rng(i).standard_normal(N)))
        x, _ = synth.draw_activations(np.random.default_rng(200 + i), M, K, 4, 30.0)
        xt = torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
        out.append((L, xt))
    aw = synth.synthetic_awq_weights(7, 256, 512)
    G = AWQW4A16Linear(aw["wgt_codes"], aw["wgt_scales"], aw["wgt_zeros"], None)
    xg = torch.from_numpy(synth.to_bf16_bits(np.random.default_rng(9).standard_normal((1, 512))).view(np.int16))
    return out, (G, xg.view(torch.bfloat16).cuda())


def _step(w4a4, gemv):
    outs = [L(x) for L, x in w4a4]
    G, xg = gemv
    outs.append(G(xg))
    return outs


def test_graph_replay_matches_eager():
    announce("graph replay", "int4 200x512->320 + nvfp4 130x256->192 + awq 1x512->256")
    w4a4, gemv = _layers()
    ref = [o.clone() for o in _step(w4a4, gemv)]            # eager; also allocates every buffer
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _step(w4a4, gemv)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = _step(w4a4, gemv)
    for rep in range(3):
        for o in outs:
            o.zero_()                                        # stale results cannot pass
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), f"replay {rep}, output {i}"
        eager = _step(w4a4, gemv)                            # eager work between replays
        torch.cuda.synchronize()
        for o, r in zip(eager, ref):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))


def test_graph_replay_matches_eager_fused_paths():
    """The next-row paths in one graph: a grouped QKV layer with the per-head
    norm/rotary epilogue, a down layer whose activation step applies GELU,
    and the AWQ layer in its GEMM regime."""
    from bit_w4a4_quantized_svdq_amd.layer import AWQW4A16Linear, SVDQW4A4Linear
    announce("graph replay", "qkv norm/rotary 130x256->384, gelu-fed 96x512->192, awq gemm 256x512->2304")
    rng = np.random.default_rng(31)
    bf = lambda a: torch.from_numpy(synth.to_bf16_bits(a).view(np.int16)).view(torch.bfloat16).cuda()
    wq = synth.synthetic_w4a4_weights(40, 384, 256, 32, "int4")
    Q = SVDQW4A4Linear("int4", wq["wgt_codes"], wq["wgt_scales"], wq["lora_down"], wq["lora_up"], wq["smooth"], None)
    xq = bf(rng.standard_normal((130, 256)))
    qw, kw = bf(rng.uniform(0.5, 1.5, 128)), bf(rng.uniform(0.5, 1.5, 128))
    th = rng.uniform(-np.pi, np.pi, (130, 64))
    cs = torch.from_numpy(np.cos(th).astype(np.float32)).cuda()
    sn = torch.from_numpy(np.sin(th).astype(np.float32)).cuda()
    wd = synth.synthetic_w4a4_weights(41, 192, 512, 32, "int4")
    D = SVDQW4A4Linear("int4", wd["wgt_codes"], wd["wgt_scales"], wd["lora_down"], wd["lora_up"], wd["smooth"], None)
    ud = bf(rng.standard_normal((96, 512)) * 3.0)
    aw = synth.synthetic_awq_weights(42, 2304, 512)
    A = AWQW4A16Linear(aw["wgt_codes"], aw["wgt_scales"], aw["wgt_zeros"], None)
    xa = bf(rng.standard_normal((256, 512)))
    bq, bd = Q.buffers(130), D.buffers(96)

    def step():
        Q.quantize(xq, bq)
        Q.gemm_qk_norm_rope(bq, qw, kw, 1e-6, cs, sn)
        D.quantize(ud, bd, gelu=True)
        D.gemm(bd)
        return [bq["out"], bd["out"], A(xa)]

    ref = [o.clone() for o in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        for o in outs:
            o.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16)), f"replay {rep}, output {i}"
        eager = step()
        torch.cuda.synchronize()
        for o, r in zip(eager, ref):
            assert torch.equal(o.view(torch.int16), r.view(torch.int16))


def test_graph_replay_matches_eager_mlp_in_the_up_epilogue():
    """A GELU MLP whose up GEMM runs the down layer's activation step in its
    epilogue (svdq_gemm_w4a4_gelu_quantize: GEMM and fixed-order
    partial sum), then the down GEMM, in one graph: every replay gives the
    eager bytes of the down layer's codes, scales, lora_act and output."""
    from bit_w4a4_quantized_svdq_amd.layer import SVDQW4A4Linear
    announce("graph replay", "mlp 130x256->320 (up epilogue gelu-quantize) ->192")
    rng = np.random.default_rng(43)
    wu = synth.synthetic_w4a4_weights(44, 320, 256, 32, "int4")
    U = SVDQW4A4Linear("int4", wu["wgt_codes"], wu["wgt_scales"], wu["lora_down"], wu["lora_up"], wu["smooth"],
                       synth.to_bf16_bits(rng.standard_normal(320)))
    wd = synth.synthetic_w4a4_weights(45, 192, 320, 16, "int4")
    D = SVDQW4A4Linear("int4", wd["wgt_codes"], wd["wgt_scales"], wd["lora_down"], wd["lora_up"], wd["smooth"], None)
    x, _ = synth.draw_activations(rng, 130, 256, 3, 30.0)
    xt = torch.from_numpy(synth.to_bf16_bits(x).view(np.int16)).view(torch.bfloat16).cuda()
    bu, bd = U.buffers(130), D.buffers(130)

    def step():
        U.quantize(xt, bu)
        U.gemm_gelu_quantize(bu, D, bd)
        D.gemm(bd)
        return [bd["codes"], bd["scales"], bd["lora_act"], bd["out"]]

    for o in (bd["codes"], bd["scales"], bd["lora_act"], bd["out"]):
        o.zero_()                                            # the FP6 layout's padding rows stay 0
    ref = [o.clone() for o in step()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step()
    for rep in range(3):
        for o in outs:
            o.zero_()
        bu["gq_workspace"].zero_()                           # the workspace needs no initialisation
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, r) in enumerate(zip(outs, ref)):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}, output {i}"
        eager = step()
        torch.cuda.synchronize()
        for o, r in zip(eager, ref):
            assert torch.equal(o.view(torch.uint8), r.view(torch.uint8))
