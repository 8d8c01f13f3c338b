"""The library under HIP graph capture.  Each path is captured once with
preallocated outputs and workspaces and replayed several times, with eager
work and synchronisations in between; every replay gives the eager pass's
bytes (the kernels are deterministic, clear nothing with memset and
allocate nothing)."""
import numpy as np
import pytest
import torch

from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _relu2():
    from fp8_tensorwise_scaled_amd import api

    w = synth.MLPWorkload(51, 512, 256, 1024, sigma_up=1 / 16, sigma_down=1 / 32)
    x, wu, wd, dy = (to_dev_bf16(t) for t in w.tensors())
    M, d, h = w.M, w.d, w.h
    dev = x.device
    bf = dict(dtype=torch.bfloat16, device=dev)
    outs = dict(y=torch.empty((M, d), **bf), dx=torch.empty((M, d), **bf), dwu=torch.empty((h, d), **bf),
                dwd=torch.empty((d, h), **bf), bsc=torch.empty(2, dtype=torch.float32, device=dev))
    saved = api.Relu2MlpSaved.empty(M, d, h, dev)
    ws_f, ws_b = api.relu2_mlp_fwd_workspace(M, d, h, dev), api.relu2_mlp_bwd_workspace(M, d, h, dev)

    def step():
        api.relu2_mlp_fwd(x, wu, wd, y=outs["y"], saved=saved, ws=ws_f)
        api.relu2_mlp_bwd(dy, saved, dx=outs["dx"], dw_up=outs["dwu"], dw_down=outs["dwd"],
                          bwd_scales=outs["bsc"], ws=ws_b)
    return step, outs


def _swiglu():
    from fp8_tensorwise_scaled_amd import api

    w = synth.SwigluWorkload(52, 256, 128, 352, sigma_in=1 / 11, sigma_down=1 / 19)
    x, wg, wu, wd, dy = (to_dev_bf16(t) for t in w.tensors())
    M, d, h = w.M, w.d, w.h
    dev = x.device
    bf = dict(dtype=torch.bfloat16, device=dev)
    outs = dict(y=torch.empty((M, d), **bf), dx=torch.empty((M, d), **bf), dwg=torch.empty((h, d), **bf),
                dwu=torch.empty((h, d), **bf), dwd=torch.empty((d, h), **bf),
                bsc=torch.empty(3, dtype=torch.float32, device=dev))
    saved = api.SwigluMlpSaved.empty(M, d, h, dev)
    ws_f, ws_b = api.swiglu_mlp_workspace("fwd", M, d, h, dev), api.swiglu_mlp_workspace("bwd", M, d, h, dev)

    def step():
        api.swiglu_mlp_fwd(x, wg, wu, wd, y=outs["y"], saved=saved, ws=ws_f)
        api.swiglu_mlp_bwd(dy, saved, dx=outs["dx"], dw_gate=outs["dwg"], dw_up=outs["dwu"], dw_down=outs["dwd"],
                           bwd_scales=outs["bsc"], ws=ws_b)
    return step, outs


def _lm_head_ce():
    from fp8_tensorwise_scaled_amd import api

    wl = synth.LMHeadCEWorkload(53, 256, 256, 600, n_classes=590, chunk=64, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    X, W = to_dev_bf16(x), to_dev_bf16(w)
    T = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).cuda()
    dev = X.device
    M, K, V = wl.M, wl.K, wl.V
    outs = dict(loss=torch.empty(1, dtype=torch.float32, device=dev),
                dx=torch.empty((M, K), dtype=torch.bfloat16, device=dev),
                dw=torch.empty((V, K), dtype=torch.bfloat16, device=dev),
                scales=torch.empty(2 + M // wl.chunk, dtype=torch.float32, device=dev))
    ws = api.fp8_lm_head_ce_workspace(M, K, V, wl.chunk, dev)

    def step():
        api.fp8_lm_head_ce(X, W, T, wl.n_classes, wl.softcap, wl.chunk, ws=ws, **outs)
    return step, outs


def _newton_schulz():
    from fp8_tensorwise_scaled_amd import api

    G = to_dev_bf16(synth.normal_bf16((208, 720), 0.02, 54))
    dev = G.device
    outs = dict(out=torch.empty((208, 720), dtype=torch.bfloat16, device=dev),
                norm=torch.empty(2, dtype=torch.float32, device=dev))
    ws = api.muon_ns_workspace(208, 720, dev)

    def step():
        api.muon_newton_schulz(G, 5, out=outs["out"], norm=outs["norm"], ws=ws)
    return step, outs


def _rmsnorm():
    from fp8_tensorwise_scaled_amd import _native, api

    rows, cols = 300, 392  # ragged row tiles and a 136-column last column tile
    x = to_dev_bf16(synth.normal_bf16((rows, cols), 2.0, 55))
    g = to_dev_bf16(synth.normal_bf16((cols,), 1.0, 56))
    dev = x.device
    f32 = dict(dtype=torch.float32, device=dev)
    outs = dict(q=torch.empty((rows, cols), dtype=torch.uint8, device=dev),
                qt=torch.empty((cols, rows), dtype=torch.uint8, device=dev),
                scale=torch.empty(1, **f32), amax=torch.empty(1, **f32), rstd=torch.empty(rows, **f32))
    ws = torch.empty(max(_native.lib().fp8_rmsnorm_quant_workspace_bytes(rows, cols), 16), dtype=torch.uint8,
                     device=dev)

    def step():
        api.fp8_rmsnorm_quant(x, g, 1e-6, api.E4M3, ws=ws, **outs)
    return step, outs


def _fp8_linear():
    """One FP8 linear layer's three GEMMs with their quantisations."""
    from fp8_tensorwise_scaled_amd import _native, api

    M, K, N = 384, 256, 320
    x = to_dev_bf16(synth.normal_bf16((M, K), 1.0, 57))
    w = to_dev_bf16(synth.normal_bf16((N, K), 0.05, 58))
    dy = to_dev_bf16(synth.normal_bf16((M, N), 1e-3, 59))
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    L = _native.lib()
    codes = {k: (torch.empty(shape, **u8), torch.empty(shape[::-1], **u8), torch.empty(1, **f32),
                 torch.empty(1, **f32), torch.empty(max(L.fp8_amax_quant_workspace_bytes(*shape), 16), **u8))
             for k, shape in (("x", (M, K)), ("w", (N, K)), ("g", (M, N)))}
    outs = dict(y=torch.empty((M, N), **bf), dx=torch.empty((M, K), **bf), dw=torch.empty((N, K), **bf))
    for k, (q, qt, sc, am, _) in codes.items():  # the codes and scales are cleared between replays too
        outs.update({k + "_q": q, k + "_qt": qt, k + "_scale": sc, k + "_amax": am})

    def step():
        for k, src, fmt in (("x", x, api.E4M3), ("w", w, api.E4M3), ("g", dy, api.E5M2)):
            q, qt, sc, am, ws = codes[k]
            api.fp8_amax_quant(src, fmt, q=q, qt=qt, scale=sc, amax=am, ws=ws)
        (xq, xqt, sx, _, _), (wq, wqt, sw, _, _), (gq, gqt, sg, _, _) = codes["x"], codes["w"], codes["g"]
        api.fp8_linear_fwd(xq, sx, wq, sw, out=outs["y"])
        api.fp8_linear_dgrad(gq, sg, wq, sw, out=outs["dx"])
        api.fp8_linear_wgrad(gq, sg, xq, sx, out=outs["dw"])
    return step, outs


def _fp8_linear_from_bf16():
    """A linear's forward from bf16 X and W (batched quantisation, then the
    GEMM) followed by its two backward GEMMs on the codes it wrote."""
    from fp8_tensorwise_scaled_amd import _native, api

    M, K, N = 300, 200, 272
    x = to_dev_bf16(synth.normal_bf16((M, K), 1.0, 61))
    w = to_dev_bf16(synth.normal_bf16((N, K), 0.05, 62))
    dy = to_dev_bf16(synth.normal_bf16((M, N), 1e-3, 63))
    dev = x.device
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    bf = dict(dtype=torch.bfloat16, device=dev)
    L = _native.lib()
    ld = -(-K // 16) * 16
    outs = dict(y=torch.empty((M, N), **bf), xq=torch.empty((M, ld), **u8)[:, :K], wq=torch.empty((N, ld), **u8)[:, :K],
                scales=torch.empty(2, **f32), gq=torch.empty((M, N), **u8), sg=torch.empty(1, **f32),
                ag=torch.empty(1, **f32), dx=torch.empty((M, K), **bf), dw=torch.empty((N, K), **bf))
    ws = torch.empty(max(L.fp8_linear_fwd_bf16_workspace_bytes(M, N, K), 16), **u8)
    wsg = torch.empty(max(L.fp8_amax_quant_workspace_bytes(M, N), 16), **u8)

    def step():
        api.fp8_linear_fwd_bf16(x, w, xq=outs["xq"], wq=outs["wq"], scales=outs["scales"], out=outs["y"], ws=ws)
        api.fp8_amax_quant(dy, api.E5M2, q=outs["gq"], scale=outs["sg"], amax=outs["ag"], ws=wsg)
        sx, sw = outs["scales"][0:1], outs["scales"][1:2]
        api.fp8_linear_dgrad(outs["gq"], outs["sg"], outs["wq"], sw, out=outs["dx"])
        api.fp8_linear_wgrad(outs["gq"], outs["sg"], outs["xq"], sx, out=outs["dw"])
    return step, outs


def _bytes(t):
    return t.detach().contiguous().view(torch.uint8).cpu().clone()


@pytest.mark.parametrize("make", [_relu2, _swiglu, _lm_head_ce, _newton_schulz, _rmsnorm, _fp8_linear,
                                  _fp8_linear_from_bf16],
                         ids=["relu2_block", "swiglu_block", "lm_head_ce", "newton_schulz", "rmsnorm_quant",
                              "fp8_linear", "fp8_linear_from_bf16"])
def test_graph_replays_match_eager(make):
    step, outs = make()
    step()
    torch.cuda.synchronize()
    eager = {k: _bytes(v) for k, v in outs.items()}

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for v in outs.values():
            v.zero_()  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k, v in outs.items():
            assert torch.equal(_bytes(v), eager[k]), (rep, k)
