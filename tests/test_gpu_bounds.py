"""Out-of-bounds writes.  Every output, saved tensor and workspace of a call
is a view into a larger buffer filled with a guard byte; after the call the
bytes around the view (and, for a strided view, between its rows) still
hold the guard.  The shapes are ragged, so edge tiles are partial: the
place where an off-by-one row or column write would land.  Values are
checked by the parity tests; here only that nothing outside the outputs
changes."""
import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import to_dev_bf16, to_dev_u8

pytestmark = pytest.mark.gpu
GUARD = 0x5A
PAD = 4096  # guard bytes before and after every view (keeps 16-byte alignment)


class Guarded:
    """A [rows, cols] view with leading dimension ld (>= cols) inside a
    guard-filled byte buffer with PAD bytes on either side."""

    def __init__(self, rows, cols, dtype, ld=None):
        self.esz = torch.empty(0, dtype=dtype).element_size()
        self.rows, self.cols, self.ld = rows, cols, cols if ld is None else ld
        span = ((rows - 1) * self.ld + cols) * self.esz if rows and cols else 0
        self.buf = torch.full((2 * PAD + span,), GUARD, dtype=torch.uint8, device="cuda:0")
        inner = self.buf[PAD:PAD + span]
        self.view = inner.view(dtype).as_strided((rows, cols), (self.ld, 1)) if span else \
            torch.empty((rows, cols), dtype=dtype, device="cuda:0")

    def intact(self) -> bool:
        b = self.buf.cpu().numpy()
        mask = np.ones(b.size, bool)
        if self.rows and self.cols:
            starts = PAD + np.arange(self.rows) * self.ld * self.esz
            for s in starts:
                mask[s:s + self.cols * self.esz] = False
        return bool((b[mask] == GUARD).all())


def dense(shape, dtype):
    g = Guarded(int(np.prod(shape[:-1])), shape[-1], dtype)
    return g, g.view.view(shape)


def ws_guarded(nbytes):
    g = Guarded(1, nbytes, torch.uint8)
    return g, g.view.view(-1)


def scal(v):
    return torch.tensor([v], dtype=torch.float32, device="cuda:0")


def codes(shape, fmt, seed):
    x = synth.normal_bf16(shape, 1.0, seed)
    q, s, _ = oracle.quant(x, fmt)
    return q, s


def test_gemm_outputs_stay_in_bounds():
    """fwd / dgrad / wgrad, M=304, N=208, K=160 (every output dimension a
    ragged tile), outputs with a leading dimension 40 elements wider than the
    row."""
    from fp8_tensorwise_scaled_amd import api

    M, N, K = 304, 208, 160
    E4, E5 = oracle.E4M3, oracle.E5M2
    xq, sx = codes((M, K), E4, 1)
    wq, sw = codes((N, K), E4, 2)
    gq, sg = codes((M, N), E5, 3)
    calls = (
        ("fwd", (M, N), lambda out, acc: api.fp8_linear_fwd(to_dev_u8(xq), scal(sx), to_dev_u8(wq), scal(sw),
                                                            out=out, accum=acc)),
        ("dgrad", (M, K), lambda out, acc: api.fp8_linear_dgrad(to_dev_u8(gq), scal(sg), to_dev_u8(wq), scal(sw),
                                                                out=out, accum=acc)),
        ("wgrad", (N, K), lambda out, acc: api.fp8_linear_wgrad(to_dev_u8(gq), scal(sg), to_dev_u8(xq), scal(sx),
                                                                out=out, accum=acc)),
    )
    for accum in (0, 1):
        for name, (r, c), call in calls:
            g = Guarded(r, c, torch.bfloat16, ld=c + 40)
            call(g.view, accum)
            torch.cuda.synchronize()
            assert g.intact(), (name, accum)


def test_quantiser_outputs_stay_in_bounds():
    """[300, 700] with q, qt strided and the scale, amax and workspace
    guarded; also the RMSNorm-fused quantiser with its per-row rstd."""
    from fp8_tensorwise_scaled_amd import _native, api

    R, C = 300, 700
    x = to_dev_bf16(synth.normal_bf16((R, C), 1.0, 4))
    for fmt in (oracle.E4M3, oracle.E5M2):
        q = Guarded(R, C, torch.uint8, ld=C + 36)
        qt = Guarded(C, R, torch.uint8, ld=R + 20)
        s, sv = dense((1,), torch.float32)
        a, av = dense((1,), torch.float32)
        w, wv = ws_guarded(_native.lib().fp8_amax_quant_workspace_bytes(R, C))
        api.fp8_amax_quant(x, fmt, q=q.view, qt=qt.view, scale=sv, amax=av, ws=wv)
        torch.cuda.synchronize()
        assert q.intact() and qt.intact() and s.intact() and a.intact() and w.intact(), fmt
    gamma = to_dev_bf16(synth.normal_bf16((C,), 1.0, 5))
    q = Guarded(R, C, torch.uint8, ld=C + 36)
    qt = Guarded(C, R, torch.uint8, ld=R + 20)
    rs, rsv = dense((R,), torch.float32)
    w, wv = ws_guarded(_native.lib().fp8_rmsnorm_quant_workspace_bytes(R, C))
    api.fp8_rmsnorm_quant(x, gamma, 1e-6, oracle.E4M3, q=q.view, qt=qt.view, rstd=rsv, ws=wv)
    torch.cuda.synchronize()
    assert q.intact() and qt.intact() and rs.intact() and w.intact()


def test_relu2_block_stays_in_bounds():
    """M=48, d=64, h=176: every GEMM a single ragged tile; outputs, the
    saved set and both workspaces guarded."""
    from fp8_tensorwise_scaled_amd import _native, api

    w = synth.MLPWorkload(45, 48, 64, 176, sigma_up=1 / 8, sigma_down=1 / 13)
    x, wu, wd, dy = (to_dev_bf16(t) for t in w.tensors())
    M, d, h = w.M, w.d, w.h
    L = _native.lib()
    gs = {}
    gs["xq"], xq = dense((M, d), torch.uint8)
    gs["uq"], uq = dense((h, d), torch.uint8)
    gs["dq"], dq = dense((d, h), torch.uint8)
    gs["aq"], aq = dense((M, h), torch.uint8)
    gs["h"], hh = dense((M, h), torch.bfloat16)
    gs["scales"], sc = dense((4,), torch.float32)
    saved = api.Relu2MlpSaved(xq, uq, dq, aq, hh, sc, M, d, h)
    gs["y"], y = dense((M, d), torch.bfloat16)
    gs["dx"], dx = dense((M, d), torch.bfloat16)
    gs["dwu"], dwu = dense((h, d), torch.bfloat16)
    gs["dwd"], dwd = dense((d, h), torch.bfloat16)
    gs["bsc"], bsc = dense((2,), torch.float32)
    gs["ws_f"], wsf = ws_guarded(L.relu2_mlp_fwd_workspace_bytes(M, d, h))
    gs["ws_b"], wsb = ws_guarded(L.relu2_mlp_bwd_workspace_bytes(M, d, h))
    api.relu2_mlp_fwd(x, wu, wd, y=y, saved=saved, ws=wsf)
    api.relu2_mlp_bwd(dy, saved, dx=dx, dw_up=dwu, dw_down=dwd, bwd_scales=bsc, ws=wsb)
    torch.cuda.synchronize()
    bad = [k for k, g in gs.items() if not g.intact()]
    assert not bad, bad


def test_swiglu_block_stays_in_bounds():
    """M=48, d=64, h=176 through the gated block, everything guarded."""
    from fp8_tensorwise_scaled_amd import _native, api

    w = synth.SwigluWorkload(46, 48, 64, 176, sigma_in=1 / 8, sigma_down=1 / 13)
    x, wg, wu, wd, dy = (to_dev_bf16(t) for t in w.tensors())
    M, d, h = w.M, w.d, w.h
    L = _native.lib()
    gs = {}
    gs["xq"], xq = dense((M, d), torch.uint8)
    gs["wgq"], wgq = dense((h, d), torch.uint8)
    gs["wuq"], wuq = dense((h, d), torch.uint8)
    gs["wdq"], wdq = dense((d, h), torch.uint8)
    gs["aq"], aq = dense((M, h), torch.uint8)
    gs["g"], gg = dense((M, h), torch.bfloat16)
    gs["u"], uu = dense((M, h), torch.bfloat16)
    gs["scales"], sc = dense((5,), torch.float32)
    saved = api.SwigluMlpSaved(xq, wgq, wuq, wdq, aq, gg, uu, sc, M, d, h)
    gs["y"], y = dense((M, d), torch.bfloat16)
    gs["dx"], dx = dense((M, d), torch.bfloat16)
    gs["dwg"], dwg = dense((h, d), torch.bfloat16)
    gs["dwu"], dwu = dense((h, d), torch.bfloat16)
    gs["dwd"], dwd = dense((d, h), torch.bfloat16)
    gs["bsc"], bsc = dense((3,), torch.float32)
    gs["ws_f"], wsf = ws_guarded(L.swiglu_mlp_fwd_workspace_bytes(M, d, h))
    gs["ws_b"], wsb = ws_guarded(L.swiglu_mlp_bwd_workspace_bytes(M, d, h))
    api.swiglu_mlp_fwd(x, wg, wu, wd, y=y, saved=saved, ws=wsf)
    api.swiglu_mlp_bwd(dy, saved, dx=dx, dw_gate=dwg, dw_up=dwu, dw_down=dwd, bwd_scales=bsc, ws=wsb)
    torch.cuda.synchronize()
    bad = [k for k, g in gs.items() if not g.intact()]
    assert not bad, bad


def test_lm_head_ce_stays_in_bounds():
    """M=208, K=64, V=600 (590 classes) in chunks of 64 rows, the last
    partial; loss, gradients, chunk scales and workspace guarded."""
    from fp8_tensorwise_scaled_amd import _native, api

    wl = synth.LMHeadCEWorkload(55, 208, 64, 600, n_classes=590, chunk=64, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    X, W = to_dev_bf16(x), to_dev_bf16(w)
    T = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).cuda()
    M, K, V, C = wl.M, wl.K, wl.V, wl.chunk
    gs = {}
    gs["loss"], loss = dense((1,), torch.float32)
    gs["dx"], dx = dense((M, K), torch.bfloat16)
    gs["dw"], dw = dense((V, K), torch.bfloat16)
    gs["scales"], sc = dense((2 + -(-M // C),), torch.float32)
    gs["ws"], ws = ws_guarded(_native.lib().fp8_lm_head_ce_workspace_bytes(M, K, V, C))
    api.fp8_lm_head_ce(X, W, T, wl.n_classes, wl.softcap, C, loss=loss, dx=dx, dw=dw, scales=sc, ws=ws)
    torch.cuda.synchronize()
    bad = [k for k, g in gs.items() if not g.intact()]
    assert not bad, bad


def test_bf16_products_and_newton_schulz_stay_in_bounds():
    """bf16 product 300x200x264 with aux and the transposed store, strided;
    symmetric product 208x720 with its workspace; Newton-Schulz on
    208x720 and 720x208."""
    from fp8_tensorwise_scaled_amd import _native, api

    a = to_dev_bf16(synth.normal_bf16((300, 264), 1.0, 6))
    b = to_dev_bf16(synth.normal_bf16((200, 264), 1.0, 7))
    aux = to_dev_bf16(synth.normal_bf16((300, 200), 1.0, 8))
    c = Guarded(300, 200, torch.bfloat16, ld=232)
    ct = Guarded(200, 300, torch.bfloat16, ld=328)
    api.bf16_gemm_nt(a, b, 2.0, -1.5, aux, out=c.view, out_t=ct.view)
    torch.cuda.synchronize()
    assert c.intact() and ct.intact()

    g = to_dev_bf16(synth.normal_bf16((208, 720), 0.02, 9))
    s = Guarded(208, 208, torch.bfloat16, ld=216)
    w, wv = ws_guarded(_native.lib().bf16_gemm_sym_workspace_bytes(208, 720))
    api.bf16_gemm_sym(g, out=s.view, ws=wv)
    torch.cuda.synchronize()
    assert s.intact() and w.intact()

    for shape in ((208, 720), (720, 208)):
        gm = to_dev_bf16(synth.normal_bf16(shape, 0.02, 10))
        o, ov = dense(shape, torch.bfloat16)
        n, nv = dense((2,), torch.float32)
        w, wv = ws_guarded(_native.lib().muon_ns_workspace_bytes(*shape))
        api.muon_newton_schulz(gm, 5, out=ov, norm=nv, ws=wv)
        torch.cuda.synchronize()
        assert o.intact() and n.intact() and w.intact(), shape
