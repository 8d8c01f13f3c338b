"""fp8_amax_quant_noalloc through the C ABI against fp8_amax_quant: two calls
in a row on one GPU, the second on a smaller tensor (its partials fewer than
the first call left in the shared scratch), each bit-identical to the
workspace entry point (codes, transposed codes, scale, amax)."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import _native, api, synth
from tests.gpu_util import to_dev_bf16

pytestmark = pytest.mark.gpu


def _noalloc(x, fmt, q, qt, scale, amax):
    L = _native.lib()
    rows, cols = x.shape
    st = L.fp8_amax_quant_noalloc(ctypes.c_void_p(x.data_ptr()), rows, cols, x.stride(0), fmt,
                                  ctypes.c_void_p(q.data_ptr()), q.stride(0), ctypes.c_void_p(qt.data_ptr()),
                                  qt.stride(0), ctypes.c_void_p(scale.data_ptr()), ctypes.c_void_p(amax.data_ptr()),
                                  ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, _native.status_string(st)


@pytest.mark.parametrize("fmt", [oracle.E4M3, oracle.E5M2])
def test_noalloc_matches_workspace_entry_point(fmt):
    dev = torch.device("cuda:0")
    # first call: 4096 x 3000 (188 partials); second: 300 x 700 (4 partials)
    for i, (rows, cols) in enumerate(((4096, 3000), (300, 700))):
        x = to_dev_bf16(synth.normal_bf16((rows, cols), 1.0 if fmt == oracle.E4M3 else 1e-3, 70 + i,
                                          outlier_frac=1e-3))
        u8 = dict(dtype=torch.uint8, device=dev)
        q, qt = torch.full((rows, cols), 7, **u8), torch.full((cols, rows), 7, **u8)
        sc, am = torch.zeros(1, dtype=torch.float32, device=dev), torch.zeros(1, dtype=torch.float32, device=dev)
        _noalloc(x, fmt, q, qt, sc, am)
        rq, rqt, rsc, ram = api.fp8_amax_quant(x, fmt, want_qt=True)
        torch.cuda.synchronize()
        assert torch.equal(q, rq) and torch.equal(qt, rqt), (rows, cols)
        assert torch.equal(sc, rsc) and torch.equal(am, ram), (rows, cols, float(sc), float(rsc))
        # and both equal the oracle's quantisation
        oq, osc, oam = oracle.quant(x.cpu().view(torch.int16).numpy().view(np.uint16), fmt)
        assert (q.cpu().numpy() == oq).all() and np.float32(float(sc[0])) == np.float32(osc)


def test_noalloc_validates_before_launching():
    L = _native.lib()
    fake = ctypes.c_void_p(0x10000)
    ok = [fake, 64, 64, 64, 0, ctypes.c_void_p(0x20000), 64, None, 0, fake, None, None]
    a = list(ok); a[9] = None
    assert L.fp8_amax_quant_noalloc(*a) == 1          # no scale
    a = list(ok); a[4] = 9
    assert L.fp8_amax_quant_noalloc(*a) == 1          # unknown format
    a = list(ok); a[0] = ctypes.c_void_p(0x10001)
    assert L.fp8_amax_quant_noalloc(*a) == 2          # x not 2-byte aligned
