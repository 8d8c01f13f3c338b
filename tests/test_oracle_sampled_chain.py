"""The sampled-stage oracle used by the full-size block tests reproduces the
full oracle chain bit for bit on its rows and columns (transposed products
sum the same exact products in the same order), so sampled checks at
M=8192 / 32768 carry the same expected values a full run would."""
import numpy as np
import pytest

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import bits_f64
from tests.mlp_chain import compare_block, full_chain_scales, sampled_chain


def _block():
    w = synth.MLPWorkload(31, 192, 128, 384, sigma_up=1 / 11.3, sigma_down=1 / 19.6)
    return w.tensors()


def test_sampled_chain_matches_full_chain():
    x, wu, wd, dy = _block()
    sc, f, b = full_chain_scales(x, wu, wd, dy)
    rows = np.array([0, 5, 77, 191])
    cols = np.array([1, 2, 200, 383])
    o = sampled_chain(x, wu, wd, dy, sc, rows, cols)
    assert (o["H_r"] == f["h"][rows]).all()
    assert (o["Aq_r"] == f["aq"][rows]).all()
    assert (o["Y_r"] == f["y"][rows]).all()
    assert (o["dA_r"] == b["da"][rows]).all()
    assert (o["dH_r"] == b["dh"][rows]).all()
    assert (o["Hq_r"] == b["hq"][rows]).all()
    assert (o["dX_r"] == b["dx"][rows]).all()
    assert (o["Ht_c"] == f["h"][:, cols].T).all()
    assert (o["dAt_c"] == b["da"][:, cols].T).all()
    assert (o["Aqt_c"] == f["aq"][:, cols].T).all()
    assert (o["Hqt_c"] == b["hq"][:, cols].T).all()
    assert (o["dWup_c"] == b["dw_up"][cols]).all()
    assert (o["dWdnT_c"] == b["dw_down"][:, cols].T).all()


def _as_gpu_dict(x, wu, wd, dy, f, b):
    """The oracle's own chain laid out like the GPU tests' collected outputs."""
    return dict(x=x, wu=wu, wd=wd, dy=dy, y=f["y"], dx=b["dx"], dw_up=b["dw_up"], dw_down=b["dw_down"],
                h=f["h"], scales=np.array([f["sx"], f["su"], f["sd"], f["sa"]], np.float32),
                bsc=np.array([b["sg"], b["sh"]], np.float32), xq=f["xq"], uq=f["uq"], dq=f["dq"], aq=f["aq"],
                gq=b["gq"], dh=b["dh"], hq=b["hq"])


@pytest.mark.parametrize("accum", [0, 1], ids=["fast", "exact"])
def test_compare_block_accepts_the_oracle_and_rejects_planted_errors(accum):
    """The comparison passes the oracle's own chain in both accumulation
    modes, and fails on one flipped A code, on one dX element moved by a few
    ulps, and on one dW_down element moved likewise."""
    x, wu, wd, dy = _block()
    sc, f, b = full_chain_scales(x, wu, wd, dy)
    rows, cols = np.arange(192), np.arange(384)
    o = sampled_chain(x, wu, wd, dy, sc, rows, cols)
    g = _as_gpu_dict(x, wu, wd, dy, f, b)
    compare_block(g, o, sc, rows, cols, accum)

    def planted(key, i, delta):
        bad = dict(g)
        bad[key] = g[key].copy()
        bad[key][i] = (bad[key][i].astype(np.int64) + delta).astype(bad[key].dtype)
        return bad

    i = tuple(np.argwhere(g["aq"] != 0)[0])
    j = tuple(np.argwhere(np.abs(bits_f64(g["dx"])) > 0)[3])
    k = tuple(np.argwhere(np.abs(bits_f64(g["dw_down"])) > 0)[5])
    for what, bad in (("A code", planted("aq", i, 1)), ("dX element", planted("dx", j, 40)),
                      ("dW_down element", planted("dw_down", k, 40))):
        with pytest.raises(AssertionError):
            compare_block(bad, o, sc, rows, cols, accum)


def test_chain_bar_exempts_only_rows_downstream_of_a_moved_code():
    """Exact mode holds every output row to the max-relative bar except the
    rows marked as downstream of a moved code; the Frobenius bar holds for
    all rows."""
    from tests.mlp_chain import chain_close

    rng = np.random.default_rng(7)
    ref32 = rng.standard_normal((64, 96)).astype(np.float32)
    to_bits = lambda a: (a.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ref = to_bits(ref32)
    got = ref.copy()
    got[5] = to_bits(bits_f64(ref[5]) * 1.02)  # one row off by 2% (a moved code's worth)
    marked = np.zeros(64, bool)
    marked[5] = True
    chain_close(got, ref, "planted row, marked", accum=1, moved=marked)
    chain_close(got, ref, "planted row, fast mode", accum=0)
    with pytest.raises(AssertionError):
        chain_close(got, ref, "planted row, unmarked", accum=1)
    with pytest.raises(AssertionError):
        chain_close(got, ref, "planted row, another row marked", accum=1, moved=np.roll(marked, 1))
    wide = ref.copy()
    wide[:] = to_bits(bits_f64(ref) * 1.05)  # every row off: the Frobenius bar fails
    with pytest.raises(AssertionError):
        chain_close(wide, ref, "every row off", accum=1, moved=np.ones(64, bool))
