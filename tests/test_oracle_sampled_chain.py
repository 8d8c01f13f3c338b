"""The sampled-stage oracle used by the full-size block tests reproduces the
full oracle chain bit for bit on its rows and columns (transposed products
sum the same exact products in the same order), so sampled checks at
M=8192 / 32768 carry the same expected values a full run would."""
import numpy as np

import oracle
from fp8_tensorwise_scaled_amd import synth
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
                xq_t=f["xq"].T, uq_t=f["uq"].T, dq_t=f["dq"].T, aq_t=f["aq"].T, gq=b["gq"], gq_t=b["gq"].T,
                dh=b["dh"], hq=b["hq"], hq_t=b["hq"].T)


def test_compare_block_accepts_the_oracle_and_rejects_a_planted_error():
    x, wu, wd, dy = _block()
    sc, f, b = full_chain_scales(x, wu, wd, dy)
    rows, cols = np.arange(192), np.arange(384)
    o = sampled_chain(x, wu, wd, dy, sc, rows, cols)
    g = _as_gpu_dict(x, wu, wd, dy, f, b)
    compare_block(g, o, sc, rows, cols)
    # one wrong A code where H is identical must fail
    bad = dict(g)
    bad["aq"] = g["aq"].copy()
    i = np.argwhere(g["aq"] != 0)[0]
    bad["aq"][tuple(i)] ^= 1
    try:
        compare_block(bad, o, sc, rows, cols)
    except AssertionError:
        pass
    else:
        raise AssertionError("a flipped A code went unnoticed")
