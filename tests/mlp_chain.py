"""Oracle stage values of the relu^2 MLP block on sampled rows and columns,
and their comparison with the GPU's stages.

Every expected value here is the oracle applied to the seeded bf16 inputs.
Two scales of the block are maxima over whole intermediate tensors (amax of
A = relu(H)^2 and of dH); they come from the full oracle chain, computed in
the test for small blocks and stored by tests/golden/make_block_scales.py
for the full-size ones.  Given those, every stage value on a sampled token
row or hidden column is a short oracle computation:

  rows r:    H[r], Aq[r], Y[r], dA[r] -> dH[r], Hq[r], dX[r]
  columns j: H[:, j] and dA[:, j] (as transposed products, same sums in the
             same order), Aq[:, j], Hq[:, j], dW_up[j, :], dW_down[:, j].

Comparison: a GPU stage is held to the strict bar (bit-exact for codes, the
GEMM bound for GEMM outputs) wherever its own inputs equal the oracle's bit
for bit; everywhere it is held to the chain bar (relative Frobenius error
<= 1e-2), since a one-ulp difference in H or dH may move an FP8 code by a
whole step."""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np

import oracle
from tests.gpu_util import bits_f64, gemm_bound, gemm_close, oracle_gemm, ulp_bf16

E4, E5 = oracle.E4M3, oracle.E5M2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "block_scales.json")


def f32_from_hex(s: str) -> float:
    return float(np.array([int(s, 16)], dtype=np.uint32).view(np.float32)[0])


def golden_scales(name: str, tensors) -> dict:
    """Stored oracle scales of a full-size block; checks that they were made
    from the same input bytes."""
    data = json.load(open(GOLDEN))[name]
    h = hashlib.sha256()
    for t in tensors:
        h.update(np.ascontiguousarray(t).tobytes())
    assert h.hexdigest() == data["inputs_sha256"], (
        f"{name}: inputs changed since block_scales.json was written; rerun tests/golden/make_block_scales.py")
    return {k: f32_from_hex(v["f32"]) for k, v in data.items() if isinstance(v, dict)}


def full_chain_scales(x, wu, wd, dy) -> tuple[dict, dict, dict]:
    """Full oracle chain (small blocks): (scales, forward stages, backward stages)."""
    f = oracle.mlp_fwd(x, wu, wd)
    b = oracle.mlp_bwd(dy, f)
    sc = dict(sx=f["sx"], su=f["su"], sd=f["sd"], sg=b["sg"], amax_a=f["amax_a"], sa=f["sa"],
              amax_dh=b["amax_dh"], sh=b["sh"])
    return sc, f, b


def sampled_chain(x, wu, wd, dy, sc: dict, rows, cols) -> dict:
    """Oracle stage values on token rows `rows` and hidden columns `cols`,
    plus the GEMMs on sign-cleared codes that the GEMM bound needs."""
    xq, sx, _ = oracle.quant(x, E4)
    uq, su, _ = oracle.quant(wu, E4)
    dq, sd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    for k, v in (("sx", sx), ("su", su), ("sd", sd), ("sg", sg)):
        assert np.float32(v) == np.float32(sc[k]), k
    sa, sh = sc["sa"], sc["sh"]
    o = dict(xq=xq, uq=uq, dq=dq, gq=gq)
    o["H_r"], o["H_r_abs"], _ = oracle_gemm("nt", xq, E4, sx, uq, E4, su, rows=rows)
    o["Aq_r"] = oracle.cast(oracle.relu2(o["H_r"]), sa, E4)
    o["Y_r"], o["Y_r_abs"], o["Y_K"] = oracle_gemm("nt", o["Aq_r"], E4, sa, dq, E4, sd)
    o["dA_r"], o["dA_r_abs"], o["dA_K"] = oracle_gemm("nn", gq, E5, sg, dq, E4, sd, rows=rows)
    o["dH_r"] = oracle.relu2_bwd(o["H_r"], o["dA_r"])
    o["Hq_r"] = oracle.cast(o["dH_r"], sh, E5)
    o["dX_r"], o["dX_r_abs"], o["dX_K"] = oracle_gemm("nn", o["Hq_r"], E5, sh, uq, E4, su)
    # columns: H[:, j] = (Uq Xq^T)[j, :] and dA[:, j] = (Dq^T Gq^T)[j, :]
    o["Ht_c"], o["Ht_c_abs"], _ = oracle_gemm("nt", uq, E4, su, xq, E4, sx, rows=cols)
    o["dAt_c"] = oracle.gemm_tn(dq, E4, sd, np.ascontiguousarray(gq.T), E5, sg, rows=cols)
    o["Aqt_c"] = oracle.cast(oracle.relu2(o["Ht_c"]), sa, E4)
    o["Hqt_c"] = oracle.cast(oracle.relu2_bwd(o["Ht_c"], o["dAt_c"]), sh, E5)
    o["dWup_c"], o["dWup_c_abs"], o["dWup_K"] = oracle_gemm(
        "tn", np.ascontiguousarray(o["Hqt_c"].T), E5, sh, xq, E4, sx)
    o["dWdnT_c"], o["dWdnT_c_abs"], o["dWdn_K"] = oracle_gemm(
        "tn", np.ascontiguousarray(o["Aqt_c"].T), E4, sa, gq, E5, sg)
    return o


def chain_close(got, ref, what):
    """Chain bar: relative Frobenius error <= 1e-2.  When a fraction f of an
    operand's FP8 codes sits one step (relative size delta <= 1/4 for E5M2)
    away from the oracle's, the output moves by about sqrt(f) * delta / 2
    of its norm for sums of random-sign products: 1e-2 covers f up to 2.5%
    (measured f <= 1.6%, errors 0.05-0.4%).  Max-relative error and the
    one-ulp fraction are printed, not required: with K = 12288 every output
    row has a few moved codes, and only 85% of dX stays within one ulp."""
    gv, rv = bits_f64(got), bits_f64(ref)
    err = np.abs(gv - rv)
    fro = np.linalg.norm(gv - rv) / max(np.linalg.norm(rv), 1e-300)
    frac = float((err <= ulp_bf16(rv)).mean())
    mrel = err.max() / max(np.abs(rv).max(), 1e-300)
    print(f"[chain] {what}: rel fro {fro:.3g}, max rel {mrel:.3g}, within 1 ulp {frac:.5f}")
    assert fro <= 1e-2, (what, fro, mrel, frac)


def _strict_rows(got, ref, ref_abs, K, same_rows, what):
    """GEMM bound on the rows whose operand row equals the oracle's."""
    n = int(same_rows.sum())
    print(f"[stage] {what}: {n}/{same_rows.size} rows with identical FP8 operands")
    if n:
        gemm_close(got[same_rows], ref[same_rows], what, sabs_bits=ref_abs[same_rows], K=K)
    chain_close(got, ref, what)


def _codes_equal_where(got, ref, inputs_same, what, min_frac=0.9):
    frac = float(inputs_same.mean())
    bad = int((got[inputs_same] != ref[inputs_same]).sum())
    print(f"[stage] {what}: inputs identical on {frac:.5f}, code mismatches there: {bad}")
    assert bad == 0, what
    assert frac >= min_frac, (what, frac)


def compare_block(g: dict, o: dict, sc: dict, rows, cols):
    """Compare the GPU's block outputs `g` (as collected by the MLP tests)
    with the oracle's sampled stages `o`."""
    sx, su, sd, sa = (float(v) for v in g["scales"])
    sg, sh = (float(v) for v in g["bsc"])
    for name, got, want in (("sx", sx, sc["sx"]), ("su", su, sc["su"]), ("sd", sd, sc["sd"]),
                            ("sa", sa, sc["sa"]), ("sg", sg, sc["sg"]), ("sh", sh, sc["sh"])):
        assert np.float32(got) == np.float32(want), (name, got, want)
    for name, q, qt in (("Xq", "xq", "xq_t"), ("Uq", "uq", "uq_t"), ("Dq", "dq", "dq_t"), ("Gq", "gq", "gq_t")):
        assert (g[q] == o[q]).all(), name
        if qt in g:
            assert (g[qt] == o[q].T).all(), name + "^T"
    # forward, token rows
    gemm_close(g["h"][rows], o["H_r"], "H rows", sabs_bits=o["H_r_abs"], K=o["xq"].shape[1])
    h_same = g["h"][rows] == o["H_r"]
    _codes_equal_where(g["aq"][rows], o["Aq_r"], h_same, "Aq rows")
    _strict_rows(g["y"][rows], o["Y_r"], o["Y_r_abs"], o["Y_K"], (g["aq"][rows] == o["Aq_r"]).all(1), "Y rows")
    # backward, token rows: dH = RN_bf16(2 relu(H) dA) with dA within the GEMM bound
    two_r = 2 * np.maximum(bits_f64(o["H_r"]), 0.0)
    bound = 1.5 * ulp_bf16(bits_f64(o["dH_r"])) + (1 + 2.0 ** -8) * two_r * gemm_bound(
        o["dA_r"], o["dA_r_abs"], o["dA_K"])
    dh = g["dh"][rows]
    err = np.abs(bits_f64(dh) - bits_f64(o["dH_r"]))
    assert not (err > bound)[h_same].any(), "dH rows beyond the bound where H is identical"
    chain_close(dh, o["dH_r"], "dH rows")
    _codes_equal_where(g["hq"][rows], o["Hq_r"], dh == o["dH_r"], "Hq rows")
    _strict_rows(g["dx"][rows], o["dX_r"], o["dX_r_abs"], o["dX_K"], (g["hq"][rows] == o["Hq_r"]).all(1),
                 "dX rows")
    # hidden columns
    ht = g["h"][:, cols].T
    gemm_close(ht, o["Ht_c"], "H columns", sabs_bits=o["Ht_c_abs"], K=o["xq"].shape[1])
    _codes_equal_where(g["aq_t"][cols], o["Aqt_c"], ht == o["Ht_c"], "Aq columns")
    dht = g["dh"][:, cols].T
    chain_close(dht, oracle.relu2_bwd(o["Ht_c"], o["dAt_c"]), "dH columns")
    _codes_equal_where(g["hq_t"][cols], o["Hqt_c"], dht == oracle.relu2_bwd(o["Ht_c"], o["dAt_c"]), "Hq columns")
    _strict_rows(g["dw_up"][cols], o["dWup_c"], o["dWup_c_abs"], o["dWup_K"],
                 (g["hq_t"][cols] == o["Hqt_c"]).all(1), "dW_up rows")
    _strict_rows(np.ascontiguousarray(g["dw_down"][:, cols].T), o["dWdnT_c"], o["dWdnT_c_abs"], o["dWdn_K"],
                 (g["aq_t"][cols] == o["Aqt_c"]).all(1), "dW_down columns")
