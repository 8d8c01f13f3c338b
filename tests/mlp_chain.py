"""Oracle stage values of the relu^2 MLP block on sampled rows and columns,
and their comparison with the GPU's stages.

Every expected value here is the oracle applied to seeded bf16 inputs or to
the GPU's own FP8 operands.  Two scales of the block are maxima over whole
intermediate tensors (amax of A = relu(H)^2 and of dH); they come from the
full oracle chain, computed in the test for small blocks and stored by
tests/golden/make_block_scales.py for the full-size ones.

Three levels of comparison:

* Stage parity, given the GPU's own stage inputs: every GEMM output against
  the oracle GEMM of the GPU's own FP8 operands and scales (the GEMM bar of
  the accumulation mode: in exact mode max|gpu - oracle| / max|oracle| <=
  5e-3 with >= 99.9% of the elements within one bf16 ulp), every cast
  (Aq from H, Hq from dH) bit-exact against the oracle's cast of the GPU's
  own bf16 input, dH within the bound its dA GEMM implies.
* Chain parity of the codes: wherever a cast's input equals the oracle
  chain's bit for bit, its codes equal the oracle chain's.
* End to end, against the oracle chain run from the same bf16 inputs: a
  one-ulp difference in H or dH can move an FP8 code by a whole step, and
  such codes propagate into the later GEMMs.  Exact mode: max-relative error
  <= 5e-3.  Both modes: relative Frobenius error <= 1e-2; the number of
  output rows whose operands hold a moved code is reported.

  rows r:    H[r], Aq[r], Y[r], dA[r] -> dH[r], Hq[r], dX[r]
  columns j: H[:, j] and dA[:, j] (as transposed products, same sums in the
             same order), Aq[:, j], Hq[:, j], dW_up[j, :], dW_down[:, j]."""
from __future__ import annotations

import hashlib
import json
import os

import numpy as np

import oracle
from tests.gpu_util import (ACC_EXACT, ACC_FAST, STRICT_MAX_REL, bits_f64, gemm_bound, gemm_close, gemm_stats,
                            oracle_gemm, ulp_bf16)

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
    """Oracle chain stage values on token rows `rows` and hidden columns
    `cols` (from the bf16 inputs and the chain's tensor-wide scales)."""
    xq, sx, _ = oracle.quant(x, E4)
    uq, su, _ = oracle.quant(wu, E4)
    dq, sd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    for k, v in (("sx", sx), ("su", su), ("sd", sd), ("sg", sg)):
        assert np.float32(v) == np.float32(sc[k]), k
    sa, sh = sc["sa"], sc["sh"]
    o = dict(xq=xq, uq=uq, dq=dq, gq=gq)
    o["H_r"] = oracle.gemm_nt(xq, E4, sx, uq, E4, su, rows=rows)
    o["Aq_r"] = oracle.cast(oracle.relu2(o["H_r"]), sa, E4)
    o["Y_r"] = oracle.gemm_nt(o["Aq_r"], E4, sa, dq, E4, sd)
    o["dA_r"], o["dA_r_abs"], o["dA_K"] = oracle_gemm("nn", gq, E5, sg, dq, E4, sd, rows=rows)
    o["dH_r"] = oracle.relu2_bwd(o["H_r"], o["dA_r"])
    o["Hq_r"] = oracle.cast(o["dH_r"], sh, E5)
    o["dX_r"] = oracle.gemm_nn(o["Hq_r"], E5, sh, uq, E4, su)
    # columns: H[:, j] = (Uq Xq^T)[j, :] and dA[:, j] = (Dq^T Gq^T)[j, :]
    o["Ht_c"] = oracle.gemm_nt(uq, E4, su, xq, E4, sx, rows=cols)
    o["dAt_c"], o["dAt_c_abs"], _ = oracle_gemm("tn", dq, E4, sd, np.ascontiguousarray(gq.T), E5, sg, rows=cols)
    o["Aqt_c"] = oracle.cast(oracle.relu2(o["Ht_c"]), sa, E4)
    o["dHt_c"] = oracle.relu2_bwd(o["Ht_c"], o["dAt_c"])
    o["Hqt_c"] = oracle.cast(o["dHt_c"], sh, E5)
    o["dWup_c"] = oracle.gemm_tn(np.ascontiguousarray(o["Hqt_c"].T), E5, sh, xq, E4, sx)
    o["dWdnT_c"] = oracle.gemm_tn(np.ascontiguousarray(o["Aqt_c"].T), E4, sa, gq, E5, sg)
    return o


def chain_close(got, ref, what, accum=ACC_FAST, moved=None):
    """End-to-end bar against the oracle chain.  Both modes: relative
    Frobenius error <= 1e-2.  When a fraction f of an operand's FP8 codes sits
    one step (relative size delta <= 1/4 for E5M2) away from the oracle's,
    the output moves by about sqrt(f) * delta / 2 of its norm for sums of
    random-sign products: 1e-2 covers f up to 2.5%.  Exact mode also:
    max|gpu - oracle| / max|oracle| <= 5e-3 (the strict bar) over the output
    rows whose operand row holds the oracle chain's codes.  (The GEMM before
    a cast may differ from the oracle by one bf16 ulp, within that GEMM's
    bar; at a rounding boundary of the cast this moves a code by a whole
    FP8 step, and the output row that sums it is off by that step times its
    partner, which no relative bar on the row bounds.)  `moved`: boolean
    per output row, True where its operand row holds a code that differs
    from the oracle chain's."""
    gv, rv = bits_f64(got), bits_f64(ref)
    err = np.abs(gv - rv)
    fro = np.linalg.norm(gv - rv) / max(np.linalg.norm(rv), 1e-300)
    frac = float((err <= ulp_bf16(rv)).mean())
    mrel = err.max() / max(np.abs(rv).max(), 1e-300)
    keep = np.ones(gv.shape[0], bool) if moved is None else ~np.asarray(moved)
    mrel_keep = err[keep].max() / max(np.abs(rv[keep]).max(), 1e-300) if keep.any() else 0.0
    extra = "" if moved is None else (f", rows downstream of a moved code {int((~keep).sum())}/{keep.size}"
                                      f", max rel on the others {mrel_keep:.3g}")
    print(f"[chain] {what} ({'exact' if accum == ACC_EXACT else 'fast'}): rel fro {fro:.3g}, max rel {mrel:.3g}, "
          f"within 1 ulp {frac:.5f}{extra}")
    assert fro <= 1e-2, (what, fro, mrel, frac)
    if accum == ACC_EXACT:
        assert mrel_keep <= STRICT_MAX_REL, (what, "max rel on rows with the oracle chain's codes", mrel_keep)


def stage_gemm(got, kind, a, fa, sa, b, fb, sb, what, accum, rows=None):
    """A GEMM stage against the oracle GEMM of the GPU's own operands."""
    ref, sabs, K = oracle_gemm(kind, a, fa, sa, b, fb, sb, rows=rows)
    gemm_close(got, ref, what, sabs_bits=sabs, K=K, accum=accum)


def _codes_equal_where(got, ref, inputs_same, what, min_frac=0.9):
    frac = float(inputs_same.mean())
    bad = int((got[inputs_same] != ref[inputs_same]).sum())
    print(f"[stage] {what}: inputs identical to the oracle chain's on {frac:.5f}, code mismatches there: {bad}")
    assert bad == 0, what
    assert frac >= min_frac, (what, frac)


def _relu2_bwd_close(got_dh, h_bits, da_ref, da_abs, K, accum, what):
    """dH = RN_bf16(2 relu(H) dA) with dA within its GEMM bound: given the
    GPU's own H, |dH_gpu - dH(H, dA_oracle)| <= 1.5 ulp + (1 + 2^-8) 2 relu(H)
    * bound(dA)."""
    two_r = 2 * np.maximum(bits_f64(h_bits), 0.0)
    ref = oracle.relu2_bwd(h_bits, da_ref)
    bound = 1.5 * ulp_bf16(bits_f64(ref)) + (1 + 2.0 ** -8) * two_r * gemm_bound(da_ref, da_abs, K, accum)
    err = np.abs(bits_f64(got_dh) - bits_f64(ref))
    rel, within = gemm_stats(got_dh, ref)
    print(f"[stage] {what}: max_rel={rel:.3g} within1={within:.6f} max_err/bound={float((err / bound).max()):.3g}")
    assert not (err > bound).any(), f"{what}: {int((err > bound).sum())} beyond the bound"
    return ref


def compare_block(g: dict, o: dict, sc: dict, rows, cols, accum=ACC_FAST):
    """Compare the GPU's block pass `g` (tests/gpu_util.collect_block) with
    the oracle: stage parity on the GPU's own operands, code parity with the
    oracle chain `o` (sampled_chain) where inputs agree, end to end."""
    sx, su, sd, sa = (float(v) for v in g["scales"])
    sg, sh = (float(v) for v in g["bsc"])
    for name, got, want in (("sx", sx, sc["sx"]), ("su", su, sc["su"]), ("sd", sd, sc["sd"]),
                            ("sa", sa, sc["sa"]), ("sg", sg, sc["sg"]), ("sh", sh, sc["sh"])):
        assert np.float32(got) == np.float32(want), (name, got, want)
    for name, q in (("Xq", "xq"), ("Uq", "uq"), ("Dq", "dq"), ("Gq", "gq")):
        assert (g[q] == o[q]).all(), name
    xq, uq, dq, gq = o["xq"], o["uq"], o["dq"], o["gq"]
    h_r, aq_r, dh_r, hq_r = g["h"][rows], g["aq"][rows], g["dh"][rows], g["hq"][rows]
    h_c = np.ascontiguousarray(g["h"][:, cols].T)
    aq_c = np.ascontiguousarray(g["aq"][:, cols].T)
    dh_c = np.ascontiguousarray(g["dh"][:, cols].T)
    hq_c = np.ascontiguousarray(g["hq"][:, cols].T)

    # ---- stage parity on the GPU's own operands
    stage_gemm(h_r, "nt", xq, E4, sx, uq, E4, su, "H rows", accum, rows=rows)
    stage_gemm(h_c, "nt", uq, E4, su, xq, E4, sx, "H columns", accum, rows=cols)
    assert (aq_r == oracle.cast(oracle.relu2(h_r), sa, E4)).all(), "Aq rows: cast of the GPU's H"
    assert (aq_c == oracle.cast(oracle.relu2(h_c), sa, E4)).all(), "Aq columns: cast of the GPU's H"
    stage_gemm(g["y"][rows], "nt", aq_r, E4, sa, dq, E4, sd, "Y rows", accum)
    _relu2_bwd_close(dh_r, h_r, o["dA_r"], o["dA_r_abs"], o["dA_K"], accum, "dH rows")
    _relu2_bwd_close(dh_c, h_c, o["dAt_c"], o["dAt_c_abs"], o["dA_K"], accum, "dH columns")
    assert (hq_r == oracle.cast(dh_r, sh, E5)).all(), "Hq rows: cast of the GPU's dH"
    assert (hq_c == oracle.cast(dh_c, sh, E5)).all(), "Hq columns: cast of the GPU's dH"
    stage_gemm(g["dx"][rows], "nn", hq_r, E5, sh, uq, E4, su, "dX rows", accum)
    stage_gemm(g["dw_up"][cols], "tn", np.ascontiguousarray(g["hq"][:, cols]), E5, sh, xq, E4, sx, "dW_up rows", accum)
    stage_gemm(np.ascontiguousarray(g["dw_down"][:, cols].T), "tn", np.ascontiguousarray(g["aq"][:, cols]), E4, sa,
               gq, E5, sg, "dW_down columns", accum)

    # ---- code parity with the oracle chain where the cast's input agrees
    _codes_equal_where(aq_r, o["Aq_r"], h_r == o["H_r"], "Aq rows")
    _codes_equal_where(aq_c, o["Aqt_c"], h_c == o["Ht_c"], "Aq columns")
    _codes_equal_where(hq_r, o["Hq_r"], dh_r == o["dH_r"], "Hq rows")
    _codes_equal_where(hq_c, o["Hqt_c"], dh_c == o["dHt_c"], "Hq columns")

    # ---- end to end against the oracle chain
    moved = lambda q, r: (q != r).any(1)
    chain_close(g["y"][rows], o["Y_r"], "Y rows", accum, moved(aq_r, o["Aq_r"]))
    chain_close(g["dx"][rows], o["dX_r"], "dX rows", accum, moved(hq_r, o["Hq_r"]))
    chain_close(g["dw_up"][cols], o["dWup_c"], "dW_up rows", accum, moved(hq_c, o["Hqt_c"]))
    chain_close(np.ascontiguousarray(g["dw_down"][:, cols].T), o["dWdnT_c"], "dW_down columns", accum,
                moved(aq_c, o["Aqt_c"]))
