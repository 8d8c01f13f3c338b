"""Oracle stage values of the gated (SwiGLU) MLP block on sampled token rows
and hidden columns, and their comparison with the GPU's stages.

Every expected value is the oracle applied to the seeded bf16 inputs.  Three
scales of the block are maxima over whole intermediate tensors (amax of
A = silu(G) U, of dG and of dU); they come from the full oracle chain, run in
the test for small blocks and stored by tests/golden/make_block_scales.py for
the full-size one.  Given those, the stages on a token row r or a hidden
column j are short oracle computations:

  rows r:    G[r], U[r], A[r], Aq[r], Y[r], dA[r] -> dG[r], dU[r], their
             codes, dX[r] (the two dgrad products summed before rounding)
  columns j: G[:, j], U[:, j], dA[:, j] (transposed products: the same sums),
             A, Aq, dG, dU and their codes on column j, dW_gate[j, :],
             dW_up[j, :], dW_down[:, j].

Comparison as for the relu^2 block: strict (bit-exact codes, the GEMM bound,
the gate's own bound) wherever a stage's inputs equal the oracle's bit for
bit, and the chain bar everywhere."""
from __future__ import annotations

import numpy as np

import oracle
from tests.gpu_util import bf16_bits, bits_f64, f32, gemm_bound, gemm_close, oracle_gemm, u8, ulp_bf16
from tests.mlp_chain import _codes_equal_where, _strict_rows, chain_close

E4, E5 = oracle.E4M3, oracle.E5M2


def full_chain_scales(x, wg, wu, wd, dy):
    """Full oracle chain (small blocks): (scales, forward stages, backward stages)."""
    f = oracle.swiglu_fwd(x, wg, wu, wd)
    b = oracle.swiglu_bwd(dy, f)
    sc = dict(sx=f["sx"], swg=f["swg"], swu=f["swu"], swd=f["swd"], sa=f["sa"], sg=b["sg"], sdg=b["sdg"],
              sdu=b["sdu"])
    return sc, f, b


def _abs_acc_nn(pairs, rows_out, n):
    """Two-term dgrad sum of |products| (for the bound), rounded to bf16."""
    acc = np.zeros((rows_out, n))
    for a, fa, sa, b, fb, sb in pairs:
        oracle.gemm_nn_acc(a & np.uint8(0x7F), fa, sa, b & np.uint8(0x7F), fb, sb, acc)
    return oracle.double_to_bf16(acc)


def sampled_chain(x, wg, wu, wd, dy, sc: dict, rows, cols) -> dict:
    xq, sx, _ = oracle.quant(x, E4)
    wgq, swg, _ = oracle.quant(wg, E4)
    wuq, swu, _ = oracle.quant(wu, E4)
    wdq, swd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    for k, v in (("sx", sx), ("swg", swg), ("swu", swu), ("swd", swd), ("sg", sg)):
        assert np.float32(v) == np.float32(sc[k]), k
    sa, sdg, sdu = sc["sa"], sc["sdg"], sc["sdu"]
    o = dict(xq=xq, wgq=wgq, wuq=wuq, wdq=wdq, gq=gq)
    # token rows
    o["G_r"], o["G_r_abs"], _ = oracle_gemm("nt", xq, E4, sx, wgq, E4, swg, rows=rows)
    o["U_r"], o["U_r_abs"], _ = oracle_gemm("nt", xq, E4, sx, wuq, E4, swu, rows=rows)
    o["A_r"] = oracle.swiglu_gate(o["G_r"], o["U_r"])
    o["Aq_r"] = oracle.cast(o["A_r"], sa, E4)
    o["Y_r"], o["Y_r_abs"], o["Y_K"] = oracle_gemm("nt", o["Aq_r"], E4, sa, wdq, E4, swd)
    o["dA_r"], o["dA_r_abs"], o["dA_K"] = oracle_gemm("nn", gq, E5, sg, wdq, E4, swd, rows=rows)
    o["dG_r"], o["dU_r"] = oracle.swiglu_gate_bwd(o["G_r"], o["U_r"], o["dA_r"])
    o["dGq_r"] = oracle.cast(o["dG_r"], sdg, E5)
    o["dUq_r"] = oracle.cast(o["dU_r"], sdu, E5)
    acc = np.zeros((len(rows), xq.shape[1]))
    oracle.gemm_nn_acc(o["dGq_r"], E5, sdg, wgq, E4, swg, acc)
    oracle.gemm_nn_acc(o["dUq_r"], E5, sdu, wuq, E4, swu, acc)
    o["dX_r"] = oracle.double_to_bf16(acc)
    o["dX_r_abs"] = _abs_acc_nn([(o["dGq_r"], E5, sdg, wgq, E4, swg), (o["dUq_r"], E5, sdu, wuq, E4, swu)],
                                len(rows), xq.shape[1])
    # hidden columns: G[:, j] = (Wgq Xq^T)[j, :], dA[:, j] = (Wdq^T Gq^T)[j, :]
    o["Gt_c"], o["Gt_c_abs"], _ = oracle_gemm("nt", wgq, E4, swg, xq, E4, sx, rows=cols)
    o["Ut_c"], o["Ut_c_abs"], _ = oracle_gemm("nt", wuq, E4, swu, xq, E4, sx, rows=cols)
    gqt = np.ascontiguousarray(gq.T)
    o["dAt_c"], o["dAt_c_abs"], _ = oracle_gemm("tn", wdq, E4, swd, gqt, E5, sg, rows=cols)
    o["At_c"] = oracle.swiglu_gate(o["Gt_c"], o["Ut_c"])
    o["Aqt_c"] = oracle.cast(o["At_c"], sa, E4)
    o["dGt_c"], o["dUt_c"] = oracle.swiglu_gate_bwd(o["Gt_c"], o["Ut_c"], o["dAt_c"])
    o["dGqt_c"] = oracle.cast(o["dGt_c"], sdg, E5)
    o["dUqt_c"] = oracle.cast(o["dUt_c"], sdu, E5)
    o["dWg_c"], o["dWg_c_abs"], o["dW_K"] = oracle_gemm("tn", np.ascontiguousarray(o["dGqt_c"].T), E5, sdg, xq,
                                                        E4, sx)
    o["dWu_c"], o["dWu_c_abs"], _ = oracle_gemm("tn", np.ascontiguousarray(o["dUqt_c"].T), E5, sdu, xq, E4, sx)
    o["dWdT_c"], o["dWdT_c_abs"], _ = oracle_gemm("tn", np.ascontiguousarray(o["Aqt_c"].T), E4, sa, gq, E5, sg)
    return o


def collect(inputs, y, saved, ws_f, ws_b, dx, dwg, dwu, dwd, bsc) -> dict:
    """Host copies of one gated block pass: inputs, outputs, saved forward
    quantities and the workspace intermediates."""
    from fp8_tensorwise_scaled_amd import api

    x, wg, wu, wd, dy = inputs
    M, d = x.shape
    h = wg.shape[0]
    of = api.swiglu_workspace_layout("fwd", M, d, h)
    ob = api.swiglu_workspace_layout("bwd", M, d, h)
    wf, wb = ws_f.cpu().numpy(), ws_b.cpu().numpy()

    def sl(buf, o, shape, bf16=False):
        n = int(np.prod(shape)) * (2 if bf16 else 1)
        v = buf[o:o + n]
        return (v.view(np.uint16) if bf16 else v).reshape(shape)

    return dict(
        x=x, wg=wg, wu=wu, wd=wd, dy=dy, y=bf16_bits(y), dx=bf16_bits(dx), dw_gate=bf16_bits(dwg),
        dw_up=bf16_bits(dwu), dw_down=bf16_bits(dwd), g=bf16_bits(saved.g), u=bf16_bits(saved.u),
        scales=f32(saved.scales), bsc=f32(bsc), xq_t=u8(saved.xq_t), wgq_t=u8(saved.wgq_t),
        wuq_t=u8(saved.wuq_t), wdq_t=u8(saved.wdq_t), aq_t=u8(saved.aq_t),
        xq=sl(wf, of[0], (M, d)), wgq=sl(wf, of[1], (h, d)), wuq=sl(wf, of[2], (h, d)), wdq=sl(wf, of[3], (d, h)),
        a=sl(wf, of[4], (M, h), True), aq=sl(wf, of[5], (M, h)),
        gq=sl(wb, ob[0], (M, d)), gq_t=sl(wb, ob[1], (d, M)), da=sl(wb, ob[2], (M, h), True),
        dg=sl(wb, ob[3], (M, h), True), du=sl(wb, ob[4], (M, h), True), dgq=sl(wb, ob[5], (M, h)),
        dgq_t=sl(wb, ob[6], (h, M)), duq=sl(wb, ob[7], (M, h)), duq_t=sl(wb, ob[8], (h, M)))


def _silu_d(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def _gate_close(got, ref, same, what):
    """The gate evaluates in fp32 (exp, reciprocal, three products) where the
    oracle evaluates in fp64: relative differences of a few 2^-24 before the
    bf16 rounding, so at most one bf16 ulp, and only for values that lie that
    close to a rounding boundary."""
    err = np.abs(bits_f64(got) - bits_f64(ref))
    ok = err <= ulp_bf16(bits_f64(ref))
    eq = float((got == ref)[same].mean()) if same.any() else 1.0
    print(f"[stage] {what}: inputs identical on {float(same.mean()):.5f}, equal there {eq:.6f}")
    assert ok[same].all(), what
    assert eq >= 0.999, (what, eq)
    chain_close(got, ref, what)


def _gate_bwd_close(dg, du, ref_dg, ref_du, g_ref, u_ref, da_ref, da_ref_abs, K, gu_same, what):
    """dG = RN(dA U silu'(G)), dU = RN(dA silu(G)) with G, U identical and dA
    within the GEMM bound D: the results differ by at most the factor times
    D (1 + 2^-8) plus 1.5 ulp (two roundings and the fp32 evaluation)."""
    gv, uv = bits_f64(g_ref), bits_f64(u_ref)
    D = gemm_bound(da_ref, da_ref_abs, K)
    for name, got, ref, fac in (("dG", dg, ref_dg, np.abs(uv * _silu_d(gv))),
                                ("dU", du, ref_du, np.abs(gv / (1.0 + np.exp(-gv))))):
        bound = 1.5 * ulp_bf16(bits_f64(ref)) + (1 + 2.0 ** -8) * fac * D
        err = np.abs(bits_f64(got) - bits_f64(ref))
        assert not (err > bound)[gu_same].any(), f"{name} {what} beyond the bound where G, U are identical"
        chain_close(got, ref, f"{name} {what}")


def compare(g: dict, o: dict, sc: dict, rows, cols):
    sx, swg, swu, swd, sa = (float(v) for v in g["scales"])
    sg, sdg, sdu = (float(v) for v in g["bsc"])
    for name, got in (("sx", sx), ("swg", swg), ("swu", swu), ("swd", swd), ("sa", sa), ("sg", sg),
                      ("sdg", sdg), ("sdu", sdu)):
        assert np.float32(got) == np.float32(sc[name]), (name, got, sc[name])
    for name, q, qt in (("Xq", "xq", "xq_t"), ("Wgq", "wgq", "wgq_t"), ("Wuq", "wuq", "wuq_t"),
                        ("Wdq", "wdq", "wdq_t"), ("Gq", "gq", "gq_t")):
        assert (g[q] == o[q]).all(), name
        assert (g[qt] == o[q].T).all(), name + "^T"
    d = o["xq"].shape[1]
    h = o["wgq"].shape[0]
    # forward, token rows
    gemm_close(g["g"][rows], o["G_r"], "G rows", sabs_bits=o["G_r_abs"], K=d)
    gemm_close(g["u"][rows], o["U_r"], "U rows", sabs_bits=o["U_r_abs"], K=d)
    gu_same = (g["g"][rows] == o["G_r"]) & (g["u"][rows] == o["U_r"])
    _gate_close(g["a"][rows], o["A_r"], gu_same, "A rows")
    _codes_equal_where(g["aq"][rows], o["Aq_r"], g["a"][rows] == o["A_r"], "Aq rows")
    _strict_rows(g["y"][rows], o["Y_r"], o["Y_r_abs"], o["Y_K"], (g["aq"][rows] == o["Aq_r"]).all(1), "Y rows")
    # backward, token rows
    gemm_close(g["da"][rows], o["dA_r"], "dA rows", sabs_bits=o["dA_r_abs"], K=o["dA_K"])
    _gate_bwd_close(g["dg"][rows], g["du"][rows], o["dG_r"], o["dU_r"], o["G_r"], o["U_r"], o["dA_r"],
                    o["dA_r_abs"], o["dA_K"], gu_same, "rows")
    _codes_equal_where(g["dgq"][rows], o["dGq_r"], g["dg"][rows] == o["dG_r"], "dGq rows")
    _codes_equal_where(g["duq"][rows], o["dUq_r"], g["du"][rows] == o["dU_r"], "dUq rows")
    # dX sums two products before one rounding: one more fp32 rounding than a
    # single GEMM, covered by counting 64 more reduction steps in the bound
    same = (g["dgq"][rows] == o["dGq_r"]).all(1) & (g["duq"][rows] == o["dUq_r"]).all(1)
    _strict_rows(g["dx"][rows], o["dX_r"], o["dX_r_abs"], h + 64, same, "dX rows")
    # hidden columns
    gt, ut = g["g"][:, cols].T, g["u"][:, cols].T
    gemm_close(gt, o["Gt_c"], "G columns", sabs_bits=o["Gt_c_abs"], K=d)
    gemm_close(ut, o["Ut_c"], "U columns", sabs_bits=o["Ut_c_abs"], K=d)
    gu_c = (gt == o["Gt_c"]) & (ut == o["Ut_c"])
    at = g["a"][:, cols].T
    _gate_close(at, o["At_c"], gu_c, "A columns")
    _codes_equal_where(g["aq_t"][cols], o["Aqt_c"], at == o["At_c"], "Aq columns")
    dat = g["da"][:, cols].T
    gemm_close(dat, o["dAt_c"], "dA columns", sabs_bits=o["dAt_c_abs"], K=d)
    dgt, dut = g["dg"][:, cols].T, g["du"][:, cols].T
    _gate_bwd_close(dgt, dut, o["dGt_c"], o["dUt_c"], o["Gt_c"], o["Ut_c"], o["dAt_c"], o["dAt_c_abs"], d, gu_c,
                    "columns")
    _codes_equal_where(g["dgq_t"][cols], o["dGqt_c"], dgt == o["dGt_c"], "dGq columns")
    _codes_equal_where(g["duq_t"][cols], o["dUqt_c"], dut == o["dUt_c"], "dUq columns")
    _strict_rows(g["dw_gate"][cols], o["dWg_c"], o["dWg_c_abs"], o["dW_K"],
                 (g["dgq_t"][cols] == o["dGqt_c"]).all(1), "dW_gate rows")
    _strict_rows(g["dw_up"][cols], o["dWu_c"], o["dWu_c_abs"], o["dW_K"],
                 (g["duq_t"][cols] == o["dUqt_c"]).all(1), "dW_up rows")
    _strict_rows(np.ascontiguousarray(g["dw_down"][:, cols].T), o["dWdT_c"], o["dWdT_c_abs"], o["dW_K"],
                 (g["aq_t"][cols] == o["Aqt_c"]).all(1), "dW_down columns")
