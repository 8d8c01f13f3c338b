"""Oracle stage values of the gated (SwiGLU) MLP block on sampled token rows
and hidden columns, and their comparison with the GPU's stages.

Every expected value is the oracle applied to the seeded bf16 inputs or to
the GPU's own stage inputs.  Three scales of the block are maxima over whole
intermediate tensors (amax of A = silu(G) U, of dG and of dU); they come from
the full oracle chain, run in the test for small blocks and stored by
tests/golden/make_block_scales.py for the full-size one.  Given those, the
stages on a token row r or a hidden column j are short oracle computations:

  rows r:    G[r], U[r], A[r], Aq[r], Y[r], dA[r] -> dG[r], dU[r], their
             codes, dX[r] (the two dgrad products summed before rounding)
  columns j: G[:, j], U[:, j], dA[:, j] (transposed products: the same sums),
             A, Aq, dG, dU and their codes on column j, dW_gate[j, :],
             dW_up[j, :], dW_down[:, j].

Comparison as for the relu^2 block (tests/mlp_chain.py): every GEMM stage
against the oracle GEMM of the GPU's own FP8 operands, every cast bit-exact
given its own bf16 input, the gate within the bound of its fp32 evaluation,
codes equal to the oracle chain's where their input agrees, the end-to-end
outputs against the oracle chain."""
from __future__ import annotations

import numpy as np

import oracle
from tests.gpu_util import (ACC_FAST, bf16_bits, bits_f64, f32, gemm_bound, gemm_close, oracle_gemm, u8,
                            ulp_bf16)
from tests.mlp_chain import _codes_equal_where, chain_close, stage_gemm

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
        scales=f32(saved.scales), bsc=f32(bsc), xq=u8(saved.xq), wgq=u8(saved.wgq), wuq=u8(saved.wuq),
        wdq=u8(saved.wdq), aq=u8(saved.aq), a=sl(wf, of[0], (M, h), True),
        gq=sl(wb, ob[0], (M, d)), dg=sl(wb, ob[1], (M, h), True), du=sl(wb, ob[2], (M, h), True),
        dgq=sl(wb, ob[3], (M, h)), duq=sl(wb, ob[4], (M, h)))


def _silu_d(g):
    s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def _gate_close(got, g_bits, u_bits, what):
    """A = RN_bf16(silu(G) U) given the GPU's own G and U: the gate evaluates
    in fp32 (exp, reciprocal, two products) where the oracle evaluates in
    fp64, relative differences of a few 2^-24 before the bf16 rounding, so at
    most one bf16 ulp, and only for values that lie that close to a rounding
    boundary."""
    ref = oracle.swiglu_gate(g_bits, u_bits)
    err = np.abs(bits_f64(got) - bits_f64(ref))
    eq = float((got == ref).mean())
    print(f"[stage] {what}: equal to the oracle's gate of the GPU's G, U on {eq:.6f}")
    assert (err <= ulp_bf16(bits_f64(ref))).all(), what
    assert eq >= 0.999, (what, eq)
    return ref


def _gate_bwd_close(dg, du, g_bits, u_bits, da_ref, da_abs, K, accum, what):
    """dG = RN(dA U silu'(G)), dU = RN(dA silu(G)) given the GPU's own G and
    U, with dA within its GEMM bound D: the results differ by at most the
    factor times D (1 + 2^-8), plus 1.5 ulp (two roundings), plus the fp32
    evaluation of the factor (exp and reciprocal within a few 2^-23 of
    sigmoid, then products and a sum whose terms stay below (1 + |g|)):
    |dA U| (1 + |g|) 2^-20 for dG, |dA g| 2^-20 for dU."""
    gv, uv, dav = bits_f64(g_bits), bits_f64(u_bits), bits_f64(da_ref)
    ref_dg, ref_du = oracle.swiglu_gate_bwd(g_bits, u_bits, da_ref)
    D = gemm_bound(da_ref, da_abs, K, accum)
    for name, got, ref, fac, ev in (("dG", dg, ref_dg, np.abs(uv * _silu_d(gv)), np.abs(dav * uv) * (1 + np.abs(gv))),
                                    ("dU", du, ref_du, np.abs(gv / (1.0 + np.exp(-gv))), np.abs(dav * gv))):
        bound = 1.5 * ulp_bf16(bits_f64(ref)) + (1 + 2.0 ** -8) * fac * D + ev * 2.0 ** -20
        err = np.abs(bits_f64(got) - bits_f64(ref))
        print(f"[stage] {name} {what}: max_err/bound={float((err / bound).max()):.3g}")
        assert not (err > bound).any(), f"{name} {what}: {int((err > bound).sum())} beyond the bound"
    return ref_dg, ref_du


def _dx_oracle(dgq, sdg, duq, sdu, wgq, swg, wuq, swu):
    """The two-term dgrad sum of the given codes and its sum of |products|."""
    acc = np.zeros((dgq.shape[0], wgq.shape[1]))
    oracle.gemm_nn_acc(dgq, E5, sdg, wgq, E4, swg, acc)
    oracle.gemm_nn_acc(duq, E5, sdu, wuq, E4, swu, acc)
    return oracle.double_to_bf16(acc), _abs_acc_nn([(dgq, E5, sdg, wgq, E4, swg), (duq, E5, sdu, wuq, E4, swu)],
                                                   dgq.shape[0], wgq.shape[1])


def compare(g: dict, o: dict, sc: dict, rows, cols, accum=ACC_FAST):
    sx, swg, swu, swd, sa = (float(v) for v in g["scales"])
    sg, sdg, sdu = (float(v) for v in g["bsc"])
    for name, got in (("sx", sx), ("swg", swg), ("swu", swu), ("swd", swd), ("sa", sa), ("sg", sg),
                      ("sdg", sdg), ("sdu", sdu)):
        assert np.float32(got) == np.float32(sc[name]), (name, got, sc[name])
    for name, q in (("Xq", "xq"), ("Wgq", "wgq"), ("Wuq", "wuq"), ("Wdq", "wdq"), ("Gq", "gq")):
        assert (g[q] == o[q]).all(), name
    xq, wgq, wuq, wdq, gq = o["xq"], o["wgq"], o["wuq"], o["wdq"], o["gq"]
    d = xq.shape[1]
    h = wgq.shape[0]
    T = lambda a: np.ascontiguousarray(a[:, cols].T)
    g_r, u_r, a_r, aq_r = g["g"][rows], g["u"][rows], g["a"][rows], g["aq"][rows]
    g_c, u_c, a_c, aq_c = T(g["g"]), T(g["u"]), T(g["a"]), T(g["aq"])
    dg_r, du_r, dgq_r, duq_r = g["dg"][rows], g["du"][rows], g["dgq"][rows], g["duq"][rows]
    dg_c, du_c, dgq_c, duq_c = T(g["dg"]), T(g["du"]), T(g["dgq"]), T(g["duq"])

    # ---- stage parity on the GPU's own operands
    stage_gemm(g_r, "nt", xq, E4, sx, wgq, E4, swg, "G rows", accum, rows=rows)
    stage_gemm(u_r, "nt", xq, E4, sx, wuq, E4, swu, "U rows", accum, rows=rows)
    stage_gemm(g_c, "nt", wgq, E4, swg, xq, E4, sx, "G columns", accum, rows=cols)
    stage_gemm(u_c, "nt", wuq, E4, swu, xq, E4, sx, "U columns", accum, rows=cols)
    _gate_close(a_r, g_r, u_r, "A rows")
    _gate_close(a_c, g_c, u_c, "A columns")
    assert (aq_r == oracle.cast(a_r, sa, E4)).all() and (aq_c == oracle.cast(a_c, sa, E4)).all(), "Aq: cast of A"
    stage_gemm(g["y"][rows], "nt", aq_r, E4, sa, wdq, E4, swd, "Y rows", accum)
    # dA lives only inside the grad-input GEMM's epilogue: dG and dU are held
    # to the oracle's gate derivative of the oracle's dA (same Gq and Wdq
    # codes), within dA's GEMM bound carried through the derivative
    _gate_bwd_close(dg_r, du_r, g_r, u_r, o["dA_r"], o["dA_r_abs"], o["dA_K"], accum, "rows")
    _gate_bwd_close(dg_c, du_c, g_c, u_c, o["dAt_c"], o["dAt_c_abs"], d, accum, "columns")
    for name, q, v, s in (("dGq rows", dgq_r, dg_r, sdg), ("dUq rows", duq_r, du_r, sdu),
                          ("dGq columns", dgq_c, dg_c, sdg), ("dUq columns", duq_c, du_c, sdu)):
        assert (q == oracle.cast(v, s, E5)).all(), name + ": cast of the GPU's gradient"
    # dX sums two products before one rounding.  The library accumulates
    # both in one fp32 accumulator (the first scaled by RN32(p_g / p_u) at
    # the boundary) or stores the first in fp32 and adds the second: at most
    # the 2h reduction steps of one accumulation plus a scaling rounding,
    # counted in the bound as 2h + 64 steps
    ref, sabs = _dx_oracle(dgq_r, sdg, duq_r, sdu, wgq, swg, wuq, swu)
    gemm_close(g["dx"][rows], ref, "dX rows", sabs_bits=sabs, K=2 * h + 64, accum=accum)
    stage_gemm(g["dw_gate"][cols], "tn", np.ascontiguousarray(g["dgq"][:, cols]), E5, sdg, xq, E4, sx,
               "dW_gate rows", accum)
    stage_gemm(g["dw_up"][cols], "tn", np.ascontiguousarray(g["duq"][:, cols]), E5, sdu, xq, E4, sx,
               "dW_up rows", accum)
    stage_gemm(T(g["dw_down"]), "tn", np.ascontiguousarray(g["aq"][:, cols]), E4, sa, gq, E5, sg,
               "dW_down columns", accum)

    # ---- code parity with the oracle chain where the cast's input agrees
    _codes_equal_where(aq_r, o["Aq_r"], a_r == o["A_r"], "Aq rows")
    _codes_equal_where(aq_c, o["Aqt_c"], a_c == o["At_c"], "Aq columns")
    _codes_equal_where(dgq_r, o["dGq_r"], dg_r == o["dG_r"], "dGq rows")
    _codes_equal_where(duq_r, o["dUq_r"], du_r == o["dU_r"], "dUq rows")
    _codes_equal_where(dgq_c, o["dGqt_c"], dg_c == o["dGt_c"], "dGq columns")
    _codes_equal_where(duq_c, o["dUqt_c"], du_c == o["dUt_c"], "dUq columns")

    # ---- end to end against the oracle chain
    moved = lambda q, r: (q != r).any(1)
    chain_close(g["y"][rows], o["Y_r"], "Y rows", accum, moved(aq_r, o["Aq_r"]))
    chain_close(g["dx"][rows], o["dX_r"], "dX rows", accum,
                moved(np.concatenate([dgq_r, duq_r], 1), np.concatenate([o["dGq_r"], o["dUq_r"]], 1)))
    chain_close(g["dw_gate"][cols], o["dWg_c"], "dW_gate rows", accum, moved(dgq_c, o["dGqt_c"]))
    chain_close(g["dw_up"][cols], o["dWu_c"], "dW_up rows", accum, moved(duq_c, o["dUqt_c"]))
    chain_close(T(g["dw_down"]), o["dWdT_c"], "dW_down columns", accum, moved(aq_c, o["Aqt_c"]))
