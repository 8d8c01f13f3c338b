"""Writes block_scales.json: the oracle's tensor-wide scales of the relu^2 MLP
block (and of the gated SwiGLU block) at the full workload sizes.

Two of the block's scales depend on a maximum over a whole intermediate
tensor (amax of A = relu(H)^2 and amax of dH), so checking sampled rows of
the later stages at M=8192 or M=32768 needs the complete H = Xq Uq^T and
dA = Gq Dq; this script computes them once with the oracle (two full GEMMs
per workload, a few minutes on a multi-core host) and stores the scales.
Everything here is the oracle applied to the seeded inputs; nothing comes
from the HIP path.

    python tests/golden/make_block_scales.py            # all workloads
    python tests/golden/make_block_scales.py mlp_3p8b   # one
"""
from __future__ import annotations

import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
from fp8_tensorwise_scaled_amd import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "block_scales.json")
WORKLOADS = {"mlp_3p8b": lambda: synth.MLP_3P8B, "proj_set_mlp": lambda: synth.PROJ_SET.mlp(),
             "swiglu_3p8b": lambda: synth.SWIGLU_3P8B}


def f32_hex(v: float) -> str:
    return "0x%08x" % int(np.float32(v).view(np.uint32))


def input_digest(tensors) -> str:
    h = hashlib.sha256()
    for t in tensors:
        h.update(np.ascontiguousarray(t).tobytes())
    return h.hexdigest()


def block_scales(w) -> dict:
    E4, E5 = oracle.E4M3, oracle.E5M2
    x, wu, wd, dy = w.tensors()
    t0 = time.time()
    xq, sx, _ = oracle.quant(x, E4)
    uq, su, _ = oracle.quant(wu, E4)
    dq, sd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    h = oracle.gemm_nt(xq, E4, sx, uq, E4, su)
    _, sa, amax_a = oracle.quant(oracle.relu2(h), E4)
    da = oracle.gemm_nn(gq, E5, sg, dq, E4, sd)
    _, sh, amax_dh = oracle.quant(oracle.relu2_bwd(h, da), E5)
    vals = dict(sx=sx, su=su, sd=sd, sg=sg, amax_a=amax_a, sa=sa, amax_dh=amax_dh, sh=sh)
    return dict(M=w.M, d=w.d, h=w.h, inputs_sha256=input_digest((x, wu, wd, dy)),
                seconds=round(time.time() - t0, 1),
                **{k: {"f32": f32_hex(v), "value": float(v)} for k, v in vals.items()})


def swiglu_scales(w) -> dict:
    """Gated block: amax of A = silu(G) U, of dG and of dU need the complete
    G, U (two GEMMs) and dA (one GEMM)."""
    E4, E5 = oracle.E4M3, oracle.E5M2
    x, wg, wu, wd, dy = w.tensors()
    t0 = time.time()
    xq, sx, _ = oracle.quant(x, E4)
    gq_w, swg, _ = oracle.quant(wg, E4)
    uq_w, swu, _ = oracle.quant(wu, E4)
    dq, swd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    g = oracle.gemm_nt(xq, E4, sx, gq_w, E4, swg)
    u = oracle.gemm_nt(xq, E4, sx, uq_w, E4, swu)
    _, sa, amax_a = oracle.quant(oracle.swiglu_gate(g, u), E4)
    da = oracle.gemm_nn(gq, E5, sg, dq, E4, swd)
    dg, du = oracle.swiglu_gate_bwd(g, u, da)
    _, sdg, amax_dg = oracle.quant(dg, E5)
    _, sdu, amax_du = oracle.quant(du, E5)
    vals = dict(sx=sx, swg=swg, swu=swu, swd=swd, sg=sg, amax_a=amax_a, sa=sa, amax_dg=amax_dg, sdg=sdg,
                amax_du=amax_du, sdu=sdu)
    return dict(M=w.M, d=w.d, h=w.h, inputs_sha256=input_digest((x, wg, wu, wd, dy)),
                seconds=round(time.time() - t0, 1),
                **{k: {"f32": f32_hex(v), "value": float(v)} for k, v in vals.items()})


def main(names):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    data["_about"] = ("Oracle scales of the relu^2 and SwiGLU MLP blocks at full size, written by "
                      "make_block_scales.py (oracle only).  f32 = IEEE binary32 bits.")
    for n in names:
        print(f"{n}: computing", flush=True)
        fn = swiglu_scales if n.startswith("swiglu") else block_scales
        data[n] = fn(WORKLOADS[n]())
        print(f"{n}: {data[n]}", flush=True)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")


if __name__ == "__main__":
    main(sys.argv[1:] or list(WORKLOADS))
