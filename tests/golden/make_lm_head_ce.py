"""Writes lm_head_ce.json: the oracle's tensor-wide quantities of the FP8 LM
head fused with the softcapped cross-entropy at full size (M=16384, K=3072,
V=50304 with 50257 classes, chunks of 8192 rows, softcap 15).

Every chunk's dZ scale depends on all its logits and every row's gradient on
the row's log-sum-exp, so sampled checks of dX rows and dW rows at this size
need the chunk scales, each row's log-sum-exp and the mean loss.  This
script runs the oracle's logits GEMM and loss for every chunk once (no
gradient GEMMs; a few minutes on a multi-core host) and stores them.
Everything here is the oracle applied to the seeded inputs.

    python tests/golden/make_lm_head_ce.py
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

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "lm_head_ce.json")


def f32_hex(v: float) -> str:
    return "0x%08x" % int(np.float32(v).view(np.uint32))


def main():
    w = synth.LM_HEAD_CE
    x, wt, t = w.tensors()
    h = hashlib.sha256()
    for a in (x, wt, t):
        h.update(np.ascontiguousarray(a).tobytes())
    t0 = time.time()
    xq, sx, _ = oracle.quant(x, oracle.E4M3)
    wq, sw, _ = oracle.quant(wt, oracle.E4M3)
    tg = t.astype(np.int64)
    n_valid = int(((tg >= 0) & (tg < w.n_classes)).sum())
    lse = np.zeros(w.M)
    loss_rows = np.zeros(w.M)
    sdz = []
    for c0 in range(0, w.M, w.chunk):
        c1 = min(c0 + w.chunk, w.M)
        z = oracle.gemm_nt(xq[c0:c1], oracle.E4M3, sx, wq, oracle.E4M3, sw)
        lr, g, dz = oracle.softcap_ce_rows(z, tg[c0:c1], w.n_classes, w.softcap, n_valid)
        zz = oracle.bf16_bits_to_f64(z)[:, :w.n_classes]
        s = w.softcap * np.tanh(zz / w.softcap)
        m = s.max(axis=1, keepdims=True)
        lse[c0:c1] = m[:, 0] + np.log(np.exp(s - m).sum(axis=1))
        loss_rows[c0:c1] = lr
        _, sk, _ = oracle.quant(dz, oracle.E5M2)
        sdz.append(sk)
        print(f"chunk {c0 // w.chunk}: sdz {sk:.6g}  ({time.time() - t0:.0f} s)", flush=True)
    loss = float(loss_rows.sum() / n_valid)
    rec = dict(about="Oracle quantities of the LM head + softcapped CE at full size, written by "
                     "make_lm_head_ce.py (oracle only).  f32 = IEEE binary32 bits; lse as fp64 hex.",
               M=w.M, K=w.K, V=w.V, n_classes=w.n_classes, chunk=w.chunk, softcap=w.softcap,
               inputs_sha256=h.hexdigest(), sx=f32_hex(sx), sw=f32_hex(sw), n_valid=n_valid,
               sdz=[f32_hex(v) for v in sdz], loss=loss, seconds=round(time.time() - t0, 1),
               lse=[float(v).hex() for v in lse])
    with open(OUT, "w") as f:
        json.dump(rec, f, indent=0)
        f.write("\n")
    print(f"loss {loss}  written {OUT}")


if __name__ == "__main__":
    main()
