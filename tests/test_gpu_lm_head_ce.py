"""GPU parity of fp8_lm_head_ce: the FP8 LM head fused with the softcapped
cross-entropy, chunked over rows, against the oracle's lm_head_ce.

Expected values are the oracle's on the seeded inputs.  Held to the strict
bar (bit-exact codes and scales, the GEMM bound) wherever their inputs equal
the oracle's bit for bit: the X and W quantisation, the logits of the last
chunk, its dZ codes where dZ and the chunk scale agree, grad-input rows
whose dZ codes agree.  The last chunk's dZ is held element by element to the
bound that the logits' GEMM bound implies (plus one bf16 ulp and the fp32
evaluation of tanh and exp; the oracle works in fp64), the loss to the bound
the logits imply, dX and dW to the chain bar."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from fp8_tensorwise_scaled_amd import synth
from tests.gpu_util import (abs_codes, bf16_bits, bits_f64, f32, gemm_bound, gemm_close, oracle_gemm, to_dev_bf16,
                            ulp_bf16)
from tests.mlp_chain import chain_close

pytestmark = pytest.mark.gpu
E4, E5 = oracle.E4M3, oracle.E5M2
GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "lm_head_ce.json")


def pad16(v):
    return (v + 15) // 16 * 16


def run(x, w, t, n, chunk, softcap=15.0, accum=0):
    from fp8_tensorwise_scaled_amd import api

    dev = torch.device("cuda:0")
    M, K = x.shape
    V = w.shape[0]
    X, W = to_dev_bf16(x), to_dev_bf16(w)
    T = torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).to(dev)
    ws = api.fp8_lm_head_ce_workspace(M, K, V, chunk, dev)
    loss, dx, dw, sc = api.fp8_lm_head_ce(X, W, T, n, softcap, chunk, ws=ws, accum=accum)
    torch.cuda.synchronize()
    offs = api.lm_head_ce_layout(M, K, V, chunk)
    wsn = ws.cpu().numpy()
    Vp = pad16(V)
    nch = (M + chunk - 1) // chunk
    last = M - (nch - 1) * chunk if M > 0 else 0
    g = dict(loss=float(f32(loss)[0]), dx=bf16_bits(dx), dw=bf16_bits(dw), sc=f32(sc),
             xq=wsn[offs[0]:offs[0] + M * K].reshape(M, K), wq=wsn[offs[1]:offs[1] + V * K].reshape(V, K),
             dz_last=wsn[offs[2]:offs[2] + last * Vp * 2].view(np.uint16).reshape(last, Vp)[:, :V],
             dzq_last=wsn[offs[3]:offs[3] + last * Vp].reshape(last, Vp)[:, :V],
             last=last, X=X, W=W, T=T, ws=ws)
    return g


def small_case():
    wl = synth.LMHeadCEWorkload(61, 256, 256, 600, n_classes=590, chunk=64, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    t[[7, 100]] = [595, 599]       # padded class ids: ignored like -100
    return wl, x, w, t


@pytest.fixture(scope="module")
def small():
    wl, x, w, t = small_case()
    g = run(x, w, t, wl.n_classes, wl.chunk)
    r = oracle.lm_head_ce(x, w, t, wl.n_classes, wl.softcap, wl.chunk)
    return wl, x, w, t, g, r


def test_quantisation_and_scales(small):
    wl, x, w, t, g, r = small
    assert np.float32(g["sc"][0]) == np.float32(r["sx"]) and np.float32(g["sc"][1]) == np.float32(r["sw"])
    assert (g["xq"] == r["xq"]).all() and (g["wq"] == r["wq"]).all()
    for k, ch in enumerate(r["chunks"]):
        gs, os_ = float(g["sc"][2 + k]), float(ch["sdz"])
        print(f"chunk {k}: dZ scale gpu {gs:.9g} oracle {os_:.9g}")
        assert abs(gs - os_) <= 2.0 ** -7 * os_, (k, gs, os_)


def test_loss_within_logit_bound(small):
    """|S' - S| <= |Z' - Z| (the capped map is 1-Lipschitz), so each row's
    loss moves by at most twice the row's largest logit bound."""
    wl, x, w, t, g, r = small
    n, C = wl.n_classes, wl.chunk
    valid = (t >= 0) & (t < n)
    total = 0.0
    for k, c0 in enumerate(range(0, x.shape[0], C)):
        z, sabs, K = oracle_gemm("nt", r["xq"][c0:c0 + C], E4, r["sx"], r["wq"], E4, r["sw"])
        assert (z == r["chunks"][k]["z"]).all()
        b = gemm_bound(z, sabs, K)[:, :n].max(axis=1)
        total += float((2 * b * valid[c0:c0 + C]).sum())
    bound = total / max(int(valid.sum()), 1) + 2e-6 * abs(r["loss"]) + 1e-6
    print(f"loss gpu {g['loss']:.9g} oracle {r['loss']:.9g} bound {bound:.3g}")
    assert abs(g["loss"] - r["loss"]) <= bound


def dz_bound(z_bits, b, t, n, softcap, n_valid):
    """Element-wise bound on |dZ_gpu - dZ_oracle| when the GPU's logits lie
    within b of the oracle's: the capped logits move by at most b (the cap is
    1-Lipschitz), the row's log-sum-exp by at most E = max_j b_j, so p_j moves
    by at most p_j (exp(b_j + E) - 1); 1 - tanh^2 moves by at most
    (2/c) |tanh| (1 - tanh^2) b_j.  Plus one bf16 ulp of the result (the two
    roundings) and the fp32 evaluation of exp, tanh and the products."""
    z = bits_f64(z_bits)[:, :n]
    th = np.tanh(z / softcap)
    s = softcap * th
    lse = np.log(np.exp(s).sum(axis=1, keepdims=True))
    p = np.exp(s - lse)
    y = np.zeros_like(p)
    valid = (t >= 0) & (t < n)
    y[np.arange(len(t))[valid], t[valid]] = 1.0
    bb = b[:, :n]
    E = bb.max(axis=1, keepdims=True)
    with np.errstate(over="ignore"):
        d = 1.0 / np.cosh(z / softcap) ** 2   # 1 - tanh^2 without its cancellation at saturation
    g = (p - y) * d / n_valid
    dev = (p * np.expm1(bb + E) * d + np.abs(p - y) * (2.0 / softcap) * np.abs(th) * d * bb) / n_valid
    bound = np.full(z_bits.shape, 1e-30)
    bound[:, :n] = dev * 1.01 + ulp_bf16(g) + 4e-6 * (p + y) * d / n_valid + 1e-30
    bound[~valid] = 1e-30
    return bound


@pytest.mark.parametrize("sigma_w,beyond20", [(4.0, False), (9.0, True)])
def test_saturated_logits_dz(sigma_w, beyond20):
    """Logits far beyond the cap (|Z / c| up to about 20, and with the wider
    weights up to about 43, where the kernel's exponent reaches its clamp):
    where tanh saturates, 1 - tanh^2 must keep its relative precision (the
    bound allows 4e-6 of it beyond what the logits' GEMM bound implies)."""
    wl = synth.LMHeadCEWorkload(66, 128, 256, 600, n_classes=590, chunk=64, sigma_w=sigma_w, ignored=0.05)
    x, w, t = wl.tensors()
    g = run(x, w, t, wl.n_classes, wl.chunk)
    r = oracle.lm_head_ce(x, w, t, wl.n_classes, wl.softcap, wl.chunk)
    n = wl.n_classes
    ch = r["chunks"][-1]
    c0 = x.shape[0] - g["last"]
    _, sabs, K = oracle_gemm("nt", r["xq"][c0:], E4, r["sx"], r["wq"], E4, r["sw"])
    z = bits_f64(ch["z"])[:, :n]
    sat = float((np.abs(z / wl.softcap) > 5.0).mean())
    nv = int(((t >= 0) & (t < n)).sum())
    bound = dz_bound(ch["z"], gemm_bound(ch["z"], sabs, K), t[c0:], n, wl.softcap, nv)
    err = np.abs(bits_f64(g["dz_last"]) - bits_f64(ch["dz"]))
    zc = np.abs(z / wl.softcap)
    in_20_43 = float(((zc > 20) & (zc < 43)).mean())
    print(f"saturated dZ: |Z/c| > 5 for {sat:.2%} of logits, in (20, 43) for {in_20_43:.2%}, "
          f"max err / bound {float((err / bound).max()):.3g}")
    assert sat > 0.2
    if beyond20:
        assert in_20_43 > 0.02
    assert (err <= bound).all()
    assert abs(g["loss"] - r["loss"]) <= 1e-3 * abs(r["loss"]), (g["loss"], r["loss"])


@pytest.mark.parametrize("accum", [0, 1], ids=["fast", "exact"])
def test_last_chunk_stages(small, accum):
    """The last chunk's stages: its logits (recomputed through the same GEMM
    entry, in the accumulation mode) against the oracle's, its dZ within the
    bound the logits imply, its codes bit-exact where dZ agrees, and its dX
    rows against the oracle GEMM of the GPU's own codes."""
    from fp8_tensorwise_scaled_amd import api

    wl, x, w, t, g, r = small
    if accum:
        g = run(x, w, t, wl.n_classes, wl.chunk, accum=accum)
    n = wl.n_classes
    ch = r["chunks"][-1]
    c0 = x.shape[0] - g["last"]
    # the GPU's logits of the last chunk, recomputed through the same GEMM entry
    xq = torch.from_numpy(g["xq"][c0:]).cuda()
    wq = torch.from_numpy(g["wq"]).cuda()
    sx = torch.tensor([g["sc"][0]], device="cuda")
    sw = torch.tensor([g["sc"][1]], device="cuda")
    zg = bf16_bits(api.fp8_linear_fwd(xq, sx, wq, sw, accum=accum))
    _, sabs, K = oracle_gemm("nt", r["xq"][c0:], E4, r["sx"], r["wq"], E4, r["sw"])
    gemm_close(zg, ch["z"], "logits (last chunk)", sabs_bits=sabs, K=K, accum=accum)
    # dZ within the bound the logits' GEMM bound implies
    nv = int(((t >= 0) & (t < n)).sum())
    bound = dz_bound(ch["z"], gemm_bound(ch["z"], sabs, K), t[c0:], n, wl.softcap, nv)
    err = np.abs(bits_f64(g["dz_last"]) - bits_f64(ch["dz"]))
    print(f"dZ: max err / bound {float((err / bound).max()):.3g}, identical {float((g['dz_last'] == ch['dz']).mean()):.4f}")
    assert (err <= bound).all()
    chain_close(g["dz_last"], ch["dz"], "dZ (last chunk)")
    # codes: bit-exact where dZ and the chunk scale agree
    sk = float(g["sc"][2 + len(r["chunks"]) - 1])
    same_dz = g["dz_last"] == ch["dz"]
    assert np.float32(sk) == np.float32(ch["sdz"])
    assert (g["dzq_last"][same_dz] == ch["dzq"][same_dz]).all()
    # dX of the chunk against the oracle GEMM of the GPU's own dZ codes
    ref, sab, KK = oracle_gemm("nn", np.ascontiguousarray(g["dzq_last"]), E5, sk, r["wq"], E4, r["sw"])
    gemm_close(g["dx"][c0:], ref, "dX rows of the last chunk", sabs_bits=sab, K=KK, accum=accum)


def test_gradients_chain_bar(small):
    wl, x, w, t, g, r = small
    chain_close(g["dx"], r["dx"], "dX")
    chain_close(g["dw"], r["dw"], "dW")
    assert (g["dw"][wl.n_classes:] == 0).all()
    ignored = ~((t >= 0) & (t < wl.n_classes))
    assert (g["dx"][ignored] & 0x7FFF == 0).all()


def test_deterministic(small):
    wl, x, w, t, g, r = small
    g2 = run(x, w, t, wl.n_classes, wl.chunk)
    assert g2["loss"] == g["loss"] and (g2["dx"] == g["dx"]).all() and (g2["dw"] == g["dw"]).all()


def test_no_counted_rows_and_no_rows():
    wl, x, w, t = small_case()
    g = run(x, w, np.full_like(t, -100), wl.n_classes, wl.chunk)
    assert g["loss"] == 0.0 and (g["dx"] & 0x7FFF == 0).all() and (g["dw"] & 0x7FFF == 0).all()
    g = run(x[:0], w, t[:0], wl.n_classes, wl.chunk)
    assert g["loss"] == 0.0 and (g["dw"] == 0).all()


def test_full_size_sampled():
    """M=16384, K=3072, V=50304 (50257 classes), chunks of 8192: the oracle's
    stored chunk scales, row log-sum-exps and loss, and 12 sampled rows of dX
    and 12 rows of dW computed by the oracle from them."""
    wl = synth.LM_HEAD_CE
    x, w, t = wl.tensors()
    gold = json.load(open(GOLDEN))
    import hashlib
    h = hashlib.sha256()
    for a in (x, w, t):
        h.update(np.ascontiguousarray(a).tobytes())
    assert h.hexdigest() == gold["inputs_sha256"], "inputs changed; rerun tests/golden/make_lm_head_ce.py"
    f32h = lambda s: float(np.array([int(s, 16)], np.uint32).view(np.float32)[0])
    g = run(x, w, t, wl.n_classes, wl.chunk, wl.softcap)
    assert np.float32(g["sc"][0]) == np.float32(f32h(gold["sx"]))
    assert np.float32(g["sc"][1]) == np.float32(f32h(gold["sw"]))
    xq, sx, _ = oracle.quant(x, E4)
    wq, sw, _ = oracle.quant(w, E4)
    assert (g["xq"] == xq).all() and (g["wq"] == wq).all()
    sdz = [f32h(s) for s in gold["sdz"]]
    for k, s in enumerate(sdz):
        assert abs(float(g["sc"][2 + k]) - s) <= 2.0 ** -7 * s, (k, float(g["sc"][2 + k]), s)
    print(f"loss gpu {g['loss']:.9g} oracle {gold['loss']:.9g}")
    assert abs(g["loss"] - gold["loss"]) <= 1e-3 * abs(gold["loss"])
    n, C, nv = wl.n_classes, wl.chunk, gold["n_valid"]
    lse = np.array([float.fromhex(v) for v in gold["lse"]])
    rng = np.random.default_rng(66)
    rows = np.sort(rng.choice(x.shape[0], 12, replace=False))
    z = oracle.gemm_nt(xq, E4, sx, wq, E4, sw, rows=rows)
    _, _, dz = oracle.softcap_ce_rows(z, t[rows], n, wl.softcap, nv)
    dzq = np.stack([oracle.cast(dz[i:i + 1], sdz[r // C], E5)[0] for i, r in enumerate(rows)])
    dx_ref = np.stack([oracle.gemm_nn(dzq[i:i + 1], E5, sdz[r // C], wq, E4, sw)[0] for i, r in enumerate(rows)])
    chain_close(g["dx"][rows], dx_ref, "dX sampled rows")
    cols = np.sort(np.concatenate([rng.choice(n, 10, replace=False), [n, wl.V - 1]]))
    zt = oracle.gemm_nt(wq, E4, sw, xq, E4, sx, rows=cols)          # logits columns, transposed
    _, dzt = oracle.softcap_ce_columns(zt, cols, lse, t, n, wl.softcap, nv)
    acc = np.zeros((cols.size, x.shape[1]))
    for k, c0 in enumerate(range(0, x.shape[0], C)):
        codes = oracle.cast(np.ascontiguousarray(dzt[:, c0:c0 + C].T), sdz[k], E5)   # [rows, ncols]
        oracle.gemm_tn_acc(codes, E5, sdz[k], xq[c0:c0 + C], E4, sx, acc)
    dw_ref = oracle.double_to_bf16(acc)
    chain_close(g["dw"][cols[:10]], dw_ref[:10], "dW sampled rows")
    assert (g["dw"][cols[10:]] == 0).all() and (dw_ref[10:] == 0).all()


def test_wide_vocabulary_few_rows():
    """V = 56000 (wider than the 3.8B model's 50304) over 32 rows in chunks
    of 16: loss within 1e-3 relative of the oracle's, gradients within the
    chain bar, padded rows of dW zero."""
    wl = synth.LMHeadCEWorkload(62, 32, 64, 56000, n_classes=55990, chunk=16, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    g = run(x, w, t, wl.n_classes, wl.chunk)
    r = oracle.lm_head_ce(x, w, t, wl.n_classes, wl.softcap, wl.chunk)
    assert abs(g["loss"] - r["loss"]) <= 1e-3 * abs(r["loss"]), (g["loss"], r["loss"])
    chain_close(g["dx"], r["dx"], "dX (wide vocabulary)")
    chain_close(g["dw"], r["dw"], "dW (wide vocabulary)")
    assert (g["dw"][wl.n_classes:] == 0).all()


@pytest.mark.parametrize("M,K,V,n,chunk", [(208, 96, 333, 333, 48), (144, 64, 1000, 997, 128), (64, 48, 260, 250, 64)])
def test_ragged_chunks_and_vocabulary(M, K, V, n, chunk):
    """A last chunk shorter than the others, an odd or ragged vocabulary
    (last column tiles 77, 232 and 4 wide), a single chunk covering all rows:
    loss within 1e-3 relative of the oracle's, gradients within the chain
    bar, padded rows of dW zero."""
    wl = synth.LMHeadCEWorkload(67 + M, M, K, V, n_classes=n, chunk=chunk, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    g = run(x, w, t, wl.n_classes, wl.chunk)
    r = oracle.lm_head_ce(x, w, t, wl.n_classes, wl.softcap, wl.chunk)
    assert abs(g["loss"] - r["loss"]) <= 1e-3 * abs(r["loss"]), (g["loss"], r["loss"])
    chain_close(g["dx"], r["dx"], f"dX ({M}x{K}x{V}, chunk {chunk})")
    chain_close(g["dw"], r["dw"], f"dW ({M}x{K}x{V}, chunk {chunk})")
    assert (g["dw"][n:] == 0).all()


@pytest.mark.parametrize("accum", [0, 1], ids=["fast", "exact"])
def test_single_chunk_gradients_on_own_codes(accum):
    """One chunk covering all rows (the grad-weight product is stored
    directly, no fp32 accumulation across chunks): dX and dW against the
    oracle GEMMs of the GPU's own dZ codes and scale, in the accumulation
    mode (exact: the strict bar); an odd vocabulary (V = 333, 323 classes)
    so that both reductions over the vocabulary end in a masked tail."""
    wl = synth.LMHeadCEWorkload(68, 96, 80, 333, n_classes=323, chunk=96, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    g = run(x, w, t, wl.n_classes, wl.chunk, accum=accum)
    xq, sx, _ = oracle.quant(x, E4)
    wq, sw, _ = oracle.quant(w, E4)
    assert (g["xq"] == xq).all() and (g["wq"] == wq).all()
    sk = float(g["sc"][2])
    dzq = np.ascontiguousarray(g["dzq_last"])
    assert (dzq[:, wl.n_classes:] == 0).all()
    ref, sab, K = oracle_gemm("nn", dzq, E5, sk, wq, E4, sw)
    gemm_close(g["dx"], ref, "dX (one chunk)", sabs_bits=sab, K=K, accum=accum)
    ref, sab, K = oracle_gemm("tn", dzq, E5, sk, xq, E4, sx)
    gemm_close(g["dw"], ref, "dW (one chunk)", sabs_bits=sab, K=K, accum=accum)


@pytest.mark.parametrize("accum", [0, 1], ids=["fast", "exact"])
def test_two_chunks_grad_weight_on_own_codes(accum):
    """Two equal chunks of 128 rows (V a multiple of 4): dW is one
    two-segment product, RN_bf16(p_2 (S_2 + RN32(p_1 / p_2) S_1)), the first
    chunk's dZ codes kept where the fp32 sum would otherwise go.  dW against
    the oracle's exact sum of both chunks' products on the GPU's own codes
    and scales, in the accumulation mode (exact: the strict bar); the bound
    counts 2C + 128 reduction steps (the rescale adds two roundings)."""
    wl = synth.LMHeadCEWorkload(69, 256, 96, 600, n_classes=590, chunk=128, sigma_w=0.25, ignored=0.05)
    x, w, t = wl.tensors()
    g = run(x, w, t, wl.n_classes, wl.chunk, accum=accum)
    from fp8_tensorwise_scaled_amd import api

    M, K, V, C = 256, 96, 600, 128
    Vp = pad16(V)
    offs = api.lm_head_ce_layout(M, K, V, C)
    wsn = g["ws"].cpu().numpy()
    dzq = [wsn[offs[4]:offs[4] + C * Vp].reshape(C, Vp)[:, :V], g["dzq_last"]]
    xq, sx, _ = oracle.quant(x, E4)
    assert (g["xq"] == xq).all()
    for k in range(2):
        assert (dzq[k][:, wl.n_classes:] == 0).all()
    acc, acc_abs = np.zeros((V, K)), np.zeros((V, K))
    for k in range(2):
        sk = float(g["sc"][2 + k])
        oracle.gemm_tn_acc(np.ascontiguousarray(dzq[k]), E5, sk, xq[k * C:(k + 1) * C], E4, sx, acc)
        oracle.gemm_tn_acc(abs_codes(np.ascontiguousarray(dzq[k])), E5, sk, abs_codes(xq[k * C:(k + 1) * C]), E4, sx,
                           acc_abs)
    gemm_close(g["dw"], oracle.double_to_bf16(acc), "dW (two chunks, one launch)",
               sabs_bits=oracle.double_to_bf16(acc_abs), K=2 * C + 128, accum=accum)
    # dX of the first chunk read its codes from the same place
    ref, sab, KK = oracle_gemm("nn", np.ascontiguousarray(dzq[0]), E5, float(g["sc"][2]), g["wq"], E4,
                               float(g["sc"][1]))
    gemm_close(g["dx"][:C], ref, "dX (first chunk)", sabs_bits=sab, K=KK, accum=accum)
