"""Benchmark: FP8 relu^2 MLP block fwd+bwd on one MI355X.

One step = relu2_mlp_fwd + relu2_mlp_bwd on the 3.8B-model block
(M=8192 tokens, d=3072, h=12288): three quantisations of the inputs, the
relu^2 cast, the dY and dH casts and all six FP8 GEMMs, with inputs resident
in HBM.  The metric counts GEMM FLOPs only (12*M*d*h per step), the
convention of the pages' TFLOP/s figure.

Prints one JSON line.  --gpus > 1 is not supported: the library runs the
block on one GPU (no sharding, no collectives).
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(w, rows_per_gemm: int = 1536):
    """Oracle GEMM rate on a bounded sample: rows_per_gemm output rows of each
    of the six GEMMs of the block (FP8 operands from the oracle's quantiser)."""
    import numpy as np

    import oracle

    x, wu, wd, dy = w.tensors()
    t0 = time.perf_counter()
    xq, sx, _ = oracle.quant(x, oracle.E4M3)
    uq, su, _ = oracle.quant(wu, oracle.E4M3)
    dq, sd, _ = oracle.quant(wd, oracle.E4M3)
    gq, sg, _ = oracle.quant(dy, oracle.E5M2)
    t_quant = time.perf_counter() - t0
    rng = np.random.default_rng(0)
    rm = rng.choice(w.M, rows_per_gemm, replace=False)
    rh = rng.choice(w.h, rows_per_gemm, replace=False)
    rd = rng.choice(w.d, rows_per_gemm, replace=False)
    # [M, h] stand-ins with the formats of the block's A (E4M3) and dH (E5M2)
    aq, sa = np.ascontiguousarray(np.tile(xq, (1, w.h // w.d))), sx
    hq_src = np.ascontiguousarray(np.tile(gq, (1, w.h // w.d)))
    flops = 0
    t0 = time.perf_counter()
    oracle.gemm_nt(xq, 0, sx, uq, 0, su, rows=rm); flops += 2 * rows_per_gemm * w.h * w.d      # up fwd
    oracle.gemm_nt(aq, 0, sa, dq, 0, sd, rows=rm); flops += 2 * rows_per_gemm * w.d * w.h      # down fwd
    oracle.gemm_tn(gq, 1, sg, aq, 0, sa, rows=rd); flops += 2 * rows_per_gemm * w.h * w.M      # down wgrad
    oracle.gemm_nn(gq, 1, sg, dq, 0, sd, rows=rm); flops += 2 * rows_per_gemm * w.h * w.d      # down dgrad
    oracle.gemm_tn(hq_src, 1, sg, xq, 0, sx, rows=rh); flops += 2 * rows_per_gemm * w.d * w.M  # up wgrad
    oracle.gemm_nn(hq_src, 1, sg, uq, 0, su, rows=rm); flops += 2 * rows_per_gemm * w.d * w.h  # up dgrad
    t_gemm = time.perf_counter() - t0
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    model = None
    try:
        model = next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                     None)
    except OSError:
        pass
    return {
        "value": flops / t_gemm / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "host_cpus": os.cpu_count(),
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{rows_per_gemm} output rows of each of the six GEMMs of the M={w.M} d={w.d} h={w.h} "
                  f"block ({flops / 1e9:.1f} GFLOP, fp64 accumulation, {t_gemm:.1f} s); the four input "
                  f"quantisations took {t_quant:.1f} s",
        "gemm_seconds": t_gemm,
    }


def gpu_clocks():
    """Current shader and memory clock levels from sysfs (best effort; the
    starred level of pp_dpm_sclk / pp_dpm_mclk), or None where not exposed."""
    import glob

    out = {}
    for kind in ("sclk", "mclk"):
        for path in sorted(glob.glob(f"/sys/class/drm/card*/device/pp_dpm_{kind}")):
            try:
                cur = [ln.strip() for ln in open(path) if ln.strip().endswith("*")]
            except OSError:
                continue
            if cur:
                out[kind] = cur[0]
                break
    return out or None


def measured_traffic():
    """HBM bytes per launch of the roofline kernel from the committed
    rocprofv3 FETCH_SIZE / WRITE_SIZE summary (profiles/), or None when the
    GEMM source has changed since those counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "gemm_down_proj_traffic.json")
    src = os.path.join(ROOT, "fp8_tensorwise_scaled_amd", "csrc", "gemm.hip")
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(src, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_hip_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def _time_steps(step, steps, warmup):
    """Average ms per call of step() over `steps` calls after `warmup`, HIP
    events on the current stream."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    return ev0.elapsed_time(ev1) / steps


def _roofline(kernel: str, bound: str, flops_or_bytes: float, us: float, peak: float, unit: str):
    """Roofline object for one kernel: algorithmic work per launch / its
    average launch time (HIP events on the launching stream)."""
    achieved = flops_or_bytes / (us * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
    return {"kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
            "frac": round(achieved / peak, 4), "traffic": None, "avg_launch_us": round(us, 2)}


def _oracle_gemms_rate(jobs, what: str):
    """cpu_baseline from timed oracle GEMMs on sampled output rows: jobs are
    (function, args, rows, flops)."""
    t0 = time.perf_counter()
    flops = 0
    for fn, a, rows, f in jobs:
        fn(*a, rows=rows)
        flops += f
    sec = time.perf_counter() - t0
    return {"value": flops / sec / 1e12, "unit": "TFLOP/s",
            "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
            "sample": f"{what} ({flops / 1e9:.1f} GFLOP, fp64 accumulation, {sec:.1f} s)"}


def bench_other(args) -> int:
    """Projection set (M=32768) or LM head (padded and unpadded vocabulary):
    one step = forward + backward of every linear, quantisations included."""
    import numpy as np
    import torch

    from fp8_tensorwise_scaled_amd import synth, workloads

    dev = torch.device("cuda:0")
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)
    common = {"n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
              "scaling": "weak", "vs_baseline": None, "dtype": "fp8", "unit": "TFLOP/s"}
    if args.workload == "proj":
        w = synth.PROJ_SET
        log(f"generating projection-set inputs M={w.M}")
        host = {n: w.input(n) for n in w.INPUTS}
        host.update({n: w.grad(n) for n, _ in w.GRADS})
        for i, (name, _, _) in enumerate(w.projections):
            host["w_" + name] = w.weight(i)
        tens = {k: t(v) for k, v in host.items()}
        r = workloads.ProjectionSetRunner(w.M, dev)
        ms = _time_steps(lambda: r.step(tens), args.steps, args.warmup)
        tflops = r.flops / (ms * 1e-3) / 1e12
        log(f"projection set: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
        res = {"metric": "FP8 decoder projection set fwd+bwd TFLOP/s (Q,K,V,O + relu2 MLP)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) inputs, N(0,1/sqrt(fan_in)) weights, N(0,1e-3) grads "
                       "with 0.1% x100 outliers; bf16)",
               "config": {"workload": "decoder projection set fwd+bwd M=32768 d=3072 (q 3072, k/v 1024, "
                                      "o 3072, relu2 MLP 12288)", "M": w.M, "gemm_flops": r.flops},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(w.M / (ms * 1e-3))}
    elif args.workload == "rmsnorm":
        from fp8_tensorwise_scaled_amd import api

        M, d = 8192, 3072
        log(f"generating RMSNorm inputs [{M}, {d}]")
        X = t(synth.normal_bf16((M, d), 2.5, 3001))
        G = t(synth.normal_bf16((d,), 1.0, 3002))
        q = torch.empty((M, d), dtype=torch.uint8, device=dev)
        qt = torch.empty((d, M), dtype=torch.uint8, device=dev)
        sc, am, rs = (torch.empty(n, dtype=torch.float32, device=dev) for n in (1, 1, M))
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
        fused = lambda: api.fp8_rmsnorm_quant(X, G, 1e-6, api.E4M3, q=q, qt=qt, scale=sc, amax=am, rstd=rs, ws=ws)

        def unfused():  # torch's RMSNorm writing X, then the quantiser reading it
            xn = torch.nn.functional.rms_norm(X, (d,), G, 1e-6)
            api.fp8_amax_quant(xn, api.E4M3, q=q, qt=qt, scale=sc, amax=am, ws=ws)
        ms = _time_steps(fused, args.steps * 5, args.warmup)
        ms_unf = _time_steps(unfused, args.steps * 5, args.warmup)
        nbytes = M * d * 6 + M * 4
        gbs = nbytes / (ms * 1e-3) / 1e9
        cpu = None
        if not args.no_cpu_baseline:
            import oracle

            R = 1024
            xs, gs = synth.normal_bf16((M, d), 2.5, 3001)[:R], synth.normal_bf16((d,), 1.0, 3002)
            t0 = time.perf_counter()
            oracle.rmsnorm_quant(xs, gs, 1e-6, oracle.E4M3)
            sec = time.perf_counter() - t0
            cpu = {"value": R * d * 6 / sec / 1e9, "unit": "GB/s",
                   "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
                   "sample": f"RMSNorm + quantisation of the first {R} rows ({sec:.2f} s)"}
        log(f"RMSNorm + quantise: {ms * 1e3:.1f} us ({gbs:.0f} GB/s); torch rms_norm then quantise: "
            f"{ms_unf * 1e3:.1f} us")
        res = {"metric": "RMSNorm fused with FP8 tensorwise quantisation (codes + transposed codes), GB/s",
               "value": round(gbs, 1), "unit": "GB/s", "ms_per_step": round(ms, 5),
               "data": "synthetic (seeded N(0,2.5) rows, N(0,1) weight; bf16)",
               "config": {"workload": f"RMSNorm + E4M3 quantisation of X [{M}, {d}], eps 1e-6", "M": M, "d": d,
                          "algorithmic_bytes": nbytes},
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
               "unfused_torch_rmsnorm_then_quantise_ms": round(ms_unf, 5), "cpu_baseline": cpu}
        common["unit"] = "GB/s"
    elif args.workload == "muon":
        from fp8_tensorwise_scaled_amd import api

        rows, cols, steps = 3072, 12288, 5
        log(f"generating Newton-Schulz input [{rows}, {cols}]")
        res_all = {}
        for shape in ((rows, cols), (cols, rows)):
            G = t(synth.normal_bf16(shape, 0.02, 4001, outlier_frac=1e-3))
            out = torch.empty(shape, dtype=torch.bfloat16, device=dev)
            norm = torch.empty(2, dtype=torch.float32, device=dev)
            ws = api.muon_ns_workspace(*shape, dev)
            ms = _time_steps(lambda: api.muon_newton_schulz(G, steps, out=out, norm=norm, ws=ws), args.steps,
                             args.warmup)
            res_all[shape] = ms
            log(f"Newton-Schulz {shape[0]}x{shape[1]}, {steps} steps: {ms:.3f} ms")
            del G, out, ws
        m, n = rows, cols
        flops = steps * (4 * m * m * n + 2 * m * m * m)
        ms = res_all[(rows, cols)]
        tflops = flops / (ms * 1e-3) / 1e12
        # dominant kernel: X = B X + a X (and X^T) on the bf16 matrix cores
        bf = dict(dtype=torch.bfloat16, device=dev)
        Bm = (torch.randn((m, m), device=dev) / m).to(torch.bfloat16)
        Xm = (torch.randn((m, n), device=dev) / 6000).to(torch.bfloat16)
        Xt, Xt2 = Xm.t().contiguous(), torch.empty((n, m), **bf)
        us = 1e3 * _time_steps(lambda: api.bf16_gemm_nt(Bm, Xt, 1.0, 3.4445, Xm, out=Xm, out_t=Xt2),
                               args.gemm_reps, 3)
        roof = _roofline(f"gemm_nt_kernel<2,2,256,192,4,2,5> (bf16, alpha/beta epilogue with transposed store; "
                         f"X = B X + a X, M={m} N={n} K={m})", "mfma", 2 * m * n * m, us, PEAK_BF16_TFLOPS,
                         "TFLOP/s")
        log(f"X = B X + a X: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        cpu = None
        if not args.no_cpu_baseline:
            import oracle

            g = synth.normal_bf16((rows, cols), 0.02, 4001, outlier_frac=1e-3)
            t0 = time.perf_counter()
            oracle.newton_schulz(g)
            sec = time.perf_counter() - t0
            cpu = {"value": flops / sec / 1e12, "unit": "TFLOP/s",
                   "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
                   "sample": f"the whole {rows}x{cols} orthogonalisation (fp64 BLAS products, bf16 roundings, "
                             f"{sec:.1f} s)"}
            log(f"oracle: {sec:.1f} s")
        res = {"metric": "Muon Newton-Schulz orthogonalisation (5 steps, bf16 matrix cores), TFLOP/s",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,0.02) gradient with 0.1% x100 outliers; bf16)",
               "config": {"workload": f"Newton-Schulz 5 steps on a {rows}x{cols} matrix (grad of W_down; "
                                      f"the transposed W_up shape beside it)", "rows": rows, "cols": cols,
                          "steps": steps, "flops": flops},
               "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
               "tall": {"rows": cols, "cols": rows, "ms": round(res_all[(cols, rows)], 4)},
               "roofline": roof, "cpu_baseline": cpu}
        common["dtype"] = "bf16"
    elif args.workload == "swiglu":
        from fp8_tensorwise_scaled_amd import api

        w = synth.SWIGLU_3P8B
        M, d, h = w.M, w.d, w.h
        log(f"generating SwiGLU inputs M={M} d={d} h={h}")
        X, WG, WU, WD, DY = (t(a) for a in w.tensors())
        bf = dict(dtype=torch.bfloat16, device=dev)
        Y, DX = torch.empty((M, d), **bf), torch.empty((M, d), **bf)
        DWG, DWU, DWD = torch.empty((h, d), **bf), torch.empty((h, d), **bf), torch.empty((d, h), **bf)
        BSC = torch.empty(3, dtype=torch.float32, device=dev)
        saved = api.SwigluMlpSaved.empty(M, d, h, dev)
        ws_f = api.swiglu_mlp_workspace("fwd", M, d, h, dev)
        ws_b = api.swiglu_mlp_workspace("bwd", M, d, h, dev)

        def step():
            api.swiglu_mlp_fwd(X, WG, WU, WD, y=Y, saved=saved, ws=ws_f)
            api.swiglu_mlp_bwd(DY, saved, dx=DX, dw_gate=DWG, dw_up=DWU, dw_down=DWD, bwd_scales=BSC, ws=ws_b)
        ms = _time_steps(step, args.steps, args.warmup)
        tflops = w.flops / (ms * 1e-3) / 1e12
        log(f"SwiGLU block: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
        # dominant kernel: the merged gate/up projection (G, U and A from one
        # GEMM, as in the block's forward) on the block's own codes
        offs = api.swiglu_workspace_layout("fwd", M, d, h)
        xq = ws_f[offs[0]:offs[0] + M * d].view(M, d)
        wgq = ws_f[offs[1]:offs[1] + h * d].view(h, d)
        wuq = ws_f[offs[2]:offs[2] + h * d].view(h, d)
        bf = dict(dtype=torch.bfloat16, device=dev)
        gb, ub, ab = torch.empty((M, h), **bf), torch.empty((M, h), **bf), torch.empty((M, h), **bf)
        sc = saved.scales
        us = 1e3 * _time_steps(lambda: api.fp8_gated_linear_fwd(xq, sc[0:1], wgq, sc[1:2], wuq, sc[2:3],
                                                                g=gb, u=ub, a=ab), args.gemm_reps, 3)
        roof = _roofline(f"gemm_nt_kernel<0,0,256,256,2,2,6> (E4M3 x E4M3; merged gate/up projection with the gate "
                         f"epilogue, M={M} N=2x{h} K={d})", "mfma", 2 * M * 2 * h * d, us, PEAK_FP8_TFLOPS, "TFLOP/s")
        log(f"merged gate/up GEMM: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        del ws_f, ws_b, saved, gb, ub, ab
        cpu = None
        if not args.no_cpu_baseline:
            import oracle

            x, wg, wu, wd, dy = w.tensors()
            xq_o, sx, _ = oracle.quant(x, oracle.E4M3)
            wgq_o, swg, _ = oracle.quant(wg, oracle.E4M3)
            wdq_o, swd, _ = oracle.quant(wd, oracle.E4M3)
            gq_o, sg, _ = oracle.quant(dy, oracle.E5M2)
            rng = np.random.default_rng(0)
            R = 256
            rm, rh, rd = (rng.choice(n, R, replace=False) for n in (M, h, d))
            # [M, h] stand-ins with the formats of A (E4M3) and dG / dU (E5M2)
            aq = np.ascontiguousarray(np.tile(xq_o, (1, -(-h // d)))[:, :h])
            dgq = np.ascontiguousarray(np.tile(gq_o, (1, -(-h // d)))[:, :h])
            E4, E5 = oracle.E4M3, oracle.E5M2
            jobs = [(oracle.gemm_nt, (xq_o, E4, sx, wgq_o, E4, swg), rm, 2 * R * h * d)] * 2 + [
                (oracle.gemm_nt, (aq, E4, sx, wdq_o, E4, swd), rm, 2 * R * d * h),
                (oracle.gemm_tn, (gq_o, E5, sg, aq, E4, sx), rd, 2 * R * h * M),
                (oracle.gemm_nn, (gq_o, E5, sg, wdq_o, E4, swd), rm, 2 * R * h * d)] + [
                (oracle.gemm_tn, (dgq, E5, sg, xq_o, E4, sx), rh, 2 * R * d * M)] * 2 + [
                (oracle.gemm_nn, (dgq, E5, sg, wgq_o, E4, swg), rm, 2 * R * d * h)] * 2
            cpu = _oracle_gemms_rate(jobs, f"{R} output rows of each of the nine GEMMs of the M={M} d={d} h={h} "
                                           "gated block")
            log(f"oracle: {cpu['value']:.4f} TFLOP/s")
        # the relu^2 block the pages chose instead, same d, 4x intermediate
        r = synth.MLP_3P8B
        xr, wur, wdr, dyr = (t(a) for a in r.tensors())
        rs = api.Relu2MlpSaved.empty(r.M, r.d, r.h, dev)
        rf, rb = api.relu2_mlp_fwd_workspace(r.M, r.d, r.h, dev), api.relu2_mlp_bwd_workspace(r.M, r.d, r.h, dev)
        Yr, DXr = torch.empty((r.M, r.d), **bf), torch.empty((r.M, r.d), **bf)
        DWUr, DWDr = torch.empty((r.h, r.d), **bf), torch.empty((r.d, r.h), **bf)
        BSr = torch.empty(2, dtype=torch.float32, device=dev)

        def step_r():
            api.relu2_mlp_fwd(xr, wur, wdr, y=Yr, saved=rs, ws=rf)
            api.relu2_mlp_bwd(dyr, rs, dx=DXr, dw_up=DWUr, dw_down=DWDr, bwd_scales=BSr, ws=rb)
        ms_r = _time_steps(step_r, args.steps, args.warmup)
        log(f"relu2 block h={r.h}: {ms_r:.3f} ms/step, {r.flops / (ms_r * 1e-3) / 1e12:.1f} TFLOP/s")
        res = {"metric": "FP8 SwiGLU MLP fwd+bwd TFLOP/s (d=3072, h=8448)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) weights, N(0,1e-3) dY with 0.1% x100 outliers; "
                       "bf16)",
               "config": {"workload": f"SwiGLU MLP block fwd+bwd M={M} d={d} h={h}", "M": M, "d": d, "h": h,
                          "gemm_flops": w.flops},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(M / (ms * 1e-3)),
               "relu2_same_width": {"h": r.h, "ms_per_step": round(ms_r, 4),
                                    "tokens_per_s_equiv": round(r.M / (ms_r * 1e-3)),
                                    "value": round(r.flops / (ms_r * 1e-3) / 1e12, 2), "unit": "TFLOP/s"},
               "roofline": roof, "cpu_baseline": cpu}
    elif args.workload == "lmce":
        from fp8_tensorwise_scaled_amd import api

        w = synth.LM_HEAD_CE
        log(f"generating LM-head CE inputs M={w.M} K={w.K} V={w.V}")
        x, wt, tg = w.tensors()
        X, W = t(x), t(wt)
        T = torch.from_numpy(tg).to(dev)
        ws = api.fp8_lm_head_ce_workspace(w.M, w.K, w.V, w.chunk, dev)
        out = dict(loss=torch.empty(1, dtype=torch.float32, device=dev),
                   dx=torch.empty((w.M, w.K), dtype=torch.bfloat16, device=dev),
                   dw=torch.empty((w.V, w.K), dtype=torch.bfloat16, device=dev),
                   scales=torch.empty(2 + (w.M + w.chunk - 1) // w.chunk, dtype=torch.float32, device=dev))
        step = lambda: api.fp8_lm_head_ce(X, W, T, w.n_classes, w.softcap, w.chunk, ws=ws, **out)
        ms = _time_steps(step, args.steps, args.warmup)
        tflops = w.flops / (ms * 1e-3) / 1e12
        log(f"LM head + CE: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s, loss {float(out['loss'][0]):.4f}")
        # dominant kernel: one chunk's logits GEMM on the call's own codes
        offs = api.lm_head_ce_layout(w.M, w.K, w.V, w.chunk)
        xq = ws[offs[0]:offs[0] + w.M * w.K].view(w.M, w.K)[:w.chunk]
        wq = ws[offs[2]:offs[2] + w.V * w.K].view(w.V, w.K)
        zbuf = torch.empty((w.chunk, w.V), dtype=torch.bfloat16, device=dev)
        sc = out["scales"]
        us = 1e3 * _time_steps(lambda: api.fp8_linear_fwd(xq, sc[0:1], wq, sc[1:2], out=zbuf), args.gemm_reps, 3)
        roof = _roofline(f"gemm_nt_kernel<0,0,256,BN,..,0> (E4M3 x E4M3; logits of one chunk, M={w.chunk} "
                         f"N={w.V} K={w.K})", "mfma", 2 * w.chunk * w.V * w.K, us, PEAK_FP8_TFLOPS, "TFLOP/s")
        log(f"chunk logits GEMM: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        del zbuf
        cpu = None
        if not args.no_cpu_baseline:
            import oracle

            R = 128
            t0 = time.perf_counter()
            oracle.lm_head_ce(x[:R], wt, tg[:R], w.n_classes, w.softcap)
            sec = time.perf_counter() - t0
            cpu = {"value": 6 * R * w.K * w.V / sec / 1e12, "unit": "TFLOP/s",
                   "cores": int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1)), "kind": "oracle",
                   "sample": f"the whole fused head + loss on the first {R} rows (quantisation of X rows and W, "
                             f"logits, CE, both gradient GEMMs; {sec:.1f} s)"}
            log(f"oracle: {sec:.1f} s")
        res = {"metric": "FP8 LM head fused with softcapped cross-entropy, fwd+bwd TFLOP/s",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) W with zero padded rows, uniform targets, "
                       "1% ignored; bf16)",
               "config": {"workload": f"LM head + softcap-{w.softcap:g} CE M={w.M} K={w.K} V={w.V} "
                                      f"classes={w.n_classes} chunk={w.chunk}", "M": w.M, "K": w.K,
                          "V": w.V, "chunk": w.chunk, "workspace_bytes": ws.numel(),
                          "logits_bytes_if_materialised": 2 * w.M * w.V},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(w.M / (ms * 1e-3)),
               "roofline": roof, "cpu_baseline": cpu}
    else:
        w = synth.LM_HEAD_PADDED
        n = synth.LM_HEAD_UNPADDED.N
        log(f"generating LM-head inputs M={w.M} K={w.K} N={w.N}")
        x, wt, g = w.tensors()
        X = t(x)
        out = {}
        for N in (w.N, n):
            W, G = t(wt[:N]), t(g[:, :N])
            r = workloads.LMHeadRunner(w.M, w.K, N, dev)
            ms = _time_steps(lambda: r.step(X, W, G), args.steps, args.warmup)
            out[N] = (ms, r.flops / (ms * 1e-3) / 1e12)
            log(f"LM head N={N}: {ms:.3f} ms/step, {out[N][1]:.1f} TFLOP/s")
            del W, G, r
        ms, tflops = out[w.N]
        res = {"metric": "FP8 LM head fwd+bwd TFLOP/s (K=3072, vocabulary 50304 padded / 50257 unpadded)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) W, N(0,1e-4) dLogits; padded rows/cols zero; bf16)",
               "config": {"workload": f"LM head fwd+bwd M={w.M} K={w.K} N={w.N}", "M": w.M, "K": w.K,
                          "N": w.N},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "unpadded": {"N": n, "ms_per_step": round(out[n][0], 4), "value": round(out[n][1], 2),
                            "unit": "TFLOP/s", "pct_of_peak": round(100 * out[n][1] / PEAK_FP8_TFLOPS, 2)}}
    res.update(common)
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gemm-reps", type=int, default=20)
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run 5 plain device copies of 256 MiB (reference for HBM byte counters)")
    ap.add_argument("--workload", choices=("mlp", "proj", "lmhead", "lmce", "rmsnorm", "swiglu", "muon"),
                    default="mlp",
                    help="mlp: the relu2 block M=8192 (default); proj: the decoder projection set at "
                         "M=32768; lmhead: the LM head at vocabulary 50304 and 50257; lmce: the LM head "
                         "fused with the softcapped cross-entropy (chunks of 8192 rows); rmsnorm: RMSNorm fused "
                         "with the quantisation of the block input X [8192, 3072]; swiglu: the gated MLP block "
                         "M=8192 d=3072 h=8448, beside the relu2 block at the same width; muon: Muon's "
                         "Newton-Schulz orthogonalisation of a 3072x12288 matrix (and its transpose)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the library runs the FP8 MLP block on one "
              "GPU (no sharding, no collectives)", file=sys.stderr)
        return 2
    if args.workload != "mlp":
        return bench_other(args)

    import numpy as np
    import torch

    from fp8_tensorwise_scaled_amd import api, synth

    w = synth.MLP_3P8B
    M, d, h = w.M, w.d, w.h
    dev = torch.device("cuda:0")
    log(f"generating inputs M={M} d={d} h={h}")
    x, wu, wd, dy = w.tensors()
    t = lambda a: torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to(dev)
    X, WU, WD, DY = t(x), t(wu), t(wd), t(dy)
    Y = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    saved = api.Relu2MlpSaved.empty(M, d, h, dev)
    ws_f = api.relu2_mlp_fwd_workspace(M, d, h, dev)
    ws_b = api.relu2_mlp_bwd_workspace(M, d, h, dev)
    DX = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    DWU = torch.empty((h, d), dtype=torch.bfloat16, device=dev)
    DWD = torch.empty((d, h), dtype=torch.bfloat16, device=dev)
    BSC = torch.empty(2, dtype=torch.float32, device=dev)

    def step():
        api.relu2_mlp_fwd(X, WU, WD, y=Y, saved=saved, ws=ws_f)
        api.relu2_mlp_bwd(DY, saved, dx=DX, dw_up=DWU, dw_down=DWD, bwd_scales=BSC, ws=ws_b)

    log(f"warmup {args.warmup}")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    clocks_before = gpu_clocks()
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    ev0.record(stream)
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = ev0.elapsed_time(ev1) / args.steps
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    flops = w.flops
    tflops = flops / (ms * 1e-3) / 1e12
    log(f"{ms:.3f} ms/step, {tflops:.1f} TFLOP/s (wall {t_wall / args.steps * 1e3:.3f} ms/step)")

    # Dominant kernel: the FP8 GEMM.  Its down-projection forward instance
    # (E4M3 x E4M3, plain bf16 store; M=8192 N=3072 K=12288) is timed on the
    # block's own operands Aq, Dq, on the same stream, averaged over launches.
    offs = api.workspace_layout("fwd", M, d, h)
    aq = ws_f[offs[3]:offs[3] + M * h].view(M, h)
    dq = ws_f[offs[2]:offs[2] + d * h].view(d, h)
    sa, sd = saved.scales[3:4], saved.scales[2:3]
    out = torch.empty((M, d), dtype=torch.bfloat16, device=dev)
    for _ in range(3):
        api.fp8_linear_fwd(aq, sa, dq, sd, out=out)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.gemm_reps):
        api.fp8_linear_fwd(aq, sa, dq, sd, out=out)
    ev1.record(stream)
    torch.cuda.synchronize()
    gemm_ms = ev0.elapsed_time(ev1) / args.gemm_reps
    gemm_flops = 2 * M * d * h
    gemm_tflops = gemm_flops / (gemm_ms * 1e-3) / 1e12
    log(f"down-proj GEMM {gemm_ms * 1e3:.1f} us, {gemm_tflops:.1f} TFLOP/s")

    # HBM-bound kernel: quantisation of a [M, h] bf16 tensor (the dH shape) to
    # row-major and transposed E5M2 codes, amax pass included.
    qx = torch.empty((M, h), dtype=torch.bfloat16, device=dev)
    qx.normal_(0.0, 1e-3)
    qq = torch.empty((M, h), dtype=torch.uint8, device=dev)
    qqt = torch.empty((h, M), dtype=torch.uint8, device=dev)
    for _ in range(3):
        api.fp8_amax_quant(qx, api.E5M2, q=qq, qt=qqt)
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(args.gemm_reps):
        api.fp8_amax_quant(qx, api.E5M2, q=qq, qt=qqt)
    ev1.record(stream)
    torch.cuda.synchronize()
    quant_ms = ev0.elapsed_time(ev1) / args.gemm_reps
    # algorithmic bytes: amax pass reads 2 B/elem; cast reads 2 B, writes 1 B + 1 B
    quant_bytes = M * h * (2 + 2 + 1 + 1)
    quant_gbs = quant_bytes / (quant_ms * 1e-3) / 1e9
    log(f"quantise [M,h] E5M2 + transpose: {quant_ms * 1e3:.1f} us, {quant_gbs:.0f} GB/s")

    if args.copy_calibration:
        cbytes = 256 << 20
        src = torch.empty(cbytes, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        log(f"copy calibration: 5 copies of {cbytes} bytes")

    result = {
        "metric": "FP8 relu² MLP fwd+bwd TFLOP/s (d=3072,h=12288) and % of dense FP8 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic (seeded N(0,1) X, N(0,0.02) weights, N(0,1e-3) dY with 0.1% x100 outliers; bf16)",
        "config": {"workload": "relu2 MLP block fwd+bwd M=8192 d=3072 h=12288", "M": M, "d": d, "h": h,
                   "formats": "E4M3 activations/weights, E5M2 gradients, fp32 accumulate, bf16 out"},
        "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "tokens_per_s_equiv": round(M / (ms * 1e-3)),
        "ms_per_step_median": round(per_step[len(per_step) // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "gpu_clocks": {"before": clocks_before, "after": gpu_clocks()},
        "roofline": {
            "kernel": "gemm_nt_kernel<0,0,256,192,4,2,0> (E4M3 x E4M3, plain store, 8 waves; down-projection fwd, "
                      "M=8192 N=3072 K=12288)",
            "bound": "mfma",
            "achieved": round(gemm_tflops, 2),
            "peak": PEAK_FP8_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(gemm_tflops / PEAK_FP8_TFLOPS, 4),
            "traffic": None,
            "avg_launch_us": round(gemm_ms * 1e3, 2),
        },
        "quantize": {
            "what": "fp8_amax_quant of a [8192, 12288] bf16 tensor to E5M2 codes and transposed codes",
            "bound": "hbm", "achieved_GBps": round(quant_gbs, 1), "peak_GBps": PEAK_HBM_GBS,
            "frac": round(quant_gbs / PEAK_HBM_GBS, 4), "us": round(quant_ms * 1e3, 2),
            "algorithmic_bytes": quant_bytes,
        },
    }
    result["roofline"]["traffic"] = measured_traffic()
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline(w)
        result["cpu_baseline"]["value"] = round(result["cpu_baseline"]["value"], 6)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
