"""Benchmark: FP8 relu^2 MLP block fwd+bwd on one MI355X.

One step = relu2_mlp_fwd + relu2_mlp_bwd on the 3.8B-model block
(M=8192 tokens, d=3072, h=12288): the quantisations of X, W_up, W_down and
dY, the relu^2 cast, the dH cast and all six FP8 GEMMs (forward NT, grad-
input NN, grad-weight TN), with inputs resident in HBM.  The metric counts
GEMM FLOPs only (12*M*d*h per step), the convention of the pages' TFLOP/s
figure.

Prints one JSON line.  --gpus > 1 is not supported: the library runs the
block on one GPU (no sharding, no collectives).  --workload selects the
other workloads (each prints its own line): linear (one FP8 linear forward,
X [256,512] W [1024,512]), mlp_small (the block at M=2048 d=768 h=3072),
proj (decoder projection set, M=32768), lmhead (LM head, vocabulary 50304
and 50257), lmce (LM head fused with the softcapped cross-entropy),
rmsnorm, swiglu and muon.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0   # MI355X dense FP8 MFMA (no sparsity)
PEAK_HBM_GBS = 8000.0      # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0  # MI355X dense bf16 MFMA (no sparsity)
GEMM_SOURCE = os.path.join(ROOT, "fp8_tensorwise_scaled_amd", "csrc", "gemm_kernel.h")
QUANT_SOURCE = os.path.join(ROOT, "fp8_tensorwise_scaled_amd", "csrc", "quant.hip")


def log(msg: str) -> None:
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def cores() -> int:
    return int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))


def cpu_model():
    try:
        return next((ln.split(":", 1)[1].strip() for ln in open("/proc/cpuinfo") if ln.startswith("model name")),
                    None)
    except OSError:
        return None


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


def measured_traffic(name: str, source: str):
    """HBM bytes per launch of a kernel from a committed rocprofv3
    FETCH_SIZE / WRITE_SIZE summary (profiles/<name>.json), or None when the
    kernel's source has changed since those counters were taken."""
    path = os.path.join(ROOT, "profiles", f"{name}.json")
    try:
        rec = json.load(open(path))
        digest = hashlib.sha256(open(source, "rb").read()).hexdigest()
    except (OSError, ValueError):
        return None
    if rec.get("source_sha256") != digest:
        return None
    return rec.get("traffic_bytes_per_launch")


def _time_steps(step, steps, warmup):
    """Average ms per call of step() over `steps` calls after `warmup`, HIP
    events on the current stream (the library launches on it)."""
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


def _timed_region(step, steps, warmup):
    """The timed region: `warmup` untimed steps, then `steps` steps bracketed
    by synchronisation and HIP events, one event between consecutive steps.
    Returns (ms per step, sorted per-step ms, wall seconds, clocks)."""
    import torch

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    clocks_before = gpu_clocks()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    t_wall = time.perf_counter() - t_wall
    ms = evs[0].elapsed_time(evs[-1]) / steps
    per = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(steps))
    return ms, per, t_wall, {"before": clocks_before, "after": gpu_clocks()}


def _after_steps(step, calls: dict, reps: int):
    """Average launch time (us) of each call in `calls`, each launch timed by
    HIP events on the launching stream right after a full step, so that the
    kernel runs in the cache and clock state it has inside the step."""
    import torch

    stream = torch.cuda.current_stream()
    tot = {k: 0.0 for k in calls}
    evs = {k: (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for k in calls}
    for _ in range(reps):
        step()
        for k, fn in calls.items():
            evs[k][0].record(stream)
            fn()
            evs[k][1].record(stream)
        torch.cuda.synchronize()
        for k in calls:
            tot[k] += evs[k][0].elapsed_time(evs[k][1])
    return {k: 1e3 * v / reps for k, v in tot.items()}


def hbm_practical(dev, nbytes=1 << 30, reps=10):
    """Practical HBM rates on this device: a device copy (read + write), a
    fill (write only) and a sum (read only) over `nbytes`, GB/s."""
    import torch

    a = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    b = torch.empty_like(a)
    x = a.view(torch.bfloat16)
    out = {}
    for name, fn, moved in (("copy_GBps", lambda: b.copy_(a), 2 * nbytes), ("fill_GBps", lambda: b.fill_(3), nbytes),
                            ("read_GBps", lambda: x.sum(), nbytes)):
        ms = _time_steps(fn, reps, 2)
        out[name] = round(moved / (ms * 1e-3) / 1e9, 1)
    del a, b
    torch.cuda.empty_cache()
    return out


def _nt_waves(accum: int) -> str:
    """Wave grid of a 256x256 NT FP8 tile: 4x2 waves on the FP8 matrix cores,
    2x2 for exact products."""
    return "4,2" if accum == 0 else "2,2"


def _roofline(kernel: str, bound: str, work: float, us: float, peak: float, unit: str, traffic=None, **extra):
    """Roofline object for one kernel: algorithmic work per launch / its
    average launch time (HIP events on the launching stream)."""
    achieved = work / (us * 1e-6) / (1e12 if unit == "TFLOP/s" else 1e9)
    r = {"kernel": kernel, "bound": bound, "achieved": round(achieved, 2), "peak": peak, "unit": unit,
         "frac": round(achieved / peak, 4), "traffic": traffic, "avg_launch_us": round(us, 2),
         "work_per_launch": work}
    r.update(extra)
    return r


def _cpu(value, unit, sample, seconds):
    return {"value": value, "unit": unit, "cores": cores(), "host_cpus": os.cpu_count(), "cpu_model": cpu_model(),
            "kind": "oracle", "sample": sample, "seconds": round(seconds, 2)}


def _common(args, unit="TFLOP/s", dtype="fp8", higher=True):
    return {"unit": unit, "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": higher,
            "scaling": "weak", "vs_baseline": None, "dtype": dtype}


def _to_dev(dev):
    import numpy as np
    import torch

    return lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)


# --------------------------------------------------------------- relu^2 block
def cpu_baseline_block(w, rows_per_gemm: int = 256):
    """The oracle's own chain of the block on a bounded sample: the four
    input quantisations, the whole up-projection H and the relu^2 cast (its
    scale needs all of H), the whole grad-input dA with dH and its cast (its
    scale needs all of dH), and `rows_per_gemm` output rows of each of the
    other four GEMMs (Y, dW_down, dW_up, dX) from the chain's own codes."""
    import numpy as np

    import oracle

    E4, E5 = oracle.E4M3, oracle.E5M2
    x, wu, wd, dy = w.tensors()
    M, d, h = w.M, w.d, w.h
    rng = np.random.default_rng(0)
    t0 = time.perf_counter()
    xq, sx, _ = oracle.quant(x, E4)
    uq, su, _ = oracle.quant(wu, E4)
    dq, sd, _ = oracle.quant(wd, E4)
    gq, sg, _ = oracle.quant(dy, E5)
    H = oracle.gemm_nt(xq, E4, sx, uq, E4, su)                       # a3, whole
    aq, sa, _ = oracle.quant(oracle.relu2(H), E4)                     # a4
    R = rows_per_gemm
    oracle.gemm_nt(aq, E4, sa, dq, E4, sd, rows=rng.choice(M, R, replace=False))         # a5 rows
    oracle.gemm_tn(gq, E5, sg, aq, E4, sa, rows=rng.choice(d, R, replace=False))         # a7 rows
    dA = oracle.gemm_nn(gq, E5, sg, dq, E4, sd)                      # a8, whole
    hq, sh, _ = oracle.quant(oracle.relu2_bwd(H, dA), E5)             # a8 epilogue, a9
    oracle.gemm_tn(hq, E5, sh, xq, E4, sx, rows=rng.choice(h, R, replace=False))         # a10 rows
    oracle.gemm_nn(hq, E5, sh, uq, E4, su, rows=rng.choice(M, R, replace=False))         # a11 rows
    sec = time.perf_counter() - t0
    flops = 2 * 2 * M * d * h + R * 2 * (d * h + h * M + d * M + d * h)
    return _cpu(flops / sec / 1e12, "TFLOP/s",
                f"the block's oracle chain (fp64 accumulation): all four input quantisations, the whole H = XqUq^T "
                f"and its relu^2 cast, the whole dA = GqDq with dH and its cast, and {R} output rows of each of Y, "
                f"dW_down, dW_up and dX from the chain's own codes ({flops / 1e12:.3f} TFLOP of "
                f"{w.flops / 1e12:.3f})", sec)


def bench_mlp(args) -> int:
    import numpy as np
    import torch

    from fp8_tensorwise_scaled_amd import api, synth

    w = synth.MLP_3P8B
    M, d, h = w.M, w.d, w.h
    dev = torch.device("cuda:0")
    log(f"generating inputs M={M} d={d} h={h}")
    t = _to_dev(dev)
    X, WU, WD, DY = (t(a) for a in w.tensors())
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, DX = torch.empty((M, d), **bf), torch.empty((M, d), **bf)
    DWU, DWD = torch.empty((h, d), **bf), torch.empty((d, h), **bf)
    BSC = torch.empty(2, dtype=torch.float32, device=dev)
    saved = api.Relu2MlpSaved.empty(M, d, h, dev)
    ws_f = api.relu2_mlp_fwd_workspace(M, d, h, dev)
    ws_b = api.relu2_mlp_bwd_workspace(M, d, h, dev)
    acc = args.accum

    def step():
        api.relu2_mlp_fwd(X, WU, WD, y=Y, saved=saved, ws=ws_f, accum=acc)
        api.relu2_mlp_bwd(DY, saved, dx=DX, dw_up=DWU, dw_down=DWD, bwd_scales=BSC, ws=ws_b, accum=acc)

    log(f"warmup {args.warmup}, timing {args.steps} steps")
    ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"{ms:.4f} ms/step, {tflops:.1f} TFLOP/s (median {per[len(per) // 2]:.4f}, wall "
        f"{wall / args.steps * 1e3:.4f} ms/step over {wall:.2f} s)")

    # Kernels of the step that the C ABI runs on their own, on the block's
    # own codes (saved set and backward workspace), each launch timed right
    # after a full step.  Both grad-weight GEMMs are one kernel instance
    # (E5M2 x E4M3, TN, 256x192 tiles, plain store), the one with the most
    # time per step: it is the roofline kernel.
    ob = api.workspace_layout("bwd", M, d, h)
    gq = ws_b[ob[0]:ob[0] + M * d].view(M, d)
    hq = ws_b[ob[2]:ob[2] + M * h].view(M, h)
    sx, su, sd, sa = (saved.scales[i:i + 1] for i in range(4))
    sg, sh = BSC[0:1], BSC[1:2]
    E4, E5 = api.E4M3, api.E5M2
    o_dw = torch.empty((d, h), **bf)
    o_du = torch.empty((h, d), **bf)
    o_dx = torch.empty((M, d), **bf)
    o_y = torch.empty((M, d), **bf)
    qx = torch.empty((M, h), **bf).normal_(0.0, 1e-3)
    qq = torch.empty((M, h), dtype=torch.uint8, device=dev)
    qs, qa = torch.empty(1, dtype=torch.float32, device=dev), torch.empty(1, dtype=torch.float32, device=dev)
    qws = torch.empty(max(api._native.lib().fp8_amax_quant_workspace_bytes(M, h), 16), dtype=torch.uint8, device=dev)
    calls = {
        "down_wgrad_TN": lambda: api.fp8_linear_wgrad(gq, sg, saved.aq, sa, E5, E4, out=o_dw, accum=acc),
        "up_wgrad_TN": lambda: api.fp8_linear_wgrad(hq, sh, saved.xq, sx, E5, E4, out=o_du, accum=acc),
        "up_dgrad_NN": lambda: api.fp8_linear_dgrad(hq, sh, saved.uq, su, E5, E4, out=o_dx, accum=acc),
        "down_fwd_NT": lambda: api.fp8_linear_fwd(saved.aq, sa, saved.dq, sd, E4, E4, out=o_y, accum=acc),
        "quantise_MxH": lambda: api.fp8_amax_quant(qx, E5, q=qq, scale=qs, amax=qa, ws=qws),
    }
    us = _after_steps(step, calls, args.gemm_reps)
    gemm_flops = 2 * M * d * h
    kernels = {k: {"us": round(v, 2), "TFLOP/s": round(gemm_flops / (v * 1e-6) / 1e12, 1)}
               for k, v in us.items() if k != "quantise_MxH"}
    for k, v in kernels.items():
        log(f"{k}: {v['us']} us, {v['TFLOP/s']} TFLOP/s")
    wg_us = (us["down_wgrad_TN"] + us["up_wgrad_TN"]) / 2
    kname = ("gemm_kernel<1,0,256,192,4,2,0,3,%d> (E5M2 x E4M3, TN grad-weight, 256x192 tiles, 8 waves, plain "
             "store; dW_down [3072,12288] and dW_up [12288,3072], reduction over the M=8192 tokens)" % acc)
    roof = _roofline(kname, "mfma", gemm_flops, wg_us, PEAK_FP8_TFLOPS, "TFLOP/s",
                     traffic=measured_traffic("gemm_tn_wgrad_traffic", GEMM_SOURCE), launches_per_step=2)
    # quantiser, algorithmic bytes of the method's two passes: the amax reads
    # 2 B/elem, the cast reads 2 B and writes 1 B.  The single-pass kernel
    # holds part of the tensor in registers between the two and reads only
    # the rest again, so its HBM traffic (the counters) is below this.
    q_bytes = M * h * 5
    q_gbs = q_bytes / (us["quantise_MxH"] * 1e-6) / 1e9
    log(f"quantise [{M},{h}] (single pass, 5 B/elem algorithmic): {us['quantise_MxH']:.1f} us, {q_gbs:.0f} GB/s")
    hbm = hbm_practical(dev)
    log(f"practical HBM: {hbm}")

    result = {
        "metric": "FP8 relu² MLP fwd+bwd TFLOP/s (d=3072,h=12288) and % of dense FP8 MFMA peak",
        "value": round(tflops, 2), "ms_per_step": round(ms, 4),
        "data": "synthetic (seeded N(0,1) X, N(0,0.02) weights, N(0,1e-3) dY with 0.1% x100 outliers; bf16)",
        "config": {"workload": "relu2 MLP block fwd+bwd M=8192 d=3072 h=12288", "M": M, "d": d, "h": h,
                   "formats": "E4M3 activations/weights, E5M2 gradients, fp32 accumulate, bf16 out",
                   "accumulation": "exact products" if acc else "FP8 matrix cores"},
        "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
        "tokens_per_s_equiv": round(M / (ms * 1e-3)),
        "ms_per_step_median": round(per[len(per) // 2], 4), "ms_per_step_min": round(per[0], 4),
        "timed_seconds": round(wall, 3), "gpu_clocks": clocks,
        "roofline": roof,
        "kernels": kernels,
        "quantize": {"what": f"fp8_amax_quant of a [{M}, {h}] bf16 tensor (the dH shape) to E5M2 codes in one "
                             "pass (amax, grid-wide wait, cast); algorithmic bytes of the two passes: the amax "
                             "reads 2 B/elem, the cast 2 B read + 1 B written per element; the kernel holds 28 "
                             "chunks of 8 values per thread on chip (19 in registers, 9 in LDS) across the "
                             "wait and reads only the rest again (traffic: the counters)",
                     "bound": "hbm", "achieved_GBps": round(q_gbs, 1), "peak_GBps": PEAK_HBM_GBS,
                     "frac": round(q_gbs / PEAK_HBM_GBS, 4), "us": round(us["quantise_MxH"], 2),
                     "algorithmic_bytes": q_bytes,
                     "traffic": measured_traffic("quant_dh_traffic", QUANT_SOURCE)},
        "hbm_practical": hbm,
    }
    result.update(_common(args))
    if not args.no_cpu_baseline:
        log("cpu baseline (the oracle's chain on a bounded sample)")
        result["cpu_baseline"] = cpu_baseline_block(w)
        log(f"cpu: {result['cpu_baseline']['value']:.5f} TFLOP/s in {result['cpu_baseline']['seconds']} s")
    print(json.dumps(result), flush=True)
    return 0


def bench_mlp_small(args) -> int:
    """The block at M=2048, d=768, h=3072 (W ~ N(0, 1/sqrt(fan_in)))."""
    import torch

    from fp8_tensorwise_scaled_amd import api, synth

    w = synth.MLP_SMALL
    M, d, h = w.M, w.d, w.h
    dev = torch.device("cuda:0")
    t = _to_dev(dev)
    X, WU, WD, DY = (t(a) for a in w.tensors())
    bf = dict(dtype=torch.bfloat16, device=dev)
    Y, DX, DWU, DWD = (torch.empty(s, **bf) for s in ((M, d), (M, d), (h, d), (d, h)))
    BSC = torch.empty(2, dtype=torch.float32, device=dev)
    saved = api.Relu2MlpSaved.empty(M, d, h, dev)
    ws_f, ws_b = api.relu2_mlp_fwd_workspace(M, d, h, dev), api.relu2_mlp_bwd_workspace(M, d, h, dev)

    def step():
        api.relu2_mlp_fwd(X, WU, WD, y=Y, saved=saved, ws=ws_f, accum=args.accum)
        api.relu2_mlp_bwd(DY, saved, dx=DX, dw_up=DWU, dw_down=DWD, bwd_scales=BSC, ws=ws_b, accum=args.accum)

    ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
    tflops = w.flops / (ms * 1e-3) / 1e12
    log(f"small block: {ms * 1e3:.1f} us/step, {tflops:.1f} TFLOP/s")
    ob = api.workspace_layout("bwd", M, d, h)
    gq = ws_b[ob[0]:ob[0] + M * d].view(M, d)
    out = torch.empty((d, h), **bf)
    us = _after_steps(step, {"g": lambda: api.fp8_linear_wgrad(gq, BSC[0:1], saved.aq, saved.scales[3:4], api.E5M2,
                                                               api.E4M3, out=out, accum=args.accum)},
                      args.gemm_reps)["g"]
    roof = _roofline(f"gemm_kernel<1,0,128,128,2,2,0,3,{args.accum}> (E5M2 x E4M3, TN grad-weight dW_down "
                     f"[{d},{h}], reduction over M={M}; 144 tiles of 128x128, two blocks per CU)", "mfma", 2 * M * d * h, us, PEAK_FP8_TFLOPS, "TFLOP/s")
    res = {"metric": "FP8 relu² MLP fwd+bwd TFLOP/s, small block (M=2048, d=768, h=3072)",
           "value": round(tflops, 2), "ms_per_step": round(ms, 5),
           "data": "synthetic (seeded N(0,1) X, N(0,1/sqrt(fan_in)) weights, N(0,1e-3) dY with 0.1% x100 "
                   "outliers; bf16)",
           "config": {"workload": f"relu2 MLP block fwd+bwd M={M} d={d} h={h}", "M": M, "d": d, "h": h,
                      "gemm_flops": w.flops},
           "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2), "tokens_per_s_equiv": round(M / (ms * 1e-3)),
           "ms_per_step_median": round(per[len(per) // 2], 5), "gpu_clocks": clocks, "roofline": roof}
    if not args.no_cpu_baseline:
        import oracle

        x, wu, wd, dy = w.tensors()
        secs = []
        for _ in range(3):
            t0 = time.perf_counter()
            oracle.mlp_bwd(dy, oracle.mlp_fwd(x, wu, wd))
            secs.append(time.perf_counter() - t0)
        sec = min(secs)
        res["cpu_baseline"] = _cpu(w.flops / sec / 1e12, "TFLOP/s",
                                   "the whole block fwd+bwd through the oracle chain (fp64 accumulation), best of 3",
                                   sec)
    res.update(_common(args))
    print(json.dumps(res), flush=True)
    return 0


def bench_linear(args) -> int:
    """One FP8 linear forward: X [256,512] N(0,1), W [1024,512] N(0,0.02), both
    quantised per call (E4M3), Y [256,1024] bf16: latency in us.  The step is
    fp8_linear_fwd_bf16 (one amax launch and one cast launch for X and W, then
    the GEMM); the five-launch sequence of separate calls is timed beside it."""
    import torch

    from fp8_tensorwise_scaled_amd import api, synth

    w = synth.LINEAR_SMALL
    x, wt = w.tensors()
    M, K = x.shape
    N = wt.shape[0]
    dev = torch.device("cuda:0")
    t = _to_dev(dev)
    X, W = t(x), t(wt)
    u8 = dict(dtype=torch.uint8, device=dev)
    f32 = dict(dtype=torch.float32, device=dev)
    xq, wq = torch.empty((M, K), **u8), torch.empty((N, K), **u8)
    sx, sw, ax, aw = (torch.empty(1, **f32) for _ in range(4))
    sc = torch.empty(2, **f32)
    L = api._native.lib()
    wsx = torch.empty(max(L.fp8_amax_quant_workspace_bytes(M, K), 16), **u8)
    wsw = torch.empty(max(L.fp8_amax_quant_workspace_bytes(N, K), 16), **u8)
    ws = torch.empty(max(L.fp8_linear_fwd_bf16_workspace_bytes(M, N, K), 16), **u8)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def step():
        api.fp8_linear_fwd_bf16(X, W, xq=xq, wq=wq, scales=sc, out=Y, ws=ws, accum=args.accum)

    def step_separate():
        api.fp8_amax_quant(X, api.E4M3, q=xq, scale=sx, amax=ax, ws=wsx)
        api.fp8_amax_quant(W, api.E4M3, q=wq, scale=sw, amax=aw, ws=wsw)
        api.fp8_linear_fwd(xq, sx, wq, sw, out=Y, accum=args.accum)

    ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
    ms_sep = _time_steps(step_separate, args.steps, args.warmup)
    gemm_us = _after_steps(step, {"g": lambda: api.fp8_linear_fwd(xq, sc[0:1], wq, sc[1:2], out=Y,
                                                                 accum=args.accum)}, args.gemm_reps)["g"]
    flops = 2 * M * N * K
    log(f"linear fwd: {ms * 1e3:.2f} us per forward (separate calls {ms_sep * 1e3:.2f} us; GEMM alone "
        f"{gemm_us:.2f} us)")
    res = {"metric": "FP8 tensorwise-scaled linear forward latency (X [256,512], W [1024,512], quantisation "
                     "included), us",
           "value": round(ms * 1e3, 3), "ms_per_step": round(ms, 6),
           "data": "synthetic (seeded N(0,1) X, N(0,0.02) W; bf16)",
           "config": {"workload": "FP8 linear forward M=256 N=1024 K=512 (quantise X, quantise W, NT GEMM)",
                      "M": M, "N": N, "K": K, "gemm_flops": flops, "entry_point": "fp8_linear_fwd_bf16"},
           "us_separate_calls": round(ms_sep * 1e3, 3),
           "us_median": round(per[len(per) // 2] * 1e3, 3), "us_min": round(per[0] * 1e3, 3),
           "tflops": round(flops / (ms * 1e-3) / 1e12, 3),
           "roofline": _roofline("gemm_kernel<0,0,128,128,2,2,0,0,%d> (E4M3 x E4M3, NT, 16 tiles of 128x128; "
                                 "latency-bound below the machine balance)" % args.accum, "mfma", flops, gemm_us,
                                 PEAK_FP8_TFLOPS, "TFLOP/s"),
           "gpu_clocks": clocks}
    if not args.no_cpu_baseline:
        import oracle

        secs = []
        for _ in range(3):
            t0 = time.perf_counter()
            q1, s1, _ = oracle.quant(x, oracle.E4M3)
            q2, s2, _ = oracle.quant(wt, oracle.E4M3)
            oracle.gemm_nt(q1, oracle.E4M3, s1, q2, oracle.E4M3, s2)
            secs.append(time.perf_counter() - t0)
        res["cpu_baseline"] = _cpu(round(min(secs) * 1e6, 1), "us",
                                   "the whole forward (both quantisations and the GEMM, fp64 accumulation), best "
                                   "of 3", min(secs))
    res.update(_common(args, unit="us", higher=False))
    print(json.dumps(res), flush=True)
    return 0


# ---------------------------------------------------------- other workloads
def bench_other(args) -> int:
    import numpy as np
    import torch

    from fp8_tensorwise_scaled_amd import api, synth, workloads

    dev = torch.device("cuda:0")
    t = _to_dev(dev)
    common = _common(args)
    E4, E5 = api.E4M3, api.E5M2
    if args.workload == "proj":
        w = synth.PROJ_SET
        log(f"generating projection-set inputs M={w.M}")
        host = {n: w.input(n) for n in w.INPUTS}
        host.update({n: w.grad(n) for n, _ in w.GRADS})
        for i, (name, _, _) in enumerate(w.projections):
            host["w_" + name] = w.weight(i)
        tens = {k: t(v) for k, v in host.items()}
        r = workloads.ProjectionSetRunner(w.M, dev, accum=args.accum)
        step = lambda: r.step(tens)
        ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
        tflops = r.flops / (ms * 1e-3) / 1e12
        log(f"projection set: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
        q = r.q
        us = _after_steps(step, {"g": lambda: api.fp8_linear_wgrad(q.gq.q, q.gq.scale, q.xq.q, q.xq.scale,
                                                                   out=q.dw, accum=args.accum)}, args.gemm_reps)["g"]
        roof = _roofline(f"gemm_kernel<1,0,256,192,4,2,0,3,{args.accum}> (E5M2 x E4M3, TN grad-weight of the Q "
                         f"projection, dW [3072,3072], reduction over M={w.M})", "mfma", 2 * w.M * 3072 * 3072, us,
                         PEAK_FP8_TFLOPS, "TFLOP/s")
        res = {"metric": "FP8 decoder projection set fwd+bwd TFLOP/s (Q,K,V,O + relu2 MLP)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) inputs, N(0,1/sqrt(fan_in)) weights, N(0,1e-3) grads "
                       "with 0.1% x100 outliers; bf16)",
               "config": {"workload": "decoder projection set fwd+bwd M=32768 d=3072 (q 3072, k/v 1024, "
                                      "o 3072, relu2 MLP 12288)", "M": w.M, "gemm_flops": r.flops},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(w.M / (ms * 1e-3)), "ms_per_step_median": round(per[len(per) // 2], 4),
               "gpu_clocks": clocks, "roofline": roof}
        if not args.no_cpu_baseline:
            import oracle

            R = 256
            rng = np.random.default_rng(1)
            t0 = time.perf_counter()
            xa = oracle.quant(host["x_attn"], oracle.E4M3)
            xo = oracle.quant(host["x_o"], oracle.E4M3)
            flops = 0
            for name, (n_in, n_out) in (("q", (3072, 3072)), ("k", (3072, 1024)), ("v", (3072, 1024)),
                                        ("o", (3072, 3072))):
                xq_, sx_, _ = xo if name == "o" else xa
                wq_, sw_, _ = oracle.quant(host["w_" + name], oracle.E4M3)
                gq_, sg_, _ = oracle.quant(host["d" + name], oracle.E5M2)
                rows = rng.choice(w.M, R, replace=False)
                oracle.gemm_nt(xq_, oracle.E4M3, sx_, wq_, oracle.E4M3, sw_, rows=rows)
                oracle.gemm_nn(gq_, oracle.E5M2, sg_, wq_, oracle.E4M3, sw_, rows=rows)
                oracle.gemm_tn(gq_, oracle.E5M2, sg_, xq_, oracle.E4M3, sx_, rows=rng.choice(n_out, R, replace=False))
                flops += 2 * R * n_in * n_out * 2 + 2 * R * n_in * w.M
            sec = time.perf_counter() - t0
            res["cpu_baseline"] = _cpu(flops / sec / 1e12, "TFLOP/s",
                                       f"the Q, K, V and O linears through the oracle (quantisations of their "
                                       f"inputs, weights and output gradients, {R} output rows of each forward, "
                                       f"grad-input and grad-weight; {flops / 1e9:.0f} GFLOP)", sec)
    elif args.workload == "lmhead":
        w = synth.LM_HEAD_PADDED
        n = synth.LM_HEAD_UNPADDED.N
        log(f"generating LM-head inputs M={w.M} K={w.K} N={w.N}")
        x, wt, g = w.tensors()
        X = t(x)
        out = {}
        for N in (w.N, n):
            W, G = t(wt[:N]), t(g[:, :N])
            r = workloads.LMHeadRunner(w.M, w.K, N, dev, accum=args.accum)
            ms, per, wall, clocks = _timed_region(lambda: r.step(X, W, G), args.steps, args.warmup)
            out[N] = (ms, r.flops / (ms * 1e-3) / 1e12, per[len(per) // 2])
            log(f"LM head N={N}: {ms:.3f} ms/step, {out[N][1]:.1f} TFLOP/s")
            if N == w.N:
                us = _after_steps(lambda: r.step(X, W, G),
                                  {"g": lambda: api.fp8_linear_fwd(r.xq.q, r.xq.scale, r.wq.q, r.wq.scale, out=r.y,
                                                                   accum=args.accum)}, args.gemm_reps)["g"]
                roof = _roofline(f"gemm_kernel<0,0,256,256,{_nt_waves(args.accum)},0,0,{args.accum}> (E4M3 x E4M3, NT logits "
                                 f"[{w.M},{w.N}], K={w.K})", "mfma", 2 * w.M * w.N * w.K, us, PEAK_FP8_TFLOPS,
                                 "TFLOP/s")
            del W, G, r
        ms, tflops, med = out[w.N]
        res = {"metric": "FP8 LM head fwd+bwd TFLOP/s (K=3072, vocabulary 50304 padded / 50257 unpadded)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) W, N(0,1e-4) dLogits; padded rows/cols zero; bf16)",
               "config": {"workload": f"LM head fwd+bwd M={w.M} K={w.K} N={w.N}", "M": w.M, "K": w.K, "N": w.N},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2), "ms_per_step_median": round(med, 4),
               "unpadded": {"N": n, "ms_per_step": round(out[n][0], 4), "value": round(out[n][1], 2),
                            "unit": "TFLOP/s", "pct_of_peak": round(100 * out[n][1] / PEAK_FP8_TFLOPS, 2)},
               "roofline": roof}
        if not args.no_cpu_baseline:
            import oracle

            R = 64
            rng = np.random.default_rng(2)
            t0 = time.perf_counter()
            xq_, sx_, _ = oracle.quant(x, oracle.E4M3)
            wq_, sw_, _ = oracle.quant(wt, oracle.E4M3)
            gq_, sg_, _ = oracle.quant(g, oracle.E5M2)
            rows = rng.choice(w.M, R, replace=False)
            oracle.gemm_nt(xq_, oracle.E4M3, sx_, wq_, oracle.E4M3, sw_, rows=rows)
            oracle.gemm_nn(gq_, oracle.E5M2, sg_, wq_, oracle.E4M3, sw_, rows=rows)
            oracle.gemm_tn(gq_, oracle.E5M2, sg_, xq_, oracle.E4M3, sx_, rows=rng.choice(w.N, R, replace=False))
            sec = time.perf_counter() - t0
            flops = 2 * R * w.N * w.K * 2 + 2 * R * w.K * w.M
            res["cpu_baseline"] = _cpu(flops / sec / 1e12, "TFLOP/s",
                                       f"the padded head through the oracle: quantisations of X, W and dLogits, {R} "
                                       f"rows of the logits, of dX and of dW ({flops / 1e9:.0f} GFLOP)", sec)
    elif args.workload == "rmsnorm":
        M, d = 8192, 3072
        log(f"generating RMSNorm inputs [{M}, {d}]")
        X = t(synth.normal_bf16((M, d), 2.5, 3001))
        G = t(synth.normal_bf16((d,), 1.0, 3002))
        q = torch.empty((M, d), dtype=torch.uint8, device=dev)
        sc, am, rs = (torch.empty(n, dtype=torch.float32, device=dev) for n in (1, 1, M))
        ws = torch.empty(1 << 16, dtype=torch.uint8, device=dev)
        fused = lambda: api.fp8_rmsnorm_quant(X, G, 1e-6, E4, q=q, scale=sc, amax=am, rstd=rs, ws=ws)

        def unfused():  # torch's RMSNorm writing X, then the quantiser reading it
            xn = torch.nn.functional.rms_norm(X, (d,), G, 1e-6)
            api.fp8_amax_quant(xn, E4, q=q, scale=sc, amax=am, ws=ws)
        ms = _time_steps(fused, args.steps * 5, args.warmup)
        ms_unf = _time_steps(unfused, args.steps * 5, args.warmup)
        nbytes = M * d * 5 + M * 4   # x read twice (statistics, cast), codes written, r written
        gbs = nbytes / (ms * 1e-3) / 1e9
        log(f"RMSNorm + quantise: {ms * 1e3:.1f} us ({gbs:.0f} GB/s); torch rms_norm then quantise: "
            f"{ms_unf * 1e3:.1f} us")
        res = {"metric": "RMSNorm fused with FP8 tensorwise quantisation, GB/s",
               "value": round(gbs, 1), "ms_per_step": round(ms, 5),
               "data": "synthetic (seeded N(0,2.5) rows, N(0,1) weight; bf16)",
               "config": {"workload": f"RMSNorm + E4M3 quantisation of X [{M}, {d}], eps 1e-6", "M": M, "d": d,
                          "algorithmic_bytes": nbytes},
               "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                            "frac": round(gbs / PEAK_HBM_GBS, 4), "traffic": None},
               "unfused_torch_rmsnorm_then_quantise_ms": round(ms_unf, 5)}
        if not args.no_cpu_baseline:
            import oracle

            R = 1024
            xs, gs = synth.normal_bf16((M, d), 2.5, 3001)[:R], synth.normal_bf16((d,), 1.0, 3002)
            t0 = time.perf_counter()
            oracle.rmsnorm_quant(xs, gs, 1e-6, oracle.E4M3)
            sec = time.perf_counter() - t0
            res["cpu_baseline"] = _cpu(R * d * 5 / sec / 1e9, "GB/s",
                                       f"RMSNorm + quantisation of the first {R} rows", sec)
        common["unit"] = "GB/s"
    elif args.workload == "muon":
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
        bf = dict(dtype=torch.bfloat16, device=dev)
        Bm = (torch.randn((m, m), device=dev) / m).to(torch.bfloat16)
        Xm = (torch.randn((m, n), device=dev) / 6000).to(torch.bfloat16)
        Xt, Xt2 = Xm.t().contiguous(), torch.empty((n, m), **bf)
        us = 1e3 * _time_steps(lambda: api.bf16_gemm_nt(Bm, Xt, 1.0, 3.4445, Xm, out=Xm, out_t=Xt2),
                               args.gemm_reps, 3)
        roof = _roofline(f"gemm_kernel<2,2,256,192,4,2,5,0,0> (bf16, alpha/beta epilogue with transposed store; "
                         f"X = B X + a X, M={m} N={n} K={m})", "mfma", 2 * m * n * m, us, PEAK_BF16_TFLOPS,
                         "TFLOP/s")
        log(f"X = B X + a X: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        res = {"metric": "Muon Newton-Schulz orthogonalisation (5 steps, bf16 matrix cores), TFLOP/s",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,0.02) gradient with 0.1% x100 outliers; bf16)",
               "config": {"workload": f"Newton-Schulz 5 steps on a {rows}x{cols} matrix (grad of W_down; "
                                      f"the transposed W_up shape beside it)", "rows": rows, "cols": cols,
                          "steps": steps, "flops": flops},
               "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
               "tall": {"rows": cols, "cols": rows, "ms": round(res_all[(cols, rows)], 4)}, "roofline": roof}
        if not args.no_cpu_baseline:
            import oracle

            g = synth.normal_bf16((rows, cols), 0.02, 4001, outlier_frac=1e-3)
            t0 = time.perf_counter()
            oracle.newton_schulz(g)
            sec = time.perf_counter() - t0
            res["cpu_baseline"] = _cpu(flops / sec / 1e12, "TFLOP/s",
                                       f"the whole {rows}x{cols} orthogonalisation (fp64 BLAS products, bf16 "
                                       f"roundings)", sec)
        common["dtype"] = "bf16"
    elif args.workload == "swiglu":
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
            api.swiglu_mlp_fwd(X, WG, WU, WD, y=Y, saved=saved, ws=ws_f, accum=args.accum)
            api.swiglu_mlp_bwd(DY, saved, dx=DX, dw_gate=DWG, dw_up=DWU, dw_down=DWD, bwd_scales=BSC, ws=ws_b,
                               accum=args.accum)
        ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
        tflops = w.flops / (ms * 1e-3) / 1e12
        log(f"SwiGLU block: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s")
        gb, ub, ab = torch.empty((M, h), **bf), torch.empty((M, h), **bf), torch.empty((M, h), **bf)
        sc = saved.scales
        us = _after_steps(step, {"g": lambda: api.fp8_gated_linear_fwd(saved.xq, sc[0:1], saved.wgq, sc[1:2],
                                                                      saved.wuq, sc[2:3], g=gb, u=ub, a=ab,
                                                                      accum=args.accum)}, args.gemm_reps)["g"]
        roof = _roofline(f"gemm_kernel<0,0,256,256,2,2,6,0,{args.accum}> (E4M3 x E4M3; merged gate/up projection "
                         f"with the gate epilogue, M={M} N=2x{h} K={d})", "mfma", 2 * M * 2 * h * d, us,
                         PEAK_FP8_TFLOPS, "TFLOP/s")
        log(f"merged gate/up GEMM: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        del ws_f, ws_b, saved, gb, ub, ab
        r = synth.MLP_3P8B
        xr, wur, wdr, dyr = (t(a) for a in r.tensors())
        rs = api.Relu2MlpSaved.empty(r.M, r.d, r.h, dev)
        rf, rb = api.relu2_mlp_fwd_workspace(r.M, r.d, r.h, dev), api.relu2_mlp_bwd_workspace(r.M, r.d, r.h, dev)
        Yr, DXr = torch.empty((r.M, r.d), **bf), torch.empty((r.M, r.d), **bf)
        DWUr, DWDr = torch.empty((r.h, r.d), **bf), torch.empty((r.d, r.h), **bf)
        BSr = torch.empty(2, dtype=torch.float32, device=dev)

        def step_r():
            api.relu2_mlp_fwd(xr, wur, wdr, y=Yr, saved=rs, ws=rf, accum=args.accum)
            api.relu2_mlp_bwd(dyr, rs, dx=DXr, dw_up=DWUr, dw_down=DWDr, bwd_scales=BSr, ws=rb, accum=args.accum)
        ms_r = _time_steps(step_r, args.steps, args.warmup)
        log(f"relu2 block h={r.h}: {ms_r:.3f} ms/step, {r.flops / (ms_r * 1e-3) / 1e12:.1f} TFLOP/s")
        res = {"metric": "FP8 SwiGLU MLP fwd+bwd TFLOP/s (d=3072, h=8448)",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) weights, N(0,1e-3) dY with 0.1% x100 outliers; "
                       "bf16)",
               "config": {"workload": f"SwiGLU MLP block fwd+bwd M={M} d={d} h={h}", "M": M, "d": d, "h": h,
                          "gemm_flops": w.flops},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(M / (ms * 1e-3)), "ms_per_step_median": round(per[len(per) // 2], 4),
               "relu2_same_width": {"h": r.h, "ms_per_step": round(ms_r, 4),
                                    "tokens_per_s_equiv": round(r.M / (ms_r * 1e-3)),
                                    "value": round(r.flops / (ms_r * 1e-3) / 1e12, 2), "unit": "TFLOP/s"},
               "roofline": roof}
        if not args.no_cpu_baseline:
            import oracle

            x, wg, wu, wd, dy = w.tensors()
            R = 256
            rng = np.random.default_rng(0)
            t0 = time.perf_counter()
            xq_, sx_, _ = oracle.quant(x, oracle.E4M3)
            wgq_, swg_, _ = oracle.quant(wg, oracle.E4M3)
            wuq_, swu_, _ = oracle.quant(wu, oracle.E4M3)
            wdq_, swd_, _ = oracle.quant(wd, oracle.E4M3)
            gq_, sg_, _ = oracle.quant(dy, oracle.E5M2)
            rows = rng.choice(M, R, replace=False)
            G_ = oracle.gemm_nt(xq_, oracle.E4M3, sx_, wgq_, oracle.E4M3, swg_, rows=rows)
            U_ = oracle.gemm_nt(xq_, oracle.E4M3, sx_, wuq_, oracle.E4M3, swu_, rows=rows)
            dA_ = oracle.gemm_nn(gq_, oracle.E5M2, sg_, wdq_, oracle.E4M3, swd_, rows=rows)
            oracle.swiglu_gate(G_, U_)
            oracle.swiglu_gate_bwd(G_, U_, dA_)
            sec = time.perf_counter() - t0
            flops = 3 * 2 * R * h * d
            res["cpu_baseline"] = _cpu(flops / sec / 1e12, "TFLOP/s",
                                       f"the gated block's oracle stages on {R} token rows: the input "
                                       f"quantisations, G, U and dA rows and the gate forward and backward "
                                       f"({flops / 1e9:.0f} GFLOP)", sec)
    elif args.workload == "lmce":
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
        step = lambda: api.fp8_lm_head_ce(X, W, T, w.n_classes, w.softcap, w.chunk, ws=ws, accum=args.accum, **out)
        ms, per, wall, clocks = _timed_region(step, args.steps, args.warmup)
        tflops = w.flops / (ms * 1e-3) / 1e12
        log(f"LM head + CE: {ms:.3f} ms/step, {tflops:.1f} TFLOP/s, loss {float(out['loss'][0]):.4f}")
        offs = api.lm_head_ce_layout(w.M, w.K, w.V, w.chunk)
        xq = ws[offs[0]:offs[0] + w.M * w.K].view(w.M, w.K)[:w.chunk]
        wq = ws[offs[1]:offs[1] + w.V * w.K].view(w.V, w.K)
        zbuf = torch.empty((w.chunk, w.V), dtype=torch.bfloat16, device=dev)
        sc = out["scales"]
        us = _after_steps(step, {"g": lambda: api.fp8_linear_fwd(xq, sc[0:1], wq, sc[1:2], out=zbuf,
                                                                 accum=args.accum)}, args.gemm_reps)["g"]
        roof = _roofline(f"gemm_kernel<0,0,256,256,{_nt_waves(args.accum)},0,0,{args.accum}> (E4M3 x E4M3; logits of one chunk, "
                         f"M={w.chunk} N={w.V} K={w.K})", "mfma", 2 * w.chunk * w.V * w.K, us, PEAK_FP8_TFLOPS,
                         "TFLOP/s")
        log(f"chunk logits GEMM: {us:.1f} us, {roof['achieved']:.1f} TFLOP/s")
        del zbuf
        res = {"metric": "FP8 LM head fused with softcapped cross-entropy, fwd+bwd TFLOP/s",
               "value": round(tflops, 2), "ms_per_step": round(ms, 4),
               "data": "synthetic (seeded N(0,1) X, N(0,0.02) W with zero padded rows, uniform targets, "
                       "1% ignored; bf16)",
               "config": {"workload": f"LM head + softcap-{w.softcap:g} CE M={w.M} K={w.K} V={w.V} "
                                      f"classes={w.n_classes} chunk={w.chunk}", "M": w.M, "K": w.K,
                          "V": w.V, "chunk": w.chunk, "workspace_bytes": ws.numel(),
                          "logits_bytes_if_materialised": 2 * w.M * w.V},
               "pct_of_peak": round(100 * tflops / PEAK_FP8_TFLOPS, 2),
               "tokens_per_s_equiv": round(w.M / (ms * 1e-3)), "ms_per_step_median": round(per[len(per) // 2], 4),
               "roofline": roof}
        if not args.no_cpu_baseline:
            import oracle

            R = 128
            t0 = time.perf_counter()
            oracle.lm_head_ce(x[:R], wt, tg[:R], w.n_classes, w.softcap)
            sec = time.perf_counter() - t0
            res["cpu_baseline"] = _cpu(6 * R * w.K * w.V / sec / 1e12, "TFLOP/s",
                                       f"the whole fused head + loss on the first {R} rows (quantisation of X rows "
                                       f"and W, logits, CE, both gradient GEMMs)", sec)
    res.update(common)
    print(json.dumps(res), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None, help="timed steps (default: about 1 s of GPU time)")
    ap.add_argument("--warmup", type=int, default=None, help="untimed steps first (default: about 0.2 s)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--gemm-reps", type=int, default=20)
    ap.add_argument("--accum", type=int, choices=(0, 1), default=0,
                    help="0: FP8 matrix-core accumulation (the throughput path), 1: exact products")
    ap.add_argument("--workload", default="mlp",
                    choices=("mlp", "mlp_small", "linear", "proj", "lmhead", "lmce", "rmsnorm", "swiglu", "muon"),
                    help="mlp: the relu2 block M=8192 d=3072 h=12288 (default); mlp_small: the block at M=2048 "
                         "d=768 h=3072; linear: one FP8 linear forward X [256,512] W [1024,512]; proj: the "
                         "decoder projection set at M=32768; lmhead: the LM head at vocabulary 50304 and 50257; "
                         "lmce: the LM head fused with the softcapped cross-entropy; rmsnorm: RMSNorm fused with "
                         "the quantisation of X [8192, 3072]; swiglu: the gated MLP block M=8192 d=3072 h=8448; "
                         "muon: Newton-Schulz orthogonalisation of a 3072x12288 matrix")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported; the library runs the FP8 MLP block on one "
              "GPU (no sharding, no collectives)", file=sys.stderr)
        return 2
    # defaults: about 1 s of timed GPU work after about 0.2 s of warm-up
    per_step_ms = {"mlp": 1.9, "mlp_small": 0.09, "linear": 0.02, "proj": 11.0, "lmhead": 8.0, "lmce": 8.5,
                   "rmsnorm": 0.25, "swiglu": 2.3, "muon": 2.3}[args.workload]
    if args.steps is None:
        args.steps = max(20, int(round(1000.0 / per_step_ms)))
    if args.warmup is None:
        args.warmup = max(5, int(round(200.0 / per_step_ms)))
    if args.workload == "mlp":
        return bench_mlp(args)
    if args.workload == "mlp_small":
        return bench_mlp_small(args)
    if args.workload == "linear":
        return bench_linear(args)
    return bench_other(args)


if __name__ == "__main__":
    sys.exit(main())
