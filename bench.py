"""Benchmark of the FP8/FP16 GEMM hot path on one MI355X.

One step = one pass over every step of the path, on seeded synthetic inputs
already resident in HBM (the metric's configuration: GEMMs at 4096^3 and the
M = 1 decode):
  FP8 4096^3 job:  amax, scale and E4M3 quantize of A and B (two launches),
                   then the E4M3 GEMM with an E4M3 output and its own output
                   scale (sOut = amax(C) / 448, computed once beforehand)
  FP16 4096^3:     FP16 GEMM, FP16 output
  FP16 decode:     [1,4096] x [4096,12288], FP16 output (HBM-bound kernel)
B is row-major B[K,N] (the calls' contract layout) unless --b-layout kmajor.

The timed steps hold no events (a timing event recorded between two kernels
delays the next one by about 6 us); ms_per_step is their wall time. value =
2*4096^3 / the time of one FP8 job, in TFLOPS: the throughput of the whole
FP8 job, quantization included, from batches of back-to-back jobs whose FP32
A and B rotate over copies beyond the Infinity Cache (`fp8_job`). A second
pass of the steps with HIP events between the parts splits a step into its
parts (`in_step`, each part holding one event's delay). `roofline`
is the FP8 GEMM kernel against the FP8 dense peak, `roofline_f16` the FP16
GEMM against the FP16 peak, `roofline_decode` the decode against HBM, each
timed as the median over five batches of the mean per launch of back-to-back
launches between two HIP events on the launch stream (the figure a
kernel-trace profile of the same command reports as that kernel's average
duration).

The same run times every configuration of the workload list on its own
(`rows`): for each, R back-to-back calls each bracketed by HIP events on the
launch stream, reported as median / p10 / p90 / mean, for row-major B and for
K-major B (Bt[N,K]). HBM-bound rows rotate B over enough copies (>= 512 MB)
that the 256 MB Infinity Cache cannot serve it. `clock` samples the GPU's
engine clock (amd-smi) while the FP8 GEMM runs back to back for about a
second. `cpu_baseline` is the oracle on a bounded sample of the step on the
host cores.

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import subprocess
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS + % MFMA peak (FP8/FP16 GEMM 4096³); HBM GB/s at M=1 decode"
PEAK_FP8_TFLOPS = 5033.2     # MI355X dense MFMA, FP8
PEAK_F16_TFLOPS = 2516.6     # MI355X dense MFMA, FP16
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
COLD_BYTES = 512 << 20       # rotated operand footprint for HBM-bound rows (2x the Infinity Cache)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    p.add_argument("--rows-reps", type=int, default=100, help="timed calls per row")
    p.add_argument("--no-rows", action="store_true", help="time the step only")
    p.add_argument("--no-clock", action="store_true", help="skip the engine-clock sample under load (amd-smi)")
    p.add_argument("--kernel-reps", type=int, default=30,
                   help="back-to-back launches per batch timed per roofline kernel (median of 5 batches)")
    p.add_argument("--b-layout", choices=("rowmajor", "kmajor"), default="rowmajor",
                   help="layout of B in the timed step: rowmajor (B[K,N], the contract layout) or kmajor "
                        "(Bt[N,K], a linear layer's weight layout)")
    p.add_argument("--calib-copy", action="store_true",
                   help="run one 256 MiB device-to-device copy first (a known-size kernel that calibrates "
                        "HBM byte counters in a profiler run)")
    return p.parse_args()


def traffic_record(config):
    """HBM bytes per launch of `config` from the committed counter summary, or
    None when the kernel sources have changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(config)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        fp = os.path.join(ROOT, f)
        if not os.path.exists(fp):
            return None
        h.update(open(fp, "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec


def stats_us(torch, fn, reps, warm=10):
    """Times (us) of reps calls on the current stream (the stream libgemm
    launches on): median / p10 / p90 / mean of calls each bracketed by HIP
    events, and batch_mean, the mean of reps calls launched back to back
    between two events (no event between calls)."""
    for _ in range(warm):
        fn()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(reps):
        fn()
        ev[i + 1].record()
    ev[-1].synchronize()
    d = sorted(ev[i].elapsed_time(ev[i + 1]) * 1e3 for i in range(reps))
    b0, b1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    b0.record()
    for _ in range(reps):
        fn()
    b1.record()
    b1.synchronize()
    pick = lambda q: d[min(reps - 1, int(q * (reps - 1) + 0.5))]  # noqa: E731
    return {"median": pick(0.5), "p10": pick(0.1), "p90": pick(0.9), "mean": sum(d) / reps,
            "batch_mean": b0.elapsed_time(b1) * 1e3 / reps, "calls": reps}


def host_info():
    model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    try:
        nproc = int(subprocess.run(["nproc"], capture_output=True, text=True, timeout=10).stdout.strip())
    except Exception:  # noqa: BLE001
        nproc = os.cpu_count()
    return nproc, model


def sample_clock():
    """Engine clock (MHz, mean over the XCDs) and socket power from one amd-smi call."""
    try:
        r = subprocess.run(["amd-smi", "metric", "-c", "-p", "--json"], capture_output=True, text=True, timeout=20)
        d = json.loads(r.stdout)
        g0 = d["gpu_data"][0] if isinstance(d, dict) else d[0]
        clk = [v["clk"]["value"] for k, v in g0.get("clock", {}).items()
               if k.startswith("gfx") and isinstance(v.get("clk", {}).get("value"), (int, float))]
        pw = g0.get("power", {}).get("socket_power", {})
        return {"gfx_mhz": sum(clk) / len(clk) if clk else None,
                "power_w": pw.get("value") if isinstance(pw, dict) else None}
    except Exception as e:  # noqa: BLE001
        return {"error": str(e)[:160]}


def cpu_baseline(target_s):
    """The oracle, untouched, on a bounded sample of the step: full amax +
    quantize of the FP8 operands, the FP8 and FP16 4096^3 GEMMs over a row
    sample sized to about target_s seconds, and the full M=1 decode."""
    import numpy as np

    import oracle as orc
    import workloads as wl

    w8, w16, wd = wl.C4[-1], wl.M0, wl.C3[0]
    xa, xb = wl.operand(w8, 0), wl.operand(w8, 1)
    ha, hb = wl.operand(w16, 0).view(np.uint16), wl.operand(w16, 1).view(np.uint16)
    da, db = wl.operand(wd, 0).view(np.uint16), wl.operand(wd, 1).view(np.uint16)
    t0 = time.perf_counter()
    sa = orc.scale_from_amax(orc.amax(xa))
    sb = orc.scale_from_amax(orc.amax(xb))
    qa, qb = orc.quantize(xa, sa), orc.quantize(xb, sb)
    t_quant = time.perf_counter() - t0
    t1 = time.perf_counter()
    orc.gemm(orc.FMT_E4M3, qa, qb, rows=list(range(32)))
    per_row = (time.perf_counter() - t1) / 32
    rows = int(max(32, min(w8.M, (target_s / 2) / max(per_row, 1e-9))))
    t2 = time.perf_counter()
    R, _ = orc.gemm(orc.FMT_E4M3, qa, qb, rows=list(range(rows)))
    orc.out_e4m3(R * float(sa) * float(sb), 1.0)
    t_g8 = time.perf_counter() - t2
    t3 = time.perf_counter()
    R, _ = orc.gemm(orc.FMT_F16, ha, hb, rows=list(range(rows)))
    orc.out_f16(R)
    t_g16 = time.perf_counter() - t3
    t4 = time.perf_counter()
    R, _ = orc.gemm(orc.FMT_F16, da, db)
    orc.out_f16(R)
    t_dec = time.perf_counter() - t4
    flops = 2.0 * rows * w8.N * w8.K + 2.0 * rows * w16.N * w16.K + 2.0 * wd.M * wd.N * wd.K
    total = t_quant + t_g8 + t_g16 + t_dec
    nproc, model = host_info()
    return {
        "value": flops / total / 1e12, "unit": "TFLOPS", "cores": orc.num_threads(), "kind": "oracle",
        "host_nproc": nproc, "host_cpu": model,
        "sample": (f"amax+quantize of the FP8 operands A,B [4096,4096] (full, {t_quant:.2f} s); FP8 and FP16 "
                   f"4096^3 GEMMs over the first {rows} rows of A ({t_g8:.2f} s, {t_g16:.2f} s); full M=1 decode "
                   f"1x4096x12288 ({t_dec:.2f} s); double-precision triple loop, OpenMP over rows"),
        "seconds": total,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU (every figure here is a single-GPU figure); got --gpus {args.gpus}",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import precision_dense_gemm_03_amd as g
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    g.lib()

    def to(x):
        return torch.from_numpy(np.ascontiguousarray(x)).to(dev)

    if args.calib_copy:
        src = torch.ones(64 << 20, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    kmajor = args.b_layout == "kmajor"
    w8, w16, wd = wl.C4[-1], wl.M0, wl.C3[0]
    log(f"step inputs: {w8.name}, {w16.name}, {wd.name}; B {args.b_layout}")
    xa, xb = to(wl.operand(w8, 0)), to(wl.operand(w8, 1))
    if kmajor:
        xb = xb.t().contiguous()  # quantized per tensor, so Bt's codes are B's codes transposed
    amax8, scale8 = torch.empty(2, device=dev), torch.empty(2, device=dev)
    qa = torch.empty(xa.shape, dtype=torch.uint8, device=dev)
    qb = torch.empty(xb.shape, dtype=torch.uint8, device=dev)
    ws_pair = torch.empty(g.lib().amax_quantize_fp8_pair_workspace_size(), dtype=torch.uint8, device=dev)
    c8 = torch.empty((w8.M, w8.N), dtype=torch.uint8, device=dev)
    ha, hb = to(wl.operand(w16, 0)), to(wl.operand(w16, 1))
    if kmajor:
        hb = hb.t().contiguous()
    c16 = torch.empty((w16.M, w16.N), dtype=torch.float16, device=dev)
    da = to(wl.operand(wd, 0))
    db0 = to(wl.operand(wd, 1))
    if kmajor:
        db0 = db0.t().contiguous()
    db_copies = [db0] + [db0.clone() for _ in range(max(0, COLD_BYTES // (db0.numel() * 2)))]
    cd = torch.empty((wd.M, wd.N), dtype=torch.float16, device=dev)

    gemm8 = g.gemm_fp8_scaled_bt if kmajor else g.gemm_fp8_scaled
    gemm16 = g.gemm_f16_bt if kmajor else g.gemm_f16
    sel = g.select_config_bt if kmajor else g.select_config

    # output scale of the FP8 job: amax of the FP32-output product / 448, once
    g.amax_quantize_fp8_pair(xa, xb, amax=amax8, scale=scale8, qa=qa, qb=qb, workspace=ws_pair)
    c32 = torch.empty((w8.M, w8.N), dtype=torch.float32, device=dev)
    gemm8(qa, qb, scale8[0:1], scale8[1:2], c32)
    _, s_out = g.amax_f32(c32)
    del c32
    torch.cuda.synchronize()
    rot = [0]

    def fp8_job(ev=None, inputs=None):
        a, b = inputs if inputs is not None else (xa, xb)
        g.amax_quantize_fp8_pair(a, b, amax=amax8, scale=scale8, qa=qa, qb=qb, workspace=ws_pair)
        if ev is not None:
            ev[1].record()
        gemm8(qa, qb, scale8[0:1], scale8[1:2], c8, s_out)

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        fp8_job(ev)
        if ev is not None:
            ev[2].record()
        gemm16(ha, hb, c16)
        if ev is not None:
            ev[3].record()
        gemm16(da, db_copies[rot[0] % len(db_copies)], cd)
        rot[0] += 1
        if ev is not None:
            ev[4].record()

    flops8 = 2.0 * w8.M * w8.N * w8.K
    flops16 = 2.0 * w16.M * w16.N * w16.K
    dec_bytes = 2.0 * (wd.M * wd.K + wd.K * wd.N + wd.M * wd.N)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # The timed steps hold no events: a timing event recorded between two
    # kernels delays the next one by about 6 us (measured in a kernel trace of
    # this step), which is the event's cost, not the work's.
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps

    # The step's parts: the same steps again with HIP events between the
    # parts (each part's time includes one event's delay).
    log("step parts")
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    part = lambda a, b: sum(e[a].elapsed_time(e[b]) for e in evs) / len(evs)  # noqa: E731
    ms_quant, ms_gemm8 = part(0, 1), part(1, 2)
    ms_gemm16, ms_dec = part(2, 3), part(3, 4)

    # `value`: the FP8 job (amax, scale and codes of A and B, then the GEMM)
    # back to back, A and B rotated over copies beyond the Infinity Cache so
    # that every job reads its FP32 inputs from HBM; median of five batches.
    n_in = max(2, -(-COLD_BYTES // (4 * (xa.numel() + xb.numel()))))
    job_inputs = [(xa, xb)] + [(xa.clone(), xb.clone()) for _ in range(n_in - 1)]
    jrot = [0]

    def job_call():
        fp8_job(inputs=job_inputs[jrot[0] % n_in])
        jrot[0] += 1
    log("FP8 job back to back")
    for _ in range(n_in):
        job_call()
    job_means = []
    for _ in range(5):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            job_call()
        e1.record()
        e1.synchronize()
        job_means.append(e0.elapsed_time(e1) / args.steps)
    ms_job8 = sorted(job_means)[2]
    del job_inputs
    cfg8 = sel(g.KIND_FP8, g.OUT_E4M3, w8.M, w8.N, w8.K)
    cfg16 = sel(g.KIND_F16, g.OUT_F16, w16.M, w16.N, w16.K)
    cfgd = sel(g.KIND_F16, g.OUT_F16, wd.M, wd.N, wd.K)
    in_step = {
        "fp8_quantize_pair_us": ms_quant * 1e3, "fp8_gemm_us": ms_gemm8 * 1e3,
        "f16_gemm_us": ms_gemm16 * 1e3, "decode_us": ms_dec * 1e3,
        "fp8_gemm_tflops": flops8 / ms_gemm8 / 1e9, "f16_gemm_tflops": flops16 / ms_gemm16 / 1e9,
        "decode_gbs": dec_bytes / ms_dec / 1e6,
        "what": "HIP events on the launch stream between the parts of a second pass of the steps (mean); "
                "each part includes the delay of one event record (about 6 us)"}
    job_rec = {"us": ms_job8 * 1e3, "tflops": flops8 / ms_job8 / 1e9, "input_copies": n_in,
               "what": f"median over 5 batches of {args.steps} back-to-back FP8 jobs (amax_quantize_fp8_pair on "
                       "FP32 A and B, then the E4M3-out GEMM) between two HIP events, A and B rotated over "
                       f"{n_in} copies ({n_in * 4 * (w8.M * w8.K + w8.K * w8.N) >> 20} MiB)"}

    # each roofline kernel on its own: batches of R back-to-back launches on
    # the launch stream between two HIP events (per-launch duration, launch
    # gaps included; the step's own events also hold the dependency on the
    # previous part)
    def per_launch_us(fn, reps, batches=5):
        """Median over `batches` batches of the mean per launch of `reps`
        back-to-back launches between two HIP events."""
        for _ in range(3):
            fn()
        means = []
        for _ in range(batches):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            e1.synchronize()
            means.append(e0.elapsed_time(e1) * 1e3 / reps)
        return sorted(means)[len(means) // 2]

    log("timing roofline kernels back to back")
    us_gemm8 = per_launch_us(lambda: gemm8(qa, qb, scale8[0:1], scale8[1:2], c8, s_out), args.kernel_reps)
    us_gemm16 = per_launch_us(lambda: gemm16(ha, hb, c16), args.kernel_reps)

    def dec_call():
        gemm16(da, db_copies[rot[0] % len(db_copies)], cd)
        rot[0] += 1
    us_dec = per_launch_us(dec_call, args.kernel_reps)

    rows = {}
    if not args.no_rows:
        log("timing rows")
        rows = time_rows(torch, np, g, wl, to, args.rows_reps)

    # engine clock and power while the FP8 GEMM runs back to back (~2 s queued)
    clock = []
    if not args.no_clock:
        log("clock under load")
        n_launch = int(2.0e6 / max(ms_gemm8 * 1e3, 1.0))
        sa8, sb8 = scale8[0:1], scale8[1:2]
        torch.cuda.synchronize()
        for _ in range(n_launch):
            gemm8(qa, qb, sa8, sb8, c8, s_out)
        time.sleep(0.2)
        clock = [sample_clock(), sample_clock()]
        torch.cuda.synchronize()

    def roof(bound, kernel, us, work, peak, unit, traffic=None, algo=None):
        achieved = work / us / 1e6 if unit == "TFLOP/s" else work / us / 1e3
        r = {"bound": bound, "kernel": kernel, "kernel_us": us, "achieved": achieved, "peak": peak, "unit": unit,
             "frac": achieved / peak, "traffic": traffic,
             "timing": f"median over 5 batches of the mean per launch of {args.kernel_reps} back-to-back "
                       "launches between two HIP events on the launch stream, after the timed steps"}
        if algo is not None:
            r["algorithmic_bytes"] = algo
        return r

    rec8 = traffic_record(cfg8)
    roofline = roof("mfma", f"FP8 GEMM 4096^3 E4M3 out ({cfg8})", us_gemm8, flops8, PEAK_FP8_TFLOPS, "TFLOP/s",
                    None if rec8 is None else rec8["hbm_bytes"], float(w8.M * w8.K + w8.K * w8.N + w8.M * w8.N))
    roofline["traffic_unit"] = "HBM bytes per launch (FETCH_SIZE + WRITE_SIZE, scaled by a copy kernel's counters)"
    rec16 = traffic_record(cfg16)
    roofline_f16 = roof("mfma", f"FP16 GEMM 4096^3 ({cfg16})", us_gemm16, flops16, PEAK_F16_TFLOPS, "TFLOP/s",
                        None if rec16 is None else rec16["hbm_bytes"], float(2 * (3 * 4096 * 4096)))
    recd = traffic_record(cfgd)
    roofline_dec = roof("hbm", f"FP16 decode 1x4096x12288 ({cfgd}), B rotated over {len(db_copies)} copies",
                        us_dec, dec_bytes, PEAK_HBM_GBS, "GB/s",
                        None if recd is None else recd["hbm_bytes"], dec_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args.cpu_seconds)

    ok_clk = [c for c in clock if c.get("gfx_mhz")]
    out = {
        "metric": METRIC, "value": flops8 / ms_job8 / 1e9, "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3 and fp16 operands, f32 accumulate",
        "data": "synthetic (seeded; the workload list's shapes and distributions)",
        "config": {"workload": "fp8 e4m3 4096^3 job (amax, scale, quantize of A and B; GEMM, e4m3 out) + fp16 "
                               "GEMM 4096^3 + fp16 decode 1x4096x12288", "M": 4096, "N": 4096, "K": 4096,
                   "decode": [1, 4096, 12288], "b_layout": args.b_layout,
                   "value": "FP8 job TFLOPS: 2*4096^3 / the time of one job (amax, scale and quantize of A and B, "
                            "then the GEMM with E4M3 out), see fp8_job"},
        "fp8_job": job_rec, "in_step": in_step, "roofline": roofline, "roofline_f16": roofline_f16, "roofline_decode": roofline_dec,
        "clock": {"samples": ok_clk or clock, "what": "amd-smi engine clock (mean over XCDs) and socket power, "
                  "sampled twice while the FP8 4096^3 GEMM runs back to back", "peak_mhz": 2400},
        "rows": rows, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def time_rows(torch, np, g, wl, to, reps):
    """Every configuration of the workload list, row-major and K-major B."""
    rows = {}

    def add(name, st, flops=None, nbytes=None, cfg=None, peak=None, extra=None):
        r = {"us": st, "config": cfg}
        us = st["median"]
        if flops:
            r["tflops_median"] = flops / us / 1e6
            if peak:
                r["pct_peak_median"] = 100 * flops / us / 1e6 / peak
        if nbytes:
            r["gbs_median"] = nbytes / us / 1e3
            r["pct_hbm_median"] = 100 * nbytes / us / 1e3 / PEAK_HBM_GBS
        if extra:
            r.update(extra)
        rows[name] = r
        log(f"  {name}: {us:.2f} us ({cfg})")

    def fp8_inputs(w):
        xa, xb = to(wl.operand(w, 0)), to(wl.operand(w, 1))
        _, scale, qa, qb = g.amax_quantize_fp8_pair(xa, xb)
        del xa, xb
        return qa, qb, scale

    one = torch.ones(1, device="cuda")
    # ---- FP16 GEMMs: C1 (F32 out), M0 and C5 (F16 out)
    for w in (wl.C1, wl.M0, wl.C5_F16):
        a, b = to(wl.operand(w, 0)), to(wl.operand(w, 1))
        bt = b.t().contiguous()
        c = torch.empty((w.M, w.N), dtype=torch.float32 if w.out == 0 else torch.float16, device="cuda")
        out = g.OUT_F32 if w.out == 0 else g.OUT_F16
        f = 2.0 * w.M * w.N * w.K
        n_rep = reps if w.M * w.N * w.K <= 4096 ** 3 else max(20, reps // 4)
        add(w.name, stats_us(torch, lambda: g.gemm_f16(a, b, c), n_rep), f, cfg=g.select_config(g.KIND_F16, out, w.M, w.N, w.K),
            peak=PEAK_F16_TFLOPS, extra={"b_layout": "rowmajor"})
        add(w.name + "_bt", stats_us(torch, lambda: g.gemm_f16_bt(a, bt, c), n_rep), f,
            cfg=g.select_config_bt(g.KIND_F16, out, w.M, w.N, w.K), peak=PEAK_F16_TFLOPS, extra={"b_layout": "kmajor"})
        del a, b, bt, c
    # ---- FP8 GEMMs: C2 (F32 out), C5 FP8 (F16 out)
    for w in (wl.C2, wl.C5_FP8):
        qa, qb, scale = fp8_inputs(w)
        qbt = qb.t().contiguous()
        c = torch.empty((w.M, w.N), dtype=torch.float32 if w.out == 0 else torch.float16, device="cuda")
        out = g.OUT_F32 if w.out == 0 else g.OUT_F16
        f = 2.0 * w.M * w.N * w.K
        n_rep = reps if w.M * w.N * w.K <= 4096 ** 3 else max(20, reps // 4)
        add(w.name, stats_us(torch, lambda: g.gemm_fp8_scaled(qa, qb, scale[0:1], scale[1:2], c), n_rep), f,
            cfg=g.select_config(g.KIND_FP8, out, w.M, w.N, w.K), peak=PEAK_FP8_TFLOPS, extra={"b_layout": "rowmajor"})
        add(w.name + "_bt", stats_us(torch, lambda: g.gemm_fp8_scaled_bt(qa, qbt, scale[0:1], scale[1:2], c), n_rep), f,
            cfg=g.select_config_bt(g.KIND_FP8, out, w.M, w.N, w.K), peak=PEAK_FP8_TFLOPS, extra={"b_layout": "kmajor"})
        del qa, qb, qbt, c
    # ---- C4: FP8 N = K = 4096, M swept, E4M3 output; B rotated for M <= 129
    wbig = wl.C4[-1]
    xb = to(wl.operand(wbig, 1))
    _, sb = g.amax_f32(xb)
    qb = g.quantize_fp8(xb, sb)
    del xb
    qbt = qb.t().contiguous()
    n_copies = COLD_BYTES // qb.numel()
    cold_b = [qb] + [qb.clone() for _ in range(n_copies - 1)]
    cold_bt = [qbt] + [qbt.clone() for _ in range(n_copies - 1)]
    rot = [0]
    for w in wl.C4:
        xa = to(wl.operand(w, 0))
        _, sa = g.amax_f32(xa)
        qa = g.quantize_fp8(xa, sa)
        del xa
        c32 = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
        g.gemm_fp8_scaled(qa, qb, sa, sb, c32)
        _, s_out = g.amax_f32(c32)
        del c32
        c = torch.empty((w.M, w.N), dtype=torch.uint8, device="cuda")
        cold = w.M <= 129
        f = 2.0 * w.M * w.N * w.K
        nb = float(w.M * w.K + w.K * w.N + w.M * w.N)

        def run_rm(qa=qa, sa=sa, c=c, s_out=s_out, cold=cold):
            b = cold_b[rot[0] % len(cold_b)] if cold else qb
            rot[0] += 1
            g.gemm_fp8_scaled(qa, b, sa, sb, c, s_out)

        def run_km(qa=qa, sa=sa, c=c, s_out=s_out, cold=cold):
            b = cold_bt[rot[0] % len(cold_bt)] if cold else qbt
            rot[0] += 1
            g.gemm_fp8_scaled_bt(qa, b, sa, sb, c, s_out)

        ex = {"cold": f"B rotated over {n_copies} copies" if cold else "warm"}
        add(w.name, stats_us(torch, run_rm, reps), f, nb, g.select_config(g.KIND_FP8, g.OUT_E4M3, w.M, w.N, w.K),
            PEAK_FP8_TFLOPS, dict(ex, b_layout="rowmajor"))
        add(w.name + "_bt", stats_us(torch, run_km, reps), f, nb,
            g.select_config_bt(g.KIND_FP8, g.OUT_E4M3, w.M, w.N, w.K), PEAK_FP8_TFLOPS, dict(ex, b_layout="kmajor"))
        if w.M == 4096:
            # the exact-accumulation call on the same operands (context: FP16 matrix cores)
            add(w.name + "_exact", stats_us(torch, lambda: g.gemm_fp8_exact(qa, g.FMT_E4M3, qb, g.FMT_E4M3, sa, sb, c,
                                                                            s_out), reps), f, nb,
                g.select_config_exact(g.OUT_E4M3, w.M, w.N, w.K), PEAK_F16_TFLOPS, {"b_layout": "rowmajor"})
        del qa, c
    del cold_b, cold_bt, qb, qbt
    # ---- C3: FP16 decode M in {1, 4, 16}, B rotated
    b0 = to(wl.operand(wl.C3[0], 1))
    n_copies = max(2, COLD_BYTES // (b0.numel() * 2))
    cold_b = [b0] + [b0.clone() for _ in range(n_copies - 1)]
    cold_bt = [x.t().contiguous() for x in cold_b]
    for w in wl.C3:
        a = to(wl.operand(w, 0))
        c = torch.empty((w.M, w.N), dtype=torch.float16, device="cuda")
        nb = 2.0 * (w.M * w.K + w.K * w.N + w.M * w.N)
        f = 2.0 * w.M * w.N * w.K

        def run_rm(a=a, c=c):
            g.gemm_f16(a, cold_b[rot[0] % len(cold_b)], c)
            rot[0] += 1

        def run_km(a=a, c=c):
            g.gemm_f16_bt(a, cold_bt[rot[0] % len(cold_bt)], c)
            rot[0] += 1

        ex = {"cold": f"B rotated over {n_copies} copies"}
        add(w.name, stats_us(torch, run_rm, 2 * reps), f, nb, g.select_config(g.KIND_F16, g.OUT_F16, w.M, w.N, w.K),
            extra=dict(ex, b_layout="rowmajor"))
        add(w.name + "_bt", stats_us(torch, run_km, 2 * reps), f, nb,
            g.select_config_bt(g.KIND_F16, g.OUT_F16, w.M, w.N, w.K), extra=dict(ex, b_layout="kmajor"))
        del a, c
    del cold_b, cold_bt, b0
    # ---- amax / quantize of the FP8 4096^3 operands (128 MiB of FP32)
    xa, xb = to(wl.operand(wbig, 0)), to(wl.operand(wbig, 1))
    n2 = xa.numel() + xb.numel()
    ws = torch.empty(g.lib().amax_quantize_fp8_pair_workspace_size(), dtype=torch.uint8, device="cuda")
    am, sc = torch.empty(2, device="cuda"), torch.empty(2, device="cuda")
    q1, q2 = torch.empty_like(xa, dtype=torch.uint8), torch.empty_like(xb, dtype=torch.uint8)
    add("amax_quantize_pair_2x64MiB",
        stats_us(torch, lambda: g.amax_quantize_fp8_pair(xa, xb, amax=am, scale=sc, qa=q1, qb=q2, workspace=ws), reps),
        nbytes=9.0 * n2, cfg="pair_reduce + pair_quantize",
        extra={"what": "amax, scale and E4M3 codes of A and B (4 B read twice + 1 B written per element)"})
    a1, s1 = torch.empty(1, device="cuda"), torch.empty(1, device="cuda")
    add("amax_64MiB", stats_us(torch, lambda: g.amax_f32(xa, a1, s1), reps), nbytes=4.0 * xa.numel(),
        cfg="amax_init + amax_reduce + amax_finalize")
    add("quantize_64MiB", stats_us(torch, lambda: g.quantize_fp8(xa, s1, q1), reps), nbytes=5.0 * xa.numel(),
        cfg="quantize")
    del one
    return rows


if __name__ == "__main__":
    main()
