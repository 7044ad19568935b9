"""Benchmark of the FP8/FP16 GEMM hot path on one MI355X.

One step = one pass over every step of the path on seeded synthetic inputs
already resident in HBM:
  FP8 4096^3 job:  amax(A), amax(B) (with scales), quantize(A), quantize(B),
                   E4M3 GEMM with FP8 output and its own output scale
  FP16 4096^3:     FP16 GEMM, FP16 output
  FP16 decode:     [1,4096] x [4096,12288], FP16 output (HBM-bound kernel)
With --b-layout kmajor (the default) B is held K-major, as Bt[N,K] (the layout
a linear layer keeps its weight in): the FP8 job quantizes B straight into that
layout and the GEMMs take it; with rowmajor every B is B[K,N]. The results are
the same either way.
value = all GEMM flops of a step / step time (TFLOPS). The same run also times
each row on its own, for both layouts (TFLOPS and % of MFMA peak for the two
4096^3 GEMMs; HBM GB/s at M = 1 with the weights rotated over 6 copies, 604 MB,
so the 256 MB Infinity Cache cannot serve them), the dominant kernel's
roofline figure, and the oracle on a bounded sample of the same step on the
host cores.

Prints ONE JSON line. Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "TFLOPS + % MFMA peak (FP8/FP16 GEMM 4096³); HBM GB/s at M=1 decode"
PEAK_FP8_TFLOPS = 5033.2     # MI355X dense MFMA, FP8
PEAK_F16_TFLOPS = 2516.6     # MI355X dense MFMA, FP16
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-seconds", type=float, default=15.0, help="target oracle sample time")
    p.add_argument("--rows-reps", type=int, default=200, help="launches per single-row timing")
    p.add_argument("--b-layout", choices=("kmajor", "rowmajor"), default="kmajor",
                   help="layout of B in the timed step: kmajor (Bt[N,K], a linear layer's weight layout; the FP8 "
                        "job quantizes B straight into it) or rowmajor (B[K,N])")
    p.add_argument("--calib-copy", action="store_true",
                   help="run one 256 MiB device-to-device copy first (a known-size kernel that calibrates "
                        "HBM byte counters in a profiler run)")
    return p.parse_args()


def traffic_record(config):
    """HBM bytes per launch of `config` from the committed counter summary, or
    None when the kernel source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(config)
    if not rec:
        return None
    h = hashlib.sha256()
    for f in rec["sources"]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest() != rec["source_sha256"]:
        return None
    return rec


def time_launches(torch, fn, reps, warm=10):
    """Average ms per call of fn() over reps back-to-back calls, HIP events on
    the current stream (the stream libgemm launches on)."""
    for _ in range(warm):
        fn()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    for _ in range(reps):
        fn()
    e.record()
    e.synchronize()
    return s.elapsed_time(e) / reps


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
    flops = 0.0
    t0 = time.perf_counter()
    sa = orc.scale_from_amax(orc.amax(xa))
    sb = orc.scale_from_amax(orc.amax(xb))
    qa, qb = orc.quantize(xa, sa), orc.quantize(xb, sb)
    t_quant = time.perf_counter() - t0
    # probe the GEMM rate on 32 rows, then size the sample
    t1 = time.perf_counter()
    orc.gemm(orc.FMT_E4M3, qa, qb, rows=list(range(32)))
    t_probe = time.perf_counter() - t1
    per_row = t_probe / 32
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
    return {
        "value": flops / total / 1e12, "unit": "TFLOPS", "cores": orc.num_threads(), "kind": "oracle",
        "sample": (f"amax+quantize of the FP8 operands A,B [4096,4096] (full, {t_quant:.2f} s); FP8 and FP16 "
                   f"4096^3 GEMMs over the first {rows} rows of A ({t_g8:.2f} s, {t_g16:.2f} s); full M=1 decode "
                   f"1x4096x12288 ({t_dec:.2f} s); double-precision triple loop, OpenMP over rows"),
        "seconds": total,
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (this build has no multi-GPU path); got --gpus {args.gpus}",
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

    w8, w16, wd = wl.C4[-1], wl.M0, wl.C3[0]
    log(f"inputs: {w8.name}, {w16.name}, {wd.name}")
    xa, xb = to(wl.operand(w8, 0)), to(wl.operand(w8, 1))
    qa = torch.empty(xa.shape, dtype=torch.uint8, device=dev)
    qb = torch.empty(xb.shape, dtype=torch.uint8, device=dev)
    amax_a, s_a = torch.empty(1, device=dev), torch.empty(1, device=dev)
    amax_b, s_b = torch.empty(1, device=dev), torch.empty(1, device=dev)
    c8 = torch.empty((w8.M, w8.N), dtype=torch.uint8, device=dev)
    ha, hb = to(wl.operand(w16, 0)), to(wl.operand(w16, 1))
    c16 = torch.empty((w16.M, w16.N), dtype=torch.float16, device=dev)
    da = to(wl.operand(wd, 0))
    db_copies = [to(wl.operand(wd, 1))]
    for _ in range(5):
        db_copies.append(db_copies[0].clone())
    cd = torch.empty((wd.M, wd.N), dtype=torch.float16, device=dev)
    # K-major copies of the B operands (Bt[N,K]); the FP8 job writes its own
    # K-major codes with the transposed quantize
    qbt = torch.empty((w8.N, w8.K), dtype=torch.uint8, device=dev)
    hbt = hb.t().contiguous()
    dbt_copies = [b.t().contiguous() for b in db_copies]

    # output scale of the FP8 job: amax of the FP32-output product / 448 (computed once, on the GPU)
    g.amax_f32(xa, amax_a, s_a)
    g.amax_f32(xb, amax_b, s_b)
    g.quantize_fp8(xa, s_a, qa)
    g.quantize_fp8(xb, s_b, qb)
    c32 = torch.empty((w8.M, w8.N), dtype=torch.float32, device=dev)
    g.gemm_fp8_scaled(qa, qb, s_a, s_b, c32)
    _, s_out = g.amax_f32(c32)
    del c32
    torch.cuda.synchronize()

    rot = [0]
    kmajor = args.b_layout == "kmajor"

    def fp8_job_rm(ev=None):
        g.amax_f32(xa, amax_a, s_a)
        g.amax_f32(xb, amax_b, s_b)
        g.quantize_fp8(xa, s_a, qa)
        g.quantize_fp8(xb, s_b, qb)
        if ev is not None:
            ev[0].record()
        g.gemm_fp8_scaled(qa, qb, s_a, s_b, c8, s_out)
        if ev is not None:
            ev[1].record()

    def fp8_job_km(ev=None):
        g.amax_f32(xa, amax_a, s_a)
        g.amax_f32(xb, amax_b, s_b)
        g.quantize_fp8(xa, s_a, qa)
        g.quantize_fp8_transposed(xb, s_b, qbt)
        if ev is not None:
            ev[0].record()
        g.gemm_fp8_scaled_bt(qa, qbt, s_a, s_b, c8, s_out)
        if ev is not None:
            ev[1].record()

    def f16_gemm_rm():
        g.gemm_f16(ha, hb, c16)

    def f16_gemm_km():
        g.gemm_f16_bt(ha, hbt, c16)

    def decode_rm():
        g.gemm_f16(da, db_copies[rot[0] % len(db_copies)], cd)
        rot[0] += 1

    def decode_km():
        g.gemm_f16_bt(da, dbt_copies[rot[0] % len(dbt_copies)], cd)
        rot[0] += 1

    fp8_job, f16_gemm, decode = (fp8_job_km, f16_gemm_km, decode_km) if kmajor else (fp8_job_rm, f16_gemm_rm,
                                                                                     decode_rm)

    def step(ev=None):
        fp8_job(ev)
        f16_gemm()
        decode()

    flops8 = 2.0 * w8.M * w8.N * w8.K
    flops16 = 2.0 * w16.M * w16.N * w16.K
    flopsd = 2.0 * wd.M * wd.N * wd.K
    flops_step = flops8 + flops16 + flopsd

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    # HIP events around the FP8 GEMM launch of every timed step, recorded on
    # the current stream (the one libgemm launches on): the roofline's kernel
    # time is that launch's average inside the timed region.
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    ms_gemm8_step = sum(a.elapsed_time(b) for a, b in evs) / len(evs)

    # Each row on its own (HIP events on the launch stream).
    log("timing rows")
    reps = args.rows_reps
    dec_bytes = 2.0 * (wd.M * wd.K + wd.K * wd.N + wd.M * wd.N)
    n_x = xa.numel()
    rows = {}
    for lay, sfx in (("kmajor", "_bt"), ("rowmajor", "")):
        km = lay == "kmajor"
        if km:
            gemm8 = lambda: g.gemm_fp8_scaled_bt(qa, qbt, s_a, s_b, c8, s_out)  # noqa: E731
            sel8 = g.select_config_bt(g.KIND_FP8, g.OUT_E4M3, w8.M, w8.N, w8.K)
            sel16 = g.select_config_bt(g.KIND_F16, g.OUT_F16, w16.M, w16.N, w16.K)
            seld = g.select_config_bt(g.KIND_F16, g.OUT_F16, wd.M, wd.N, wd.K)
        else:
            gemm8 = lambda: g.gemm_fp8_scaled(qa, qb, s_a, s_b, c8, s_out)  # noqa: E731
            sel8 = g.select_config(g.KIND_FP8, g.OUT_E4M3, w8.M, w8.N, w8.K)
            sel16 = g.select_config(g.KIND_F16, g.OUT_F16, w16.M, w16.N, w16.K)
            seld = g.select_config(g.KIND_F16, g.OUT_F16, wd.M, wd.N, wd.K)
        ms_gemm8 = time_launches(torch, gemm8, reps)
        ms_job8 = time_launches(torch, fp8_job_km if km else fp8_job_rm, max(20, reps // 4))
        ms_gemm16 = time_launches(torch, f16_gemm_km if km else f16_gemm_rm, reps)
        ms_dec = time_launches(torch, decode_km if km else decode_rm, reps * 2)
        rows["fp8_gemm_4096" + sfx] = {
            "tflops": flops8 / ms_gemm8 / 1e9, "pct_peak": 100 * flops8 / ms_gemm8 / 1e9 / PEAK_FP8_TFLOPS,
            "us": ms_gemm8 * 1e3, "config": sel8, "b_layout": lay}
        rows["fp8_job_4096" + sfx] = {
            "tflops": flops8 / ms_job8 / 1e9, "us": ms_job8 * 1e3,
            "what": "amax x2 + quantize x2 " + ("(B transposed into Bt[N,K]) " if km else "") + "+ FP8 GEMM (E4M3 out)"}
        rows["f16_gemm_4096" + sfx] = {
            "tflops": flops16 / ms_gemm16 / 1e9, "pct_peak": 100 * flops16 / ms_gemm16 / 1e9 / PEAK_F16_TFLOPS,
            "us": ms_gemm16 * 1e3, "config": sel16, "b_layout": lay}
        rows["decode_m1" + sfx] = {
            "gbs": dec_bytes / ms_dec / 1e6, "pct_hbm": 100 * dec_bytes / ms_dec / 1e6 / PEAK_HBM_GBS,
            "us": ms_dec * 1e3, "cold": "B rotated over 6 copies (604 MB)", "config": seld, "b_layout": lay}
    # The decode config's other sizes (M = 4; M = 16 through split-K) and the
    # E4M3 M = 1 decode of the M-sweep config, all on K-major weights rotated
    # so that the Infinity Cache cannot serve them.
    for wx in wl.C3[1:]:
        ax = to(wl.operand(wx, 0))
        cx = torch.empty((wx.M, wx.N), dtype=torch.float16, device=dev)
        plan = g.splitk_plan_bt(g.KIND_F16, g.OUT_F16, wx.M, wx.N, wx.K)
        wsx = torch.empty(plan[2], dtype=torch.uint8, device=dev) if plan[1] > 1 else None

        def dec_x(ax=ax, cx=cx, wsx=wsx):
            g.gemm_f16_splitk_bt(ax, dbt_copies[rot[0] % len(dbt_copies)], cx, workspace=wsx)
            rot[0] += 1
        ms_x = time_launches(torch, dec_x, reps * 2)
        bytes_x = 2.0 * (wx.M * wx.K + wx.K * wx.N + wx.M * wx.N)
        rows[f"decode_m{wx.M}_bt"] = {"gbs": bytes_x / ms_x / 1e6, "pct_hbm": 100 * bytes_x / ms_x / 1e6 / PEAK_HBM_GBS,
                                      "us": ms_x * 1e3, "config": plan[0], "splits": plan[1], "b_layout": "kmajor"}
        del ax, cx, wsx
    wq = wl.C4[0]
    q_copies = [torch.empty((wq.N, wq.K), dtype=torch.uint8, device=dev) for _ in range(32)]
    for q in q_copies:
        q.copy_(qbt)
    a1, c1 = qa[:1], torch.empty((1, wq.N), dtype=torch.uint8, device=dev)

    def fp8_dec():
        g.gemm_fp8_scaled_bt(a1, q_copies[rot[0] % len(q_copies)], s_a, s_b, c1, s_out)
        rot[0] += 1
    ms_q = time_launches(torch, fp8_dec, reps * 2)
    bytes_q = 1.0 * (wq.K + wq.K * wq.N + wq.N)
    rows["fp8_decode_m1_bt"] = {"gbs": bytes_q / ms_q / 1e6, "pct_hbm": 100 * bytes_q / ms_q / 1e6 / PEAK_HBM_GBS,
                                "us": ms_q * 1e3, "config": g.select_config_bt(g.KIND_FP8, g.OUT_E4M3, 1, wq.N, wq.K),
                                "cold": "B rotated over 32 copies (537 MB)", "b_layout": "kmajor"}
    del q_copies
    ms_amax = time_launches(torch, lambda: g.amax_f32(xa, amax_a, s_a), reps)
    ms_quant = time_launches(torch, lambda: g.quantize_fp8(xa, s_a, qa), reps)
    ms_quant_t = time_launches(torch, lambda: g.quantize_fp8_transposed(xb, s_b, qbt), reps)
    rows["amax_64MiB"] = {"gbs": 4.0 * n_x / ms_amax / 1e6, "us": ms_amax * 1e3}
    rows["quantize_64MiB"] = {"gbs": 5.0 * n_x / ms_quant / 1e6, "us": ms_quant * 1e3}
    rows["quantize_transposed_64MiB"] = {"gbs": 5.0 * n_x / ms_quant_t / 1e6, "us": ms_quant_t * 1e3}
    key8 = "fp8_gemm_4096" + ("_bt" if kmajor else "")
    rows[key8]["us_in_step"] = ms_gemm8_step * 1e3
    achieved = flops8 / ms_gemm8_step / 1e9
    rec = traffic_record(rows[key8]["config"])
    roofline = {"bound": "mfma", "kernel": "FP8 GEMM 4096^3 (" + rows[key8]["config"] + ")",
                "kernel_us": ms_gemm8_step * 1e3,
                "achieved": achieved, "peak": PEAK_FP8_TFLOPS, "unit": "TFLOP/s", "frac": achieved / PEAK_FP8_TFLOPS,
                "traffic": None if rec is None else rec["hbm_bytes"],
                "traffic_unit": "bytes per launch (FETCH_SIZE x2.0 + WRITE_SIZE x1.0, calibrated on a copy kernel)",
                "algorithmic_bytes": float(w8.M * w8.K + w8.K * w8.N + w8.M * w8.N)}

    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        cpu = cpu_baseline(args.cpu_seconds)

    out = {
        "metric": METRIC, "value": flops_step / (ms_step * 1e-3) / 1e12, "unit": "TFLOPS", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "fp8_e4m3+f16 (f32 accumulate)", "data": "synthetic",
        "config": {"workload": "fp8 e4m3 job 4096^3 (amax, quantize, GEMM, fp8 out) + fp16 GEMM 4096^3 + "
                               "fp16 decode 1x4096x12288", "M": 4096, "N": 4096, "K": 4096,
                   "decode": [1, 4096, 12288], "b_layout": args.b_layout},
        "rows": rows, "roofline": roofline, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
