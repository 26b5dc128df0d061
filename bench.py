"""Throughput of the backprojection hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-aux]

Workload: the standard scene -- 4096 pulses x 4096 range bins (complex64,
range compressed) backprojected onto a 1024 x 1024 grid at 0.2 m with linear
interpolation, 25 point targets plus per-cell clutter; seeded synthetic data,
resident in device memory before the timed region (host-to-device copies are
excluded, as in the page's measurement).  One step = one sarbp_backproject call
over the whole scene.  Prints one JSON line.

Roofline: the kernel is bound by the vector ALUs (fp32 FMA/add/mul plus
v_sin/v_cos), not by HBM or MFMA.  `achieved` counts the algorithmic 29 flops of
one linear pixel-pulse update (range 7, bin position 2, phase 4, sample 8,
complex multiply-accumulate 8; sqrt/sin/cos count 1) times Na*Nx*Ny per launch,
divided by the launch's average duration measured with HIP events on the
launch stream; `peak` is the MI355X vector fp32 figure, 157.3 TFLOP/s.

`cpu_baseline` times the fp64 CPU oracle (test infrastructure, untuned) on a
bounded row sample of the same scene with all host threads.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3
FLOPS_PER_UPDATE = {"nearest": 23, "linear": 29, "sinc8": 103}
PAGE_RATE_G = 4096 * 1024 * 1024 / 0.8 / 1e9  # the page's 0.8 s per 4096 x 1024^2 frame
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bp_linear_std_traffic.json")
BP_SOURCE = os.path.join(ROOT, "domain_backprojection_amd", "csrc", "sarbp_bp.hip")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def traffic_bytes():
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None when the
    kernel source changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(BP_SOURCE, "rb").read()).hexdigest()
    if rec.get("kernel_sha256") != sha:
        return None
    return rec.get("bytes_per_launch")


def time_launches(fn, steps, warmup):
    import torch

    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    start, stop = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(steps):
        fn()
    stop.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return start.elapsed_time(stop) / steps, wall


def cpu_baseline(scene, target_s=12.0):
    import numpy as np

    import oracle

    threads = oracle.threads()
    rows = 4
    t = time.perf_counter()
    oracle.scene_backproject(scene, rows=(0, rows), nthreads=threads)
    dt = time.perf_counter() - t
    rows = int(min(scene.ny, max(rows, rows * target_s / max(dt, 1e-3))))
    j0 = (scene.ny - rows) // 2
    t = time.perf_counter()
    oracle.scene_backproject(scene, rows=(j0, j0 + rows), nthreads=threads)
    dt = time.perf_counter() - t
    upd = rows * scene.nx * scene.na
    del np
    return {"value": upd / dt / 1e9, "unit": "G pixel-pulse updates/s", "cores": threads, "kind": "oracle",
            "sample": f"rows {j0}..{j0 + rows - 1} of the 1024x1024 grid ({rows * scene.nx} px x {scene.na} pulses,"
                      f" {upd:.3e} updates, {dt:.1f} s)"}


def aux_end_to_end(sb, steps, warmup):
    """End-to-end scene: raw LFM (4096 x 8192) -> range compression -> backprojection."""
    import torch

    import synth

    s = synth.make_scene(5)
    with sb.Plan.for_scene(s, n_fast=s.nr) as plan:
        raw = torch.from_numpy(s.raw).cuda()
        pos = torch.from_numpy(s.positions).cuda()
        rc = torch.empty_like(raw)
        img = plan.new_image()
        rc_ms, _ = time_launches(lambda: plan.range_compress(raw, out=rc), steps, warmup)
        bp_ms, _ = time_launches(lambda: plan.backproject(pos, rc, image=img), steps, warmup)
        e2e_ms, _ = time_launches(lambda: (plan.range_compress(raw, out=rc), plan.backproject(pos, rc, image=img)),
                                  steps, warmup)
    hbm = 2 * s.na * s.nr * 8  # read raw + write compressed record, bytes
    return {"workload": "end-to-end: raw LFM 4096 x 8192 -> FFT matched filter (Hamming) -> BP 1024x1024 linear",
            "rc_ms": rc_ms, "rc_GBps_algorithmic": hbm / rc_ms / 1e6, "bp_ms": bp_ms, "e2e_ms": e2e_ms,
            "e2e_G_updates_per_s": s.updates / e2e_ms / 1e6}


def aux_interpolators(sb, steps, warmup):
    """Nearest on the standard geometry and sinc8 on the hi-fi (perturbed-track) scene."""
    import torch

    import synth

    out = {}
    for cfg, interp in ((2, "nearest"), (4, "sinc8")):
        s = synth.make_scene(cfg, interp=interp)
        with sb.Plan.for_scene(s) as plan:
            pos = torch.from_numpy(s.positions).cuda()
            echo = torch.from_numpy(s.echo).cuda()
            img = plan.new_image()
            ms, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), steps, warmup)
        upd = s.updates / (ms * 1e-3)
        out[interp] = {"scene": s.name, "ms": ms, "G_updates_per_s": upd / 1e9,
                       "TFLOPs_algorithmic": FLOPS_PER_UPDATE[interp] * upd / 1e12,
                       "frac_fp32_peak": FLOPS_PER_UPDATE[interp] * upd / 1e12 / PEAK_FP32_TFLOPS}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-aux", action="store_true", help="skip the end-to-end (range compression) figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise copy of MIB MiB (read once, write once) three times, "
                         "to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU; --gpus {args.gpus} is not supported "
              "(the multi-GPU split is a design note, not an implemented path)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from domain_backprojection_amd import sarbp

    torch.cuda.set_device(0)
    t = time.perf_counter()
    s = synth.make_scene(2)
    log(f"bench: generated the standard scene ({s.na} x {s.nr} echo, {s.nx} x {s.ny} grid) in "
        f"{time.perf_counter() - t:.1f} s")
    with sarbp.Plan.for_scene(s) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        echo = torch.from_numpy(s.echo).cuda()
        img = plan.new_image()
        torch.cuda.synchronize()
        ms, wall = time_launches(lambda: plan.backproject(pos, echo, image=img), args.steps, args.warmup)
    log(f"bench: {args.steps} launches, {ms:.3f} ms per launch (HIP events), wall {wall:.3f} s")
    if args.calibrate_copy:
        a = torch.ones(args.calibrate_copy * 2**20 // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, {args.calibrate_copy} MiB read + {args.calibrate_copy} MiB written per launch")

    value = s.updates / (ms * 1e-3) / 1e9
    achieved = FLOPS_PER_UPDATE[s.interp] * s.updates / (ms * 1e-3) / 1e12
    line = {
        "metric": "giga pixel-pulse backprojections/s (1 GPU) + % of FP32 VALU roofline",
        "value": value,
        "unit": "G pixel-pulse updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": value / PAGE_RATE_G,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "standard scene: 4096 pulses x 4096 bins -> 1024x1024 px at 0.2 m, linear, "
                               "25 targets + per-cell clutter", "na": s.na, "nr": s.nr, "nx": s.nx, "ny": s.ny,
                   "interp": s.interp, "parallelism": "single GPU"},
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_TFLOPS, "traffic": traffic_bytes()},
    }
    if not args.no_aux:
        line["aux"] = aux_end_to_end(sarbp, max(5, args.steps // 2), args.warmup)
        line["aux"]["interpolators"] = aux_interpolators(sarbp, max(5, args.steps // 2), args.warmup)
        log(f"bench: end-to-end {line['aux']}")
    if not args.no_cpu:
        line["cpu_baseline"] = cpu_baseline(s)
        log(f"bench: cpu baseline {line['cpu_baseline']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
