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

`cpu_baseline` times the fp64 CPU oracle (test infrastructure, untuned) on the
same scene with all host threads (the whole frame when that takes at most 30 s,
else a row band), and `parity` compares the timed launch's image with the
oracle's over those rows.
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
PEAK_HBM_GBPS = 8000.0
FLOPS_PER_UPDATE = {"nearest": 23, "linear": 29, "sinc8": 103}
PAGE_RATE_G = 4096 * 1024 * 1024 / 0.8 / 1e9  # the page's 0.8 s per 4096 x 1024^2 frame
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "bp_linear_std_traffic.json")
# Everything that shapes the backprojection kernel or its launch: a change to any
# of these invalidates the committed counter readings.
BP_SOURCES = [os.path.join(ROOT, "domain_backprojection_amd", "csrc", f)
              for f in ("sarbp_bp.hip", "sarbp_geom.h", "sarbp_internal.h", "sarbp_plan.hip")]


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def bp_source_hash():
    """sha256 of the kernel sources' code: comments and whitespace do not count."""
    import re

    h = hashlib.sha256()
    for f in BP_SOURCES:
        text = open(f, encoding="utf-8").read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def counter_record():
    """The committed rocprofv3 counter readings of the backprojection kernel on this
    scene, or None when the kernel's sources changed since they were taken."""
    try:
        rec = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    return rec if rec.get("kernel_sources_sha256") == bp_source_hash() else None


def time_launches(fn, steps, warmup):
    """Per-launch time [ms]: the mean over `steps` back-to-back calls between two HIP events
    on the launch stream (the timed region, synchronized on both sides), then the median and
    minimum of a second pass of `steps` calls with an event after each (those events put
    a few microseconds between the launches, so they stay out of the timed region)."""
    import torch

    # At least `warmup` launches and 0.1 s of them: after an idle gap the clock takes a
    # few tens of milliseconds of load to settle.
    t0, n = time.perf_counter(), 0
    while n < warmup or time.perf_counter() - t0 < 0.1:
        fn()
        n += 1
        if n % 4 == 0:
            torch.cuda.synchronize()
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
    mean = start.elapsed_time(stop) / steps
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(stream)
    for k in range(steps):
        fn()
        ev[k + 1].record(stream)
    torch.cuda.synchronize()
    per = sorted(ev[k].elapsed_time(ev[k + 1]) for k in range(steps))
    med = per[steps // 2] if steps % 2 else 0.5 * (per[steps // 2 - 1] + per[steps // 2])
    return {"mean": mean, "median": med, "min": per[0]}, wall


def cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(scene, target_s=12.0, whole_s=30.0):
    """The fp64 oracle on host threads over the benchmark scene: the whole frame when the
    probe predicts at most whole_s seconds, else a central row band sized to about target_s;
    plus single-thread runs on the tiny scene and on 1/64 of the rows.  Returns the record
    and the oracle rows it computed (for the parity check)."""
    import oracle
    import synth

    threads = oracle.threads()
    # Probe on a band large enough that thread start-up does not dominate, then size the
    # timed band.
    rows = 32
    t = time.perf_counter()
    oracle.scene_backproject(scene, rows=(0, rows), nthreads=threads)
    dt = time.perf_counter() - t
    per_row = max(dt, 1e-3) / rows
    rows = scene.ny if per_row * scene.ny <= whole_s else int(min(scene.ny, max(rows, target_s / per_row)))
    j0 = (scene.ny - rows) // 2
    t = time.perf_counter()
    band = oracle.scene_backproject(scene, rows=(j0, j0 + rows), nthreads=threads)
    dt = time.perf_counter() - t
    upd = rows * scene.nx * scene.na

    tiny = synth.make_scene("tiny")
    t = time.perf_counter()
    oracle.scene_backproject(tiny, nthreads=1)
    dt_tiny = time.perf_counter() - t
    r64 = max(1, scene.ny // 64)
    j1 = (scene.ny - r64) // 2
    t = time.perf_counter()
    oracle.scene_backproject(scene, rows=(j1, j1 + r64), nthreads=1)
    dt_64 = time.perf_counter() - t
    rec = {"value": upd / dt / 1e9, "unit": "G pixel-pulse updates/s", "cores": threads, "kind": "oracle",
           "sample": f"rows {j0}..{j0 + rows - 1} of the {scene.nx}x{scene.ny} grid ({rows * scene.nx} px x "
                     f"{scene.na} pulses, {upd:.3e} updates, {dt:.1f} s)",
           "cpu_model": cpu_model(),
           "single_thread": {"tiny_full_G_per_s": tiny.updates / dt_tiny / 1e9,
                             "std_1_64_rows_G_per_s": r64 * scene.nx * scene.na / dt_64 / 1e9,
                             "std_1_64_rows_s": dt_64}}
    return rec, (j0, j0 + rows), band


def parity(scene, got, rows, want, peak_db=0.05):
    """The timed GPU image against the oracle's rows [j0, j1): relative L2 error over those
    pixels (all, clutter outside the target windows, the windows), and for each target whose
    window lies in the band, whether its peak is on the oracle's pixel and the magnitude
    difference there in dB."""
    import math

    import numpy as np

    import synth

    j0, j1 = rows
    g = got[j0:j1].astype(np.complex128)
    rho_az, rho_rg = synth.resolution(scene)
    hx, hy = max(1, math.ceil(rho_az / scene.dx)), max(1, math.ceil(rho_rg / scene.dy))
    mask = np.zeros(want.shape, bool)
    peaks, worst_db = [], 0.0
    for (i, j) in scene.targets:
        if j - hy < j0 or j + hy >= j1:
            continue
        sl = (slice(j - hy - j0, j + hy + 1 - j0), slice(max(0, i - hx), min(scene.nx, i + hx + 1)))
        mask[sl] = True
        gw, ow = np.abs(g[sl]), np.abs(want[sl])
        kg, ko = np.unravel_index(np.argmax(gw), gw.shape), np.unravel_index(np.argmax(ow), ow.shape)
        db = 20 * math.log10(gw[ko] / ow[ko])
        worst_db = max(worst_db, abs(db))
        peaks.append(bool(kg == ko and abs(db) <= peak_db))

    def rel(a, b):
        return float(np.linalg.norm(a - b) / np.linalg.norm(b))

    return {"rel_l2": rel(g, want), "rel_l2_clutter": rel(g[~mask], want[~mask]),
            "rel_l2_target_windows": rel(g[mask], want[mask]) if mask.any() else None,
            "peaks_ok": all(peaks), "peaks_on_oracle_pixel": f"{sum(peaks)}/{len(peaks)}",
            "max_peak_db": worst_db, "pixels": int(g.size), "rows": [int(j0), int(j1)],
            "against": "fp64 CPU oracle on the same seeded scene", "bar": {"rel_l2": 2e-3, "peak_db": peak_db}}


def aux_end_to_end(sb, steps, warmup):
    """End-to-end scene: raw LFM (4096 x 8192) -> range compression -> backprojection."""
    import torch

    import synth

    s = synth.make_scene("e2e")
    with sb.Plan.for_scene(s, n_fast=s.nr) as plan:
        raw = torch.from_numpy(s.raw).cuda()
        pos = torch.from_numpy(s.positions).cuda()
        rc = torch.empty_like(raw)
        img = plan.new_image()
        rc_t, _ = time_launches(lambda: plan.range_compress(raw, out=rc), steps, warmup)
        bp_t, _ = time_launches(lambda: plan.backproject(pos, rc, image=img), steps, warmup)
        e2e_t, _ = time_launches(lambda: (plan.range_compress(raw, out=rc), plan.backproject(pos, rc, image=img)),
                                 steps, warmup)
    rc_ms, bp_ms, e2e_ms = rc_t["mean"], bp_t["mean"], e2e_t["mean"]
    hbm = 2 * s.na * s.nr * 8  # read raw + write compressed record, bytes
    return {"workload": "end-to-end: raw LFM 4096 x 8192 -> FFT matched filter (Hamming) -> BP 1024x1024 linear",
            "rc_ms": rc_ms, "rc_ms_median": rc_t["median"], "rc_GBps_algorithmic": hbm / rc_ms / 1e6,
            "rc_frac_hbm": hbm / rc_ms / 1e6 / PEAK_HBM_GBPS, "bp_ms": bp_ms, "e2e_ms": e2e_ms,
            "e2e_G_updates_per_s": s.updates / e2e_ms / 1e6}


def aux_scenes(sb, steps, warmup):
    """Nearest on the standard geometry, sinc8 on the hi-fi (perturbed-track) scene and
    linear on the large scene (16384 pulses x 8192 bins -> 2048 x 2048)."""
    import torch

    import synth

    out = {}
    for scene, interp, key in (("std", "nearest", "nearest"), ("hifi", "sinc8", "sinc8"), ("large", "linear", "large_linear")):
        t = time.perf_counter()
        s = synth.make_scene(scene, interp=interp)
        log(f"bench: generated the {s.name} scene ({s.na} x {s.nr} echo) in {time.perf_counter() - t:.1f} s")
        with sb.Plan.for_scene(s) as plan:
            pos = torch.from_numpy(s.positions).cuda()
            echo = torch.from_numpy(s.echo).cuda()
            img = plan.new_image()
            k = steps if scene != "large" else max(5, steps // 4)
            tm, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), k, warmup)
        upd = s.updates / (tm["mean"] * 1e-3)
        out[key] = {"scene": f"{s.name}: {s.na} pulses x {s.nr} bins -> {s.nx}x{s.ny}, {interp}",
                    "ms": tm["mean"], "ms_median": tm["median"], "ms_min": tm["min"], "launches": k,
                    "G_updates_per_s": upd / 1e9, "TFLOPs_algorithmic": FLOPS_PER_UPDATE[interp] * upd / 1e12,
                    "frac_fp32_peak": FLOPS_PER_UPDATE[interp] * upd / 1e12 / PEAK_FP32_TFLOPS}
        if scene == "large":
            out["large_shards"] = aux_shards(sb, s, pos, echo, max(5, steps // 4), warmup)
        del echo, s
    return out


def aux_shards(sb, s, pos, echo, steps, warmup):
    """One GPU's share of the large scene for G = 2, 4 and 8 GPUs, at its real shape:
    a central band of ny/G image rows with every pulse (image-domain split), or the
    whole image with the middle na/G pulses (pulse-domain split).  The projected rate
    of G GPUs is the whole scene's updates over the share's time, communication
    excluded (the pulse split would add one all-reduce of the complex image)."""
    out = {}
    for G in (2, 4, 8):
        rows, npul = s.ny // G, s.na // G
        j0, p0 = (s.ny - rows) // 2, (s.na - npul) // 2
        row = {}
        with sb.Plan.for_scene(s, ny=rows, y0=s.y0 + j0 * s.dy) as plan:
            img = plan.new_image()
            tm, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), steps, warmup)
        row["image_band"] = {"pixels": [rows, s.nx], "pulses": s.na, "ms": tm["mean"],
                             "projected_G_updates_per_s": s.updates / (tm["mean"] * 1e-3) / 1e9}
        with sb.Plan.for_scene(s, n_pulses=npul) as plan:
            img = plan.new_image()
            p, e = pos[p0:p0 + npul], echo[p0:p0 + npul]
            tm, _ = time_launches(lambda: plan.backproject(p, e, image=img), steps, warmup)
        row["pulse_share"] = {"pixels": [s.ny, s.nx], "pulses": npul, "ms": tm["mean"],
                              "projected_G_updates_per_s": s.updates / (tm["mean"] * 1e-3) / 1e9}
        out[f"G{G}"] = row
    return out


def aux_accumulators(sb, scene, steps, warmup):
    """The standard scene with the two compensated accumulators."""
    import torch

    out = {}
    for accum in ("kahan", "chunk64"):
        with sb.Plan.for_scene(scene, accum=accum) as plan:
            pos = torch.from_numpy(scene.positions).cuda()
            echo = torch.from_numpy(scene.echo).cuda()
            img = plan.new_image()
            tm, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), steps, warmup)
        out[accum] = {"ms": tm["mean"], "ms_median": tm["median"],
                      "G_updates_per_s": scene.updates / (tm["mean"] * 1e-3) / 1e9}
    return out


def aux_coarse(sb, scene, steps, warmup):
    """The standard echo onto 1024 x 1024 pixels of 0.8 m and of 1 m (linear): the
    first grid's echo windows (144 bins, 3837 carrier cycles) stay on fp32 range
    differences, the second's (178 bins, 4743 cycles) are past the 4096-cycle limit
    and use the fp64-range kernels.  Both windows are far longer than the standard
    grid's (41 bins), so the staging work per pulse grows too."""
    import torch

    out = {}
    pos = torch.from_numpy(scene.positions).cuda()
    echo = torch.from_numpy(scene.echo).cuda()
    for pixel in (0.8, 1.0):
        grid = dict(dx=pixel, dy=pixel, x0=-(scene.nx // 2) * pixel, y0=-(scene.ny // 2) * pixel)
        with sb.Plan.for_scene(scene, **grid) as plan:
            img = plan.new_image()
            tm, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), steps, warmup)
        out[f"pixel_{pixel}m"] = {"ranges": "fp64" if pixel > 0.9 else "fp32", "ms": tm["mean"],
                                  "ms_median": tm["median"],
                                  "G_updates_per_s": scene.updates / (tm["mean"] * 1e-3) / 1e9}
    return out


def aux_small_grids(sb, scene, steps, warmup):
    """Grids with fewer tiles than the GPU has room for, plain and with the pulses split over
    workgroups (sarbp_backproject_split): the tiny scene (128 x 128, 256 pulses) and the
    standard echo onto the central 256 x 256 and 512 x 512 pixels (4096 pulses)."""
    import torch

    import synth

    out = {}
    t = synth.make_scene("tiny")
    cases = (("tiny_128", t, dict()),
             ("std_256", scene, dict(nx=256, ny=256, x0=scene.x0 + 384 * scene.dx, y0=scene.y0 + 384 * scene.dy)),
             ("std_512", scene, dict(nx=512, ny=512, x0=scene.x0 + 256 * scene.dx, y0=scene.y0 + 256 * scene.dy)))
    for key, s, grid in cases:
        with sb.Plan.for_scene(s, **grid) as plan:
            pos = torch.from_numpy(s.positions).cuda()
            echo = torch.from_numpy(s.echo).cuda()
            img = plan.new_image()
            need = plan.split_workspace_bytes(s.na)
            ws = torch.empty(need, dtype=torch.uint8, device="cuda")
            plain, _ = time_launches(lambda: plan.backproject(pos, echo, image=img), steps, warmup)
            split, _ = time_launches(lambda: plan.backproject(pos, echo, image=img, split=True, workspace=ws),
                                     steps, warmup)
        upd = s.na * plan.image_shape[-1] * plan.image_shape[-2]
        out[key] = {"pixels": list(plan.image_shape), "pulses": s.na, "workspace_MB": need / 1e6,
                    "plain_ms": plain["mean"], "split_ms": split["mean"],
                    "plain_G_updates_per_s": upd / plain["mean"] / 1e6,
                    "split_G_updates_per_s": upd / split["mean"] / 1e6}
    return out


def aux_host_stream(sb, scene, steps, warmup):
    """Frames fed from page-locked host memory through the two-buffer pipeline
    (PCIe-inclusive; the headline value keeps its inputs resident in HBM):
    the standard scene's echo, and the end-to-end scene's raw pulses compressed on
    the device chunk by chunk.  A plain host-to-device copy gives the link rate."""
    import torch

    import synth

    out = {}
    pos_h = torch.from_numpy(scene.positions).pin_memory()
    echo_h = torch.from_numpy(scene.echo).pin_memory()
    dev = torch.empty(echo_h.shape, dtype=echo_h.dtype, device="cuda")
    tm, _ = time_launches(lambda: dev.copy_(echo_h, non_blocking=True), steps, warmup)
    out["h2d_GBps"] = echo_h.numel() * 8 / (tm["mean"] * 1e-3) / 1e9
    del dev
    with sb.Plan.for_scene(scene, n_pulses=1024) as plan, sb.HostStream(plan, chunk=1024) as hs:
        img = plan.new_image()
        tm, _ = time_launches(lambda: hs.backproject(pos_h, echo_h, image=img), steps, warmup)
    out["std_linear"] = {"chunk": 1024, "ms": tm["mean"], "ms_median": tm["median"],
                         "G_updates_per_s": scene.updates / (tm["mean"] * 1e-3) / 1e9,
                         "input_MB": echo_h.numel() * 8 / 1e6}
    e = synth.make_scene("e2e")
    pos_h = torch.from_numpy(e.positions).pin_memory()
    raw_h = torch.from_numpy(e.raw).pin_memory()
    with sb.Plan.for_scene(e, n_fast=e.nr, n_pulses=1024) as plan, \
            sb.HostStream(plan, chunk=1024, compress=True) as hs:
        img = plan.new_image()
        tm, _ = time_launches(lambda: hs.backproject(pos_h, raw_h, image=img), steps, warmup)
    out["e2e_raw_compress"] = {"chunk": 1024, "ms": tm["mean"], "ms_median": tm["median"],
                               "G_updates_per_s": e.updates / (tm["mean"] * 1e-3) / 1e9,
                               "input_MB": raw_h.numel() * 8 / 1e6}
    return out


def aux_terrain(sb, scene, steps, warmup):
    """The standard scene's geometry and echo backprojected onto 20 m (peak to peak) of
    seeded terrain (timing only: the per-pixel height, the wider echo windows and one
    more FMA per update)."""
    import numpy as np
    import torch

    import synth

    dem = synth.terrain(scene.nx, scene.ny, scene.dx, scene.dy, np.random.Generator(np.random.PCG64(77)), 20.0)
    relief = synth.block_relief(dem)
    with sb.Plan.for_scene(scene, dem_relief=relief) as plan:
        pos = torch.from_numpy(scene.positions).cuda()
        echo = torch.from_numpy(scene.echo).cuda()
        dem_d = torch.from_numpy(dem).cuda()
        img = plan.new_image()
        tm, _ = time_launches(lambda: plan.backproject(pos, echo, image=img, dem=dem_d), steps, warmup)
    return {"relief_m": 20.0, "block_relief_m": relief, "ms": tm["mean"], "ms_median": tm["median"],
            "G_updates_per_s": scene.updates / (tm["mean"] * 1e-3) / 1e9}


def aux_volume(sb, steps, warmup):
    """3-D backprojection: 8 parallel passes (40 m apart in height) of 512 pulses each
    onto 256 x 256 x 16 voxels (0.2 m, 0.5 m layers) -- as many updates as the
    standard scene; 5 unit targets."""
    import numpy as np
    import torch

    import synth

    pos = synth.multipass_track(8, 512, 40.0)
    nr, nx, ny, nz = 4096, 256, 256, 16
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    x0, y0, z0, dz = -(nx // 2) * synth.PIXEL, -(ny // 2) * synth.PIXEL, -4.0, 0.5
    rng = np.random.Generator(np.random.PCG64(55))
    pts = np.stack([x0 + rng.integers(20, nx - 20, 5) * synth.PIXEL, y0 + rng.integers(20, ny - 20, 5) * synth.PIXEL,
                    z0 + rng.integers(0, nz, 5) * dz], 1)
    echo = synth.render_points(pos, nr, r0, synth.DR, pts, np.ones(5), half=256).astype(np.complex64)
    with sb.Plan(n_pulses=len(pos), n_range=nr, r0=r0, dr=synth.DR, nx=nx, ny=ny, x0=x0, y0=y0, z0=z0,
                 dx=synth.PIXEL, dy=synth.PIXEL, wavelength=synth.WAVELENGTH, interp="linear", nz=nz, dz=dz) as plan:
        p_d = torch.from_numpy(pos).cuda()
        e_d = torch.from_numpy(echo).cuda()
        img = plan.new_image()
        tm, _ = time_launches(lambda: plan.backproject(p_d, e_d, image=img), steps, warmup)
    upd = len(pos) * nx * ny * nz
    return {"voxels": [nz, ny, nx], "pulses": len(pos), "ms": tm["mean"], "ms_median": tm["median"],
            "G_updates_per_s": upd / (tm["mean"] * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=25,
                    help="untimed launches first; the clock takes ~20 back-to-back launches to settle")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-aux", action="store_true", help="skip the end-to-end (range compression) figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="also run a plain elementwise copy of MIB MiB (read once, write once) three times, "
                         "to scale HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported "
              "(the library runs on one device; splitting a scene over several is not implemented)", file=sys.stderr)
        sys.exit(2)

    import torch

    import synth
    from domain_backprojection_amd import sarbp

    torch.cuda.set_device(0)
    t = time.perf_counter()
    s = synth.make_scene("std")
    log(f"bench: generated the standard scene ({s.na} x {s.nr} echo, {s.nx} x {s.ny} grid) in "
        f"{time.perf_counter() - t:.1f} s")
    with sarbp.Plan.for_scene(s) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        echo = torch.from_numpy(s.echo).cuda()
        img = plan.new_image()
        torch.cuda.synchronize()
        tm, wall = time_launches(lambda: plan.backproject(pos, echo, image=img), args.steps, args.warmup)
        got = img.cpu().numpy()  # the last timed launch's image, for the parity check
    ms = tm["mean"]
    log(f"bench: {args.steps} launches, {ms:.3f} ms per launch (HIP events; median {tm['median']:.3f}, "
        f"min {tm['min']:.3f}), wall {wall:.3f} s")
    if args.calibrate_copy:
        a = torch.ones(args.calibrate_copy * 2**20 // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        for _ in range(3):
            torch.mul(a, 1.0, out=b)
        torch.cuda.synchronize()
        log(f"bench: copy calibration, {args.calibrate_copy} MiB read + {args.calibrate_copy} MiB written per launch")

    value = s.updates / (ms * 1e-3) / 1e9
    counters = counter_record()
    achieved = FLOPS_PER_UPDATE[s.interp] * s.updates / (ms * 1e-3) / 1e12
    line = {
        "metric": "giga pixel-pulse backprojections/s (1 GPU) + % of FP32 VALU roofline",
        "value": value,
        "unit": "G pixel-pulse updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "ms_median": tm["median"],
        "ms_min": tm["min"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": value / PAGE_RATE_G,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "standard scene: 4096 pulses x 4096 bins -> 1024x1024 px at 0.2 m, linear, "
                               "25 targets + per-cell clutter", "na": s.na, "nr": s.nr, "nx": s.nx, "ny": s.ny,
                   "interp": s.interp, "parallelism": "single GPU"},
        # achieved/frac: algorithmic flops (29 per linear update) over the measured launch
        # time; the counter-derived executed fp32 flops ride beside them when the
        # committed counters were taken on these kernel sources
        "roofline": {"bound": "alu", "achieved": achieved, "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_FP32_TFLOPS, "convention": "algorithmic flops per update",
                     "flops_per_update": FLOPS_PER_UPDATE[s.interp],
                     "traffic": counters["bytes_per_launch"] if counters else None},
    }
    if counters:
        executed = counters["fp32_flops_per_update_executed"] * value / 1e3
        line["roofline"].update(achieved_executed=executed, frac_executed=executed / PEAK_FP32_TFLOPS,
                                flops_per_update_executed=counters["fp32_flops_per_update_executed"])
        line["counters"] = {k: counters[k] for k in ("valu_per_update", "fp32_flops_per_update_executed",
                                                        "l2_hit_rate", "source")}
        line["counters"]["frac_executed"] = executed / PEAK_FP32_TFLOPS
    if not args.no_aux:
        line["aux"] = aux_end_to_end(sarbp, max(5, args.steps // 2), max(10, args.warmup // 2))
        line["aux"]["scenes"] = aux_scenes(sarbp, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["accumulators"] = aux_accumulators(sarbp, s, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["coarse"] = aux_coarse(sarbp, s, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["small_grids"] = aux_small_grids(sarbp, s, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["host_stream"] = aux_host_stream(sarbp, s, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["terrain"] = aux_terrain(sarbp, s, max(5, args.steps // 5), max(5, args.warmup // 5))
        line["aux"]["volume"] = aux_volume(sarbp, max(5, args.steps // 5), max(5, args.warmup // 5))
        log(f"bench: end-to-end {line['aux']}")
    if not args.no_cpu:
        line["cpu_baseline"], rows, want = cpu_baseline(s)
        log(f"bench: cpu baseline {line['cpu_baseline']}")
        line["parity"] = parity(s, got, rows, want)
        log(f"bench: parity {line['parity']}")
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
