"""Host emulation of the backprojection kernels' index arithmetic (sarbp_check_indices; no GPU).

The library runs, on the CPU, the kernels' own tile frames, per-pulse set-up, staging index
steps and per-pixel window positions (compiled from the same source for the host) and counts
every index outside its LDS window or staging range, and every nearest-bin decision that leaves
the fp64 tie band yet differs from the definition's floor(u + 1/2).  The page's section 4.4
names out-of-window reads as the usual cause of a noisy image and asks for such a check.

Each geometry must give zero out-of-range indices, zero nearest escapes, and window-position
errors below the bound the tie band is built from (error / bound < 1)."""
import ctypes
import math
import os
import subprocess
import tempfile

import numpy as np
import pytest

import synth
from test_gpu_random import N_CASES, random_case

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TIE_MAX = 2.5e-4  # the largest band the fp32 nearest kernels accept on a 64 x 32 tile (BP_NEAREST_TIE_MAX)


@pytest.fixture(scope="module")
def sb():
    from domain_backprojection_amd import sarbp

    return sarbp


def _assert_clean(rep, what):
    assert rep["window_violations"] == 0, (what, rep)
    assert rep["staging_violations"] == 0, (what, rep)
    assert rep["nearest_escapes"] == 0, (what, rep)
    assert rep["nearest_recheck_clamped"] == 0, (what, rep)
    assert rep["max_error_to_band"] < 1.0, (what, rep)
    assert rep["min_position"] >= 0.0 and rep["max_position_margin"] < 0.0, (what, rep)
    # deferred nearest rechecks: one queued word per lane and chunk with a decision in the band, so
    # never more words than rechecked decisions, and words exactly when there are rechecks
    if rep["tie_queue_capacity"] > 0:
        assert rep["fp64_ranges"] == 0, (what, rep)
        assert 0 < rep["tie_queue_words"] <= rep["nearest_rechecks"] or rep["nearest_rechecks"] == 0 == rep[
            "tie_queue_words"], (what, rep)
        assert rep["tie_queue_tile_max"] <= rep["tie_queue_words"], (what, rep)
        # every resolution (between chunks or at a tile's end) either fits the set-up table or replays
        resolutions = rep["tie_queue_tables"] + rep["tie_queue_table_misses"]
        assert resolutions >= rep["tie_queue_drains"] and (resolutions > 0) == (rep["tie_queue_words"] > 0), (what, rep)
    else:
        assert rep["tie_queue_words"] == 0 and rep["tie_queue_drains"] == 0, (what, rep)
        assert rep["tie_queue_tables"] == 0 and rep["tie_queue_table_misses"] == 0, (what, rep)


def _scene_geometry(name):
    spec = synth.SCENES[name]
    rng = np.random.Generator(np.random.PCG64(spec["seed"]))
    pos = synth.track(spec["na"], rng, perturbed=spec["track"] == "perturbed")
    nx, ny, nr = spec["nx"], spec["ny"], spec["nr"]
    kw = dict(n_pulses=spec["na"], n_range=nr, r0=synth.RC_CENTRE - (nr // 2) * synth.DR, dr=synth.DR, nx=nx,
              ny=ny, x0=-(nx // 2) * synth.PIXEL, y0=-(ny // 2) * synth.PIXEL, z0=0.0, dx=synth.PIXEL,
              dy=synth.PIXEL, wavelength=synth.WAVELENGTH)
    return pos, kw


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
@pytest.mark.parametrize("scene, pulses", [("tiny", 256), ("std", 48), ("large", 12), ("hifi", 48), ("e2e", 24)])
def test_scene_geometries(sb, scene, pulses, interp):
    """Every workload's geometry, the whole grid, evenly spaced pulses (first and last included)."""
    pos, kw = _scene_geometry(scene)
    sel = np.unique(np.linspace(0, len(pos) - 1, pulses).astype(int))
    rep = sb.sarbp_check_indices(sb.make_params(interp=interp, **kw), pos[sel])
    _assert_clean(rep, scene)
    assert rep["fp64_ranges"] == 0 and rep["mode_chunks"][1:] == [0, 0]  # two-term series throughout
    assert rep["decisions"] >= kw["nx"] * kw["ny"] * len(sel)
    assert rep["max_position_error"] < 1e-5  # ~2^-24 of the window
    if interp == "nearest":
        assert 0 < rep["tie_band_max"] < 4e-5
        assert rep["tie_queue_capacity"] >= 2048 and rep["tie_queue_capacity"] % 64 == 0
    else:
        assert rep["tie_queue_capacity"] == 0


def test_random_geometries(sb):
    """The GPU random-geometry cases (every interpolator on each): grids of 1-160 x 1-120 pixels of
    0.05-6 m, Ka to L band, squinted tracks at 0.2-20 km, terrain, volumes, fp64-range plans."""
    seen_f64 = seen_fp32 = seen_dem = 0
    for seed in range(7000, 7000 + N_CASES):
        scene, _, _, layers = random_case(seed)
        for interp in ("nearest", "linear", "sinc8"):
            kw = dict(scene.params())
            kw["interp"] = interp
            dem = None
            if scene.dem is not None:
                kw["dem_relief"] = max(synth.block_relief(scene.dem), 1e-3)
                dem = scene.dem
            if layers is not None:
                kw["nz"], kw["dz"] = layers
            rep = sb.sarbp_check_indices(sb.make_params(**kw), scene.positions, dem=dem)
            _assert_clean(rep, (seed, interp))
            seen_f64 += rep["fp64_ranges"]
            seen_fp32 += 1 - rep["fp64_ranges"]
            seen_dem += dem is not None
    assert seen_f64 > 20 and seen_fp32 > 100 and seen_dem > 20


def _track(na, ground, height, step=0.3, squint=0.3, seed=1):
    rng = np.random.Generator(np.random.PCG64(seed))
    s = (np.arange(na) - (na - 1) / 2) * step
    pos = np.stack([s * math.cos(squint), -ground + s * math.sin(squint), np.full(na, height)], 1)
    return pos + rng.uniform(0, 0.3, 3) * np.sin(np.arange(na)[:, None] * 0.01 + rng.uniform(0, 6, 3))


def _long_params(sb, lam, dr, px, ground, height, n=96, nx=96, nr=16384, interp="nearest"):
    rc = math.hypot(ground, height)
    return sb.make_params(n_pulses=n, n_range=nr, r0=rc - (nr // 2) * dr, dr=dr, nx=nx, ny=nx, x0=-(nx // 2) * px,
                          y0=-(nx // 2) * px, z0=0.0, dx=px, dy=px, wavelength=lam, interp=interp)


def test_long_window_nearest_takes_fp64_ranges(sb):
    """L band, 5 cm bins, 1.5 m pixels: a 64 x 32 tile spans 2152 bins, whose fp32 window position
    errs by up to ~2e-4 bins -- beyond a fixed 4e-5 band.  Its tie band would pass the limit, so the
    plan runs the fp64-range kernels (fraction to 1e-7 bins, band 1e-6): no escapes."""
    prm = _long_params(sb, 0.236, 0.05, 1.5, 10000.0, 5000.0)
    rep = sb.sarbp_check_indices(prm, _track(96, 10000.0, 5000.0))
    _assert_clean(rep, "L band 1.5 m")
    assert rep["window"] == 2152 and rep["fp64_ranges"] == 1
    assert rep["tie_band_max"] == pytest.approx(1e-6)


@pytest.mark.parametrize("lam, dr, px, ground, height, mode", [
    (0.236, 0.1, 0.2, 10000.0, 5000.0, 1),   # L band, 10 cm bins: three-term series
    (0.0556, 0.1, 0.3, 150.0, 120.0, 2),     # C band at 190 m: the exact form
    (0.03125, 0.05, 0.1, 400.0, 300.0, 2),   # X band, 5 cm bins at 500 m
    (0.0556, 0.416, 0.8, 10000.0, 5000.0, 1),
])
def test_wide_tie_bands_on_fp32_ranges(sb, lam, dr, px, ground, height, mode):
    """fp32-range nearest plans whose tie band is wider than the old fixed 4e-5 bins: the band
    follows the window and the tile, the errors stay under its bound, and no decision escapes."""
    prm = _long_params(sb, lam, dr, px, ground, height)
    rep = sb.sarbp_check_indices(prm, _track(96, ground, height))
    _assert_clean(rep, (lam, dr, px))
    assert rep["fp64_ranges"] == 0
    assert rep["mode_chunks"][mode] > 0
    assert rep["tie_band_max"] > 4e-5
    assert rep["nearest_rechecks"] > 0


def test_terrain_and_volumes(sb):
    """The terrain kernels (dem) on 25 m of hills, tiles beyond the relief bound skipped, and a
    volume of 6 layers."""
    pos, kw = _scene_geometry("std")
    sel = np.linspace(0, len(pos) - 1, 24).astype(int)
    kw.update(nx=300, ny=200, x0=-150 * synth.PIXEL, y0=-100 * synth.PIXEL)
    dem = synth.terrain(300, 200, synth.PIXEL, synth.PIXEL, np.random.Generator(np.random.PCG64(4)), 25.0)
    relief = synth.block_relief(dem)
    for interp in ("nearest", "linear", "sinc8"):
        rep = sb.sarbp_check_indices(sb.make_params(interp=interp, dem_relief=relief, **kw), pos[sel], dem=dem)
        _assert_clean(rep, ("terrain", interp))
        assert rep["nan_tiles"] == 0
        # a bound below some tiles' relief: those tiles are skipped (the kernel writes NaN there)
        rep = sb.sarbp_check_indices(sb.make_params(interp=interp, dem_relief=0.5 * relief, **kw), pos[sel], dem=dem)
        _assert_clean(rep, ("terrain, tight bound", interp))
        assert rep["nan_tiles"] > 0
        rep = sb.sarbp_check_indices(sb.make_params(interp=interp, nz=6, dz=1.5, **kw), pos[sel])
        _assert_clean(rep, ("volume", interp))


def test_rejects_bad_arguments(sb):
    pos, kw = _scene_geometry("tiny")
    prm = sb.make_params(interp="nearest", **kw)
    with pytest.raises(ValueError):
        sb.sarbp_check_indices(prm, pos[:, :2])
    with pytest.raises(sb.SarbpError):  # more pulses than the plan takes
        sb.sarbp_check_indices(sb.make_params(interp="nearest", **{**kw, "n_pulses": 4}), pos[:5])
    with pytest.raises(sb.SarbpError):  # heights for a plan without terrain
        sb.sarbp_check_indices(prm, pos[:4], dem=np.zeros((kw["ny"], kw["nx"]), np.float32))
    with pytest.raises(sb.SarbpError):  # invalid parameters
        sb.sarbp_check_indices(sb.make_params(interp="nearest", **{**kw, "dr": -1.0}), pos[:4])


def test_report_struct_layout_matches_c(sb):
    fields = [f for f, _ in sb.sarbp_index_report._fields_]
    prog = ["#include <stdio.h>", "#include <stddef.h>", '#include "sarbp.h"', "int main(void){",
            'printf("%zu\\n", sizeof(sarbp_index_report));']
    prog += [f'printf("%zu\\n", offsetof(sarbp_index_report, {f}));' for f in fields]
    prog += ["return 0;}"]
    with tempfile.TemporaryDirectory() as d:
        src, exe = os.path.join(d, "p.c"), os.path.join(d, "p")
        open(src, "w").write("\n".join(prog))
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), src, "-o", exe], check=True)
        vals = [int(x) for x in subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(sb.sarbp_index_report)
    for f, off in zip(fields, vals[1:]):
        assert getattr(sb.sarbp_index_report, f).offset == off, f
