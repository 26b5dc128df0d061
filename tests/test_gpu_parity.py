"""GPU parity: the HIP library (through its C ABI) against the CPU oracle on seeded inputs."""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from _parity import PEAK_DB, PEAK_TIE, REL_L2, check_peaks, rel_l2, sample_pixels, target_windows
from _probe import nearest_index_mismatches

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sb(gpu_device):
    from domain_backprojection_amd import sarbp

    return sarbp


def _say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _run_bp(sb, scene, echo=None, positions=None, interp=None, **over):
    import torch

    e = scene.echo if echo is None else echo
    p = scene.positions if positions is None else positions
    kw = dict(over)
    if interp is not None:
        kw["interp"] = interp
    with sb.Plan.for_scene(scene, **kw) as plan:
        pos = torch.from_numpy(np.ascontiguousarray(p)).cuda()
        ech = torch.from_numpy(np.ascontiguousarray(e, dtype=np.complex64)).cuda()
        img = plan.backproject(pos, ech)
        torch.cuda.synchronize()
        return img.cpu().numpy().astype(np.complex128)


# ----------------------------------------------------------------------------- small, full image

@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_tiny_config_full_image(sb, interp):
    s = synth.make_scene("tiny", interp=interp)
    _say(f"[tiny {interp}] {s.nx}x{s.ny} na={s.na}")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
    check_peaks(lambda w: got[w[:, 1], w[:, 0]], lambda w: want[w[:, 1], w[:, 0]], target_windows(s), s.interp,
                f"{s.name} {s.interp}")


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
@pytest.mark.parametrize("shape", [(150, 70, 100), (64, 32, 64), (1, 1, 1), (65, 33, 129)])
def test_ragged_tiles_and_chunks(sb, interp, shape):
    """Grids that are not multiples of the 64x32 tile, pulse counts that are not
    multiples of the LDS chunk, perturbed track, clutter."""
    nx, ny, na = shape
    s = synth.make_scene("hifi", na=na, nr=1024, nx=nx, ny=ny, interp=interp, n_targets=1)
    _say(f"[ragged {interp}] {nx}x{ny} na={na}")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


def test_accumulate_over_pulse_chunks(sb):
    """image = BP(first half) then += BP(second half) equals one call over all pulses."""
    import torch

    s = synth.make_scene("std", na=300, nr=1024, nx=96, ny=80)
    with sb.Plan.for_scene(s) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        full = plan.backproject(pos, ech)
        part = plan.backproject(pos[:170], ech[:170])
        plan.backproject(pos[170:].contiguous(), ech[170:].contiguous(), image=part, accumulate=1)
        torch.cuda.synchronize()
        a, b = full.cpu().numpy(), part.cpu().numpy()
    assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-5


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_linearity_and_pulse_order(sb, interp):
    s = synth.make_scene("hifi", na=200, nr=1024, nx=80, ny=64, interp=interp)
    rng = np.random.Generator(np.random.PCG64(12))
    s2 = (rng.standard_normal(s.echo.shape) + 1j * rng.standard_normal(s.echo.shape)).astype(np.complex64)
    a, b = np.complex64(0.75 - 0.5j), np.complex64(-1.25 + 0.25j)
    lhs = _run_bp(sb, s, echo=(a * s.echo + b * s2).astype(np.complex64))
    rhs = a * _run_bp(sb, s) + b * _run_bp(sb, s, echo=s2)
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-5
    perm = rng.permutation(s.na)
    c = _run_bp(sb, s, echo=s.echo[perm], positions=s.positions[perm])
    d = _run_bp(sb, s)
    assert np.linalg.norm(c - d) / np.linalg.norm(d) < 1e-5


def test_one_plan_on_two_streams_concurrently(sb):
    """Calls with one plan may overlap on different streams (they share only the
    plan's progress hints, which steer scheduling): each result matches the same
    call made alone."""
    import torch

    s = synth.make_scene("std", na=512, nr=1024, nx=300, ny=200, n_targets=2)
    rng = np.random.Generator(np.random.PCG64(3))
    e2 = (rng.standard_normal(s.echo.shape) + 1j * rng.standard_normal(s.echo.shape)).astype(np.complex64)
    with sb.Plan.for_scene(s) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        ea, eb = torch.from_numpy(s.echo).cuda(), torch.from_numpy(e2).cuda()
        ref_a, ref_b = plan.backproject(pos, ea), plan.backproject(pos, eb)
        torch.cuda.synchronize()
        sa, sb_ = torch.cuda.Stream(), torch.cuda.Stream()
        ia, ib = plan.new_image(), plan.new_image()
        torch.cuda.synchronize()
        for _ in range(3):
            with torch.cuda.stream(sa):
                plan.backproject(pos, ea, image=ia)
            with torch.cuda.stream(sb_):
                plan.backproject(pos, eb, image=ib)
        torch.cuda.synchronize()
        assert torch.equal(ia, ref_a) and torch.equal(ib, ref_b)


def test_graph_capture_replays_match_eager(sb):
    """Range compression and backprojection captured once in a HIP graph (the entry
    points only enqueue kernels: they allocate and clear nothing) and replayed three
    times, with eager work and synchronisation between the replays: every replay
    reproduces the eager results bit for bit, also when accumulating into an image and
    for the pulse-group call (this 200 x 96 grid is split in 8 groups)."""
    import torch

    s = synth.make_scene("e2e", na=256, nx=200, ny=96, n_targets=2)
    with sb.Plan.for_scene(s, n_fast=s.nr) as plan:
        raw = torch.from_numpy(s.raw).cuda()
        pos = torch.from_numpy(s.positions).cuda()
        rc_ref = plan.range_compress(raw)
        ref = plan.backproject(pos, rc_ref)
        ws = torch.empty(plan.split_workspace_bytes(s.na), dtype=torch.uint8, device="cuda")
        assert ws.numel() > 0
        ref_split = plan.backproject(pos, rc_ref, split=True, workspace=ws)
        torch.cuda.synchronize()
        rc, img, acc, spl = torch.empty_like(raw), plan.new_image(), plan.new_image(), plan.new_image()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):  # one eager pass on the capture's side stream first
            plan.range_compress(raw, out=rc)
            plan.backproject(pos, rc, image=img)
            plan.backproject(pos, rc, image=spl, split=True, workspace=ws)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            plan.range_compress(raw, out=rc)
            plan.backproject(pos, rc, image=img)
            plan.backproject(pos, rc, image=acc, accumulate=1)
            plan.backproject(pos, rc, image=spl, split=True, workspace=ws)
        for k in range(3):
            rc.fill_(7.0)
            img.fill_(-3.0)
            acc.zero_()
            spl.fill_(5.0)
            junk = torch.randn(1 << 20, device="cuda").sum()  # unrelated eager work between replays
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            _say(f"[graph] replay {k}: rc {torch.equal(rc, rc_ref)}, image {torch.equal(img, ref)}, "
                 f"accumulated {torch.equal(acc, ref)}, split {torch.equal(spl, ref_split)} ({float(junk):.1f})")
            assert torch.equal(rc, rc_ref) and torch.equal(img, ref) and torch.equal(acc, ref)
            assert torch.equal(spl, ref_split)


@pytest.mark.parametrize("first, nr", [(246, 48), (226, 36)], ids=["record-starts-in-scene", "record-ends-in-scene"])
@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_zero_extension_and_far_pixels(sb, interp, first, nr):
    """A short record that only part of the grid's ranges fall into: samples beyond
    the record contribute zero, as in the oracle.  Pixels within the interpolator's
    reach of either end of the record (sinc8: 4 bins) take the in-record taps only.
    The scene spans bins 236..276 of the 512-bin record; the cut keeps bins
    first .. first + nr - 1."""
    s = synth.make_scene("tiny", na=40, nx=96, ny=96, interp=interp)
    r0 = s.r0 + first * s.dr
    sh = synth.Scene(**{**s.__dict__, "nr": nr, "r0": r0,
                        "echo": np.ascontiguousarray(s.echo[:, first:first + nr])})
    got = _run_bp(sb, sh)
    want = oracle.scene_backproject(sh)
    assert np.count_nonzero(np.abs(want) == 0) > 0
    assert rel_l2(got, want) <= REL_L2
    assert np.max(np.abs(got[np.abs(want) == 0])) == 0.0


def test_nonfinite_positions_propagate_nan(sb):
    s = synth.make_scene("tiny", na=16, nx=64, ny=32)
    pos = s.positions.copy()
    pos[5, 0] = np.nan
    got = _run_bp(sb, s, positions=pos)
    assert np.isnan(got).all()


# ----------------------------------------------------------------------------- accumulation modes

@pytest.mark.parametrize("accum", ["kahan", "chunk64"])
@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_accumulation_modes_full_image(sb, interp, accum):
    """The compensated accumulators give the same image as the oracle (tiny scene,
    plus a ragged grid on the perturbed track with a pulse count that is not a
    multiple of the chunk, and accumulate = 1 over two calls)."""
    import torch

    s = synth.make_scene("tiny", interp=interp)
    got = _run_bp(sb, s, accum=accum)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
    check_peaks(lambda w: got[w[:, 1], w[:, 0]], lambda w: want[w[:, 1], w[:, 0]], target_windows(s), s.interp,
                f"{s.name} {s.interp}")
    r = synth.make_scene("hifi", na=203, nr=1024, nx=70, ny=45, interp=interp, n_targets=1)
    with sb.Plan.for_scene(r, accum=accum) as plan:
        pos = torch.from_numpy(r.positions).cuda()
        ech = torch.from_numpy(r.echo).cuda()
        img = plan.backproject(pos[:120].contiguous(), ech[:120].contiguous())
        plan.backproject(pos[120:].contiguous(), ech[120:].contiguous(), image=img, accumulate=1)
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
    assert rel_l2(got, oracle.scene_backproject(r)) <= REL_L2


def test_compensated_accumulation_reduces_summation_error(sb):
    """16384 pulses from one antenna position with an echo that is constant along range:
    every pulse's term is s_n times the same rotation, so |I| = |sum_n s_n| up to the
    accumulation error (plus ~1e-7 from the rotation's fp32 magnitude).  A slowly rising
    s_n = 1 + n/N + 0.3j biases plain fp32 rounding (a CPU emulation of the three
    accumulators gives 8e-5, 3e-8 and 5e-7): the compensated modes must stay below
    1e-6 and the plain one must lose over ten times more."""
    import torch

    na, nr, nx, ny = 16384, 64, 64, 32
    g = np.array([[0.0, -synth.GROUND_RANGE, synth.ALTITUDE]])
    pos = np.repeat(g, na, axis=0)
    s_n = 1.0 + np.arange(na) / na + 0.3j
    echo = np.repeat(s_n.astype(np.complex64)[:, None], nr, axis=1)
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    kw = dict(n_pulses=na, n_range=nr, r0=r0, dr=synth.DR, nx=nx, ny=ny, x0=-(nx // 2) * synth.PIXEL,
              y0=-(ny // 2) * synth.PIXEL, z0=0.0, dx=synth.PIXEL, dy=synth.PIXEL, wavelength=synth.WAVELENGTH,
              interp="linear")
    exact = abs(np.sum(echo.astype(np.complex128)[:, 0]))
    errs = {}
    for accum in ("fp32", "kahan", "chunk64"):
        with sb.Plan(accum=accum, **kw) as plan:
            img = plan.backproject(torch.from_numpy(pos).cuda(), torch.from_numpy(echo).cuda())
            torch.cuda.synchronize()
            mag = np.abs(img.cpu().numpy().astype(np.complex128))
        errs[accum] = float(np.sqrt(np.mean((mag - exact) ** 2)) / exact)
    _say(f"[accumulation] relative RMS error of |I|: {errs}")
    assert errs["kahan"] < 1e-6 and errs["chunk64"] < 1e-6, errs
    assert errs["fp32"] > 10 * max(errs["kahan"], errs["chunk64"]), errs


# ----------------------------------------------------------------------------- streaming from host memory

def _pinned(a):
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a))
    return t.pin_memory()


@pytest.mark.parametrize("interp", ["linear", "sinc8"])
def test_host_stream_matches_device_path(sb, interp):
    """500 pulses from page-locked host memory in chunks of 128 (the last one ragged),
    through a plan whose per-call limit is the chunk: the same image as one
    device-resident call over all pulses, and the oracle's."""
    import torch

    s = synth.make_scene("hifi", na=500, nr=1024, nx=96, ny=80, interp=interp, n_targets=2)
    want = oracle.scene_backproject(s)
    ref = _run_bp(sb, s)
    pos_h, echo_h = _pinned(s.positions), _pinned(s.echo)
    with sb.Plan.for_scene(s, n_pulses=128) as plan, sb.HostStream(plan, chunk=128) as hs:
        img = hs.backproject(pos_h, echo_h)
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
        # the object is reused: a second call, accumulating the first 200 pulses again
        hs.backproject(pos_h[:200], echo_h[:200], image=img, accumulate=1)
        torch.cuda.synchronize()
        got2 = img.cpu().numpy().astype(np.complex128)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-5
    assert rel_l2(got, want) <= REL_L2
    s200 = synth.Scene(**{**s.__dict__, "na": 200, "positions": s.positions[:200], "echo": s.echo[:200]})
    assert rel_l2(got2, want + oracle.scene_backproject(s200)) <= REL_L2


def test_host_stream_many_calls_back_to_back(sb):
    """Twelve calls queued back to back on one stream object (8 chunks of 64 pulses
    each, so its two staging buffers and their release events are reused 96 times
    while the host waits for them): the accumulated image equals twelve times one
    call, and one call equals the device-resident path."""
    import torch

    s = synth.make_scene("std", na=512, nr=1024, nx=128, ny=96, n_targets=2)
    ref = _run_bp(sb, s)
    pos_h, echo_h = _pinned(s.positions), _pinned(s.echo)
    with sb.Plan.for_scene(s, n_pulses=64) as plan, sb.HostStream(plan, chunk=64) as hs:
        one = hs.backproject(pos_h, echo_h)
        img = plan.new_image()
        for k in range(12):
            hs.backproject(pos_h, echo_h, image=img, accumulate=1 if k else 0)
        torch.cuda.synchronize()
        one = one.cpu().numpy().astype(np.complex128)
        got = img.cpu().numpy().astype(np.complex128)
    assert np.linalg.norm(one - ref) / np.linalg.norm(ref) < 1e-5
    assert np.linalg.norm(got - 12 * one) / np.linalg.norm(12 * one) < 1e-6


def test_host_stream_with_range_compression(sb):
    """Raw pulses from host memory, range-compressed on the device chunk by chunk and
    backprojected: the same image as compressing and backprojecting on the device,
    and as the oracle's compression followed by its backprojection."""
    import torch

    s = synth.make_scene("e2e", na=300, nx=64, ny=96)
    with sb.Plan.for_scene(s, n_fast=s.nr, n_pulses=96) as plan:
        raw_d = torch.from_numpy(s.raw).cuda()
        pos_d = torch.from_numpy(s.positions).cuda()
        ref = plan.new_image()
        for n0 in range(0, s.na, 96):
            rc = plan.range_compress(raw_d[n0:n0 + 96].contiguous())
            plan.backproject(pos_d[n0:n0 + 96].contiguous(), rc, image=ref, accumulate=1 if n0 else 0)
        with sb.HostStream(plan, chunk=96, compress=True) as hs:
            img = hs.backproject(_pinned(s.positions), _pinned(s.raw))
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
        ref = ref.cpu().numpy().astype(np.complex128)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-6
    rc_orc = oracle.rc.range_compress(s.raw, s.fs, s.chirp_T, s.chirp_B, s.window)
    want = oracle.scene_backproject(s, echo=rc_orc)
    assert rel_l2(got, want) <= REL_L2


def test_image_tiling_by_sub_image_plans(sb):
    """A scene split into four row bands, one plan each (the page's tiling of images
    too large for memory): the bands reassemble the whole-image result.  Pixels are
    independent, so no overlap between bands is needed."""
    s = synth.make_scene("std", na=256, nr=1024, nx=128, ny=200, n_targets=3)
    whole = _run_bp(sb, s)
    bands = []
    for j0, j1 in ((0, 37), (37, 100), (100, 163), (163, 200)):
        sub = synth.Scene(**{**s.__dict__, "ny": j1 - j0, "y0": s.y0 + j0 * s.dy})
        bands.append(_run_bp(sb, sub))
    tiled = np.concatenate(bands, axis=0)
    want = oracle.scene_backproject(s)
    e_whole, e_tiled = rel_l2(whole, want), rel_l2(tiled, want)
    assert e_whole <= REL_L2 and e_tiled <= REL_L2
    # Bands have other tile centres, hence other fp32 range differences: each image is
    # ~1e-4 from the oracle, so the two differ by at most about twice that.
    assert np.linalg.norm(tiled - whole) / np.linalg.norm(whole) < 3e-4, (e_whole, e_tiled)


# ----------------------------------------------------------------------------- track interpolation

def test_track_interpolation_matches_oracle(sb):
    """Non-uniform navigation samples; pulse times inside, at the ends, at sample
    times, outside the span and not finite."""
    import torch

    rng = np.random.Generator(np.random.PCG64(21))
    M = 300
    nav_t = np.sort(rng.uniform(-4.0, 4.0, M))
    nav_p = np.stack([100.0 * nav_t + rng.normal(0, 0.2, M), -1e4 + rng.normal(0, 0.3, M),
                      5e3 + rng.normal(0, 0.3, M)], 1)
    t = np.concatenate([rng.uniform(-4.0, 4.0, 5000), nav_t[[0, 1, 150, M - 1]], [-4.5, 4.5, np.nan, np.inf]])
    got = sb.sarbp_interpolate_track(torch.from_numpy(nav_t).cuda(), torch.from_numpy(nav_p).cuda(),
                                     torch.from_numpy(t).cuda())
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    want = oracle.track.interpolate_track(nav_t, nav_p, t)
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.max(np.abs(got[ok] - want[ok])) < 1e-8


def test_backprojection_from_interpolated_track(sb):
    """Hi-fi geometry: navigation samples at 100 Hz of the perturbed track, positions
    interpolated on the device, then backprojected; parity with the oracle using its
    own interpolated positions, and the same image as from the exact positions."""
    import torch

    s = synth.make_scene("hifi", na=400, nr=1024, nx=96, ny=64, n_targets=2)
    model = synth.track_model(np.random.Generator(np.random.PCG64(1004)), perturbed=True)
    tp = synth.pulse_times(s.na)
    nav_t = np.arange(tp[0] - 0.05, tp[-1] + 0.05, 0.01)
    nav_p = synth.track_at(nav_t, model)
    exact = synth.track_at(tp, model)
    assert np.array_equal(exact, s.positions)  # the scene's echo was rendered from this track
    pos_o = oracle.track.interpolate_track(nav_t, nav_p, tp)
    assert np.max(np.abs(pos_o - exact)) < 1e-8
    pos_d = sb.sarbp_interpolate_track(torch.from_numpy(nav_t).cuda(), torch.from_numpy(nav_p).cuda(),
                                       torch.from_numpy(tp).cuda())
    with sb.Plan.for_scene(s) as plan:
        img = plan.backproject(pos_d, torch.from_numpy(s.echo).cuda())
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
    want = oracle.scene_backproject(synth.Scene(**{**s.__dict__, "positions": pos_o}))
    assert rel_l2(got, want) <= REL_L2
    ref = _run_bp(sb, s, positions=exact)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 1e-5


# ----------------------------------------------------------------------------- terrain (DEM)

def _run_bp_dem(sb, scene, dem, relief, **over):
    import torch

    with sb.Plan.for_scene(scene, dem_relief=relief, **over) as plan:
        img = plan.backproject(torch.from_numpy(scene.positions).cuda(), torch.from_numpy(scene.echo).cuda(),
                               dem=torch.from_numpy(np.ascontiguousarray(dem)).cuda())
        torch.cuda.synchronize()
        return img.cpu().numpy().astype(np.complex128)


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_terrain_full_image(sb, interp):
    """Targets and clutter on 25 m of seeded terrain (steep on this small grid: a
    64 x 32 block spans up to 20+ m), straight track; the plan's bound is the
    terrain's largest block range."""
    s = synth.make_scene("std", na=256, nr=1024, nx=150, ny=70, interp=interp, n_targets=3, dem_relief=25.0)
    relief = synth.block_relief(s.dem)
    _say(f"[terrain {interp}] block relief {relief:.1f} m")
    got = _run_bp_dem(sb, s, s.dem, relief)
    want = oracle.scene_backproject(s)
    assert np.isfinite(got).all()
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
    check_peaks(lambda w: got[w[:, 1], w[:, 0]], lambda w: want[w[:, 1], w[:, 0]], target_windows(s), s.interp,
                f"{s.name} {s.interp}")


@pytest.mark.parametrize("interp", ["linear", "nearest"])
def test_terrain_far_above_reference_plane(sb, interp):
    """Terrain 300 m above z0 (+-8 m) on a 150 x 70 grid, whose edge tiles are ragged in
    both directions, with a random echo over the whole record (the pixels sit ~130 m
    nearer than the reference plane): each tile is centred at its own mid-height and on
    its pixels inside the grid, and lanes past the grid's edge repeat an edge pixel, so
    none of them reaches outside its staged window.  The full image against the oracle."""
    import dataclasses

    s = synth.make_scene("std", na=128, nr=2048, nx=150, ny=70, interp=interp, n_targets=1, clutter=False,
                         dem_relief=16.0)
    rng = np.random.Generator(np.random.PCG64(59))
    echo = (rng.standard_normal(s.echo.shape) + 1j * rng.standard_normal(s.echo.shape)).astype(np.complex64)
    s = dataclasses.replace(s, dem=(s.dem + np.float32(300.0)).astype(np.float32), echo=echo)
    relief = synth.block_relief(s.dem)
    _say(f"[terrain +300 m {interp}] block relief {relief:.1f} m")
    got = _run_bp_dem(sb, s, s.dem, relief)
    want = oracle.scene_backproject(s)
    assert np.isfinite(got).all()
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_terrain_coarse_grid_fp64_ranges(sb, interp):
    """2 m pixels on up to 20 m of seeded terrain: a 64 x 32 tile's window (with the
    relief) spans about 9400 carrier cycles, past the 4096 up to which plans keep fp32
    window positions, so the terrain kernels take their range differences in fp64.
    Random echo; the full image against the oracle, within the fine grids' bar."""
    import dataclasses

    s = _custom_scene(synth.track(40), 4096, 70, 40, 2.0, 2.0, interp, 61)
    dem = synth.terrain(s.nx, s.ny, s.dx, s.dy, np.random.Generator(np.random.PCG64(62)), 20.0)
    s = dataclasses.replace(s, dem=dem)
    relief = synth.block_relief(dem)
    _say(f"[terrain 2 m {interp}] block relief {relief:.1f} m")
    got = _run_bp_dem(sb, s, dem, relief)
    want = oracle.scene_backproject(s)
    assert np.isfinite(got).all()
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


def test_terrain_perturbed_track_and_chunk64(sb):
    s = synth.make_scene("hifi", na=203, nr=1024, nx=96, ny=64, interp="sinc8", n_targets=2, dem_relief=12.0)
    got = _run_bp_dem(sb, s, s.dem, synth.block_relief(s.dem), accum="chunk64")
    assert rel_l2(got, oracle.scene_backproject(s)) <= REL_L2


def test_flat_terrain_equals_the_plane(sb):
    s = synth.make_scene("std", na=128, nr=1024, nx=96, ny=64, n_targets=2)
    got = _run_bp_dem(sb, s, np.zeros((s.ny, s.nx), np.float32), 5.0)
    ref = _run_bp(sb, s)
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < 3e-4


def test_terrain_beyond_the_bound_is_nan(sb):
    """Blocks whose height range exceeds the plan's bound come out NaN; the rest match
    the oracle."""
    s = synth.make_scene("std", na=96, nr=1024, nx=150, ny=70, n_targets=2, dem_relief=25.0)
    bound = 0.5 * synth.block_relief(s.dem)
    got = _run_bp_dem(sb, s, s.dem, bound)
    want = oracle.scene_backproject(s)
    expect_nan = np.zeros((s.ny, s.nx), bool)
    for j in range(0, s.ny, 32):
        for i in range(0, s.nx, 64):
            b = s.dem[j:j + 32, i:i + 64].astype(np.float64)
            expect_nan[j:j + 32, i:i + 64] = b.max() - b.min() > bound
    assert expect_nan.any() and not expect_nan.all()
    assert np.array_equal(np.isnan(got.real), expect_nan)
    ok = ~expect_nan
    assert np.linalg.norm(got[ok] - want[ok]) / np.linalg.norm(want[ok]) <= REL_L2


def test_terrain_nearest_index_bit_exact(sb):
    """One pulse at a time with echo s[k] = k + 1: |I| - 1 is the chosen bin, against
    floor(u + 1/2) computed in fp64 in the definition's operation order."""
    import torch

    s = synth.make_scene("std", na=64, nr=1024, nx=150, ny=70, interp="nearest", n_targets=1, dem_relief=25.0)
    relief = synth.block_relief(s.dem)
    ramp = torch.arange(1, s.nr + 1, dtype=torch.float32).to(torch.complex64).cuda()[None, :].contiguous()
    jj, ii = np.meshgrid(np.arange(s.ny), np.arange(s.nx), indexing="ij")
    x = s.x0 + ii * s.dx
    y = s.y0 + jj * s.dy
    z = s.z0 + s.dem.astype(np.float64)
    dem_d = torch.from_numpy(s.dem).cuda()
    bad = 0
    with sb.Plan.for_scene(s, interp="nearest", n_pulses=1, dem_relief=relief) as plan:
        img = plan.new_image()
        for n in range(0, s.na, 3):
            a = s.positions[n]
            plan.backproject(torch.from_numpy(s.positions[n:n + 1].copy()).cuda(), ramp, image=img, dem=dem_d)
            mag = img.abs().cpu().numpy().astype(np.float64)
            ddx, ddy, ddz = x - a[0], y - a[1], z - a[2]
            R = np.sqrt(ddx * ddx + ddy * ddy + ddz * ddz)
            k = np.floor((R - s.r0) / s.dr + 0.5)
            bad += int(np.count_nonzero(np.rint(mag) - 1 != k))
    assert bad == 0


# ----------------------------------------------------------------------------- 3-D (voxel) images

def _volume_scene(interp, nx=70, ny=45, nz=5, passes=6, na_per=40, seed=31):
    """Parallel passes 40 m apart in height, unit targets on voxel centres at several
    heights plus weak noise; the volume's layers run from z0 = -1 m by dz = 0.5 m."""
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = synth.multipass_track(passes, na_per, 40.0)
    nr = 1024
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    dx = dy = synth.PIXEL
    x0, y0, z0, dz = -(nx // 2) * dx, -(ny // 2) * dy, -1.0, 0.5
    vox = np.array([[20, 12, 1], [45, 30, 3], [60, 8, 4], [8, 38, 0]])
    pts = np.stack([x0 + vox[:, 0] * dx, y0 + vox[:, 1] * dy, z0 + vox[:, 2] * dz], 1)
    echo = synth.render_points(pos, nr, r0, synth.DR, pts, np.ones(len(vox)), half=256)
    echo = echo + synth.complex_normal(rng, echo.shape, 1e-3)
    s = synth.Scene(name="volume", seed=seed, na=len(pos), nr=nr, nx=nx, ny=ny, x0=x0, y0=y0, z0=z0,
                    dx=dx, dy=dy, r0=r0, dr=synth.DR, wavelength=synth.WAVELENGTH, interp=interp, positions=pos,
                    echo=echo.astype(np.complex64), raw=None, targets=vox[:, :2])
    return s, nz, dz, vox


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_volume_matches_oracle(sb, interp):
    import torch

    s, nz, dz, vox = _volume_scene(interp)
    with sb.Plan.for_scene(s, nz=nz, dz=dz) as plan:
        img = plan.backproject(torch.from_numpy(s.positions).cuda(), torch.from_numpy(s.echo).cuda())
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
    want = oracle.backproject_volume(s.positions, s.echo, s.r0, s.dr, s.nx, s.ny, nz, s.x0, s.y0, s.z0, s.dx, s.dy,
                                     dz, s.wavelength, interp)
    assert got.shape == (nz, s.ny, s.nx)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
    for i, j, l in vox:
        win = np.array([(a, b, c) for c in range(max(0, l - 2), min(nz, l + 3)) for b in range(j - 2, j + 3)
                        for a in range(i - 2, i + 3)])
        g, o = got[win[:, 2], win[:, 1], win[:, 0]], want[win[:, 2], win[:, 1], win[:, 0]]
        check_peaks(lambda w: g, lambda w: o, [win], interp, f"volume {interp} voxel {(i, j, l)}")
        ko = int(np.argmax(np.abs(o)))
        if interp != "nearest":  # nearest's plateaus may put the definition's own peak a voxel off
            assert tuple(win[ko]) == (i, j, l)


def test_volume_through_the_host_pipeline(sb):
    import torch

    s, nz, dz, _ = _volume_scene("linear", nx=64, ny=32, nz=3)
    with sb.Plan.for_scene(s, nz=nz, dz=dz, n_pulses=64) as plan, sb.HostStream(plan, chunk=64) as hs:
        img = hs.backproject(_pinned(s.positions), _pinned(s.echo))
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
    want = oracle.backproject_volume(s.positions, s.echo, s.r0, s.dr, s.nx, s.ny, nz, s.x0, s.y0, s.z0, s.dx, s.dy,
                                     dz, s.wavelength, "linear")
    assert rel_l2(got, want) <= REL_L2


# ----------------------------------------------------------------------------- nearest: bit-exact index

@pytest.mark.parametrize("scene", ["tiny", "std", "large", "hifi"])
def test_nearest_index_bit_exact(sb, scene):
    """>= 64 evenly spaced pulses plus the first and last of each geometry, every pixel."""
    spec = synth.SCENES[scene]
    # geometry only: the echo is replaced by the index probe
    s = synth.make_scene(scene, nr=spec["nr"], na=spec["na"], clutter=False, n_targets=1) if scene == "tiny" else None
    if s is None:
        rng = np.random.Generator(np.random.PCG64(spec["seed"]))
        na = spec["na"]
        pos = synth.track(na, rng, perturbed=spec["track"] == "perturbed")
        nx, ny, nr = spec["nx"], spec["ny"], spec["nr"]
        s = synth.Scene(name=scene, seed=spec["seed"], na=na, nr=nr, nx=nx, ny=ny,
                        x0=-(nx // 2) * synth.PIXEL, y0=-(ny // 2) * synth.PIXEL, z0=0.0, dx=synth.PIXEL,
                        dy=synth.PIXEL, r0=synth.RC_CENTRE - (nr // 2) * synth.DR, dr=synth.DR,
                        wavelength=synth.WAVELENGTH, interp="nearest", positions=pos, echo=None, raw=None,
                        targets=np.zeros((0, 2), np.int64))
    pulses = sorted(set(np.linspace(0, s.na - 1, 64).astype(int).tolist()) | {0, s.na - 1})
    _say(f"[index probe {scene}] {len(pulses)} pulses x {s.nx * s.ny} pixels")
    assert nearest_index_mismatches(sb, s, pulses) == 0


def _probe_track(na, ground, height, step=0.3, squint=0.3, seed=1):
    """A squinted straight track at the given ground range and height with a small wobble."""
    rng = np.random.Generator(np.random.PCG64(seed))
    s = (np.arange(na) - (na - 1) / 2) * step
    pos = np.stack([s * math.cos(squint), -ground + s * math.sin(squint), np.full(na, height)], 1)
    return pos + rng.uniform(0, 0.3, 3) * np.sin(np.arange(na)[:, None] * 0.01 + rng.uniform(0, 6, 3))


@pytest.mark.parametrize("lam, dr, px, ground, height", [
    (0.236, 0.05, 1.5, 10000.0, 5000.0),   # 2152-bin windows: the fp64-range kernels
    (0.236, 0.1, 0.2, 10000.0, 5000.0),    # fp32, three-term series, band ~1.1e-4
    (0.0556, 0.1, 0.3, 150.0, 120.0),      # fp32, exact form at 190 m, band ~4e-4
    (0.03125, 0.05, 0.1, 400.0, 300.0),    # fp32, exact form, 5 cm bins
], ids=["L-1.5m-f64", "L-10cm-series", "C-190m-exact", "X-5cm-exact"])
def test_nearest_index_bit_exact_long_windows(sb, lam, dr, px, ground, height):
    """Long echo windows and wide fp32 tie bands: all 96 pulses x every pixel of a 96 x 96 grid."""
    na, nx, nr = 96, 96, 16384
    rc = math.hypot(ground, height)
    s = synth.Scene(name="probe", seed=0, na=na, nr=nr, nx=nx, ny=nx, x0=-(nx // 2) * px, y0=-(nx // 2) * px,
                    z0=0.0, dx=px, dy=px, r0=rc - (nr // 2) * dr, dr=dr, wavelength=lam, interp="nearest",
                    positions=_probe_track(na, ground, height), echo=None, raw=None,
                    targets=np.zeros((0, 2), np.int64))
    _say(f"[index probe long window] lambda {lam} dr {dr} pixel {px} at {rc:.0f} m: {na} pulses x {nx * nx} px")
    assert nearest_index_mismatches(sb, s, range(na)) == 0


@pytest.mark.parametrize("n, na", [(128, 4096), (192, 2048)], ids=["128px-4096p", "192px-2048p"])
def test_nearest_tie_queue_whole_image(sb, n, na):
    """Nearest on the standard geometry with many pulses per tile, so that a workgroup queues
    hundreds of tie rechecks from many waves, resolved by every lane of the workgroup at the
    tile's end: every pixel against the oracle.  Besides the rel-L2 bar, each pixel must be
    within 2e-3 of the image's peak magnitude: the fp32 tie band keeps every term's phase
    error below 2 pi kappa band / 2 (8e-4 rad here), so even a coherent sum of such errors
    stays below 1.1e-3 of a target's peak."""
    s = synth.make_scene("std", nx=n, ny=n, na=na, interp="nearest")
    rep = sb.sarbp_check_indices(sb.make_params(**s.params()), s.positions)
    assert rep["tie_queue_tile_max"] > 64, rep
    _say(f"[nearest tie queue] {n}x{n} px x {na} pulses: {rep['tie_queue_words']} queued words, "
         f"{rep['tie_queue_tile_max']} in one tile, {rep['tie_queue_drains']} mid-tile drains")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
    err = np.abs(got - want)
    assert err.max() <= 2e-3 * np.abs(want).max(), (err.max(), np.unravel_index(err.argmax(), err.shape))


@pytest.mark.parametrize("lam, dr, px, ground, height, table, accum", [
    (0.0556, 0.1, 0.3, 150.0, 120.0, "all", "fp32"),       # C band at 190 m, band ~4e-4: 16 mid-tile drains
    (0.03125, 0.05, 0.1, 400.0, 300.0, "some", "fp32"),    # X band, 5 cm bins, band ~2.6e-4: 9
    (0.0556, 0.1, 0.3, 150.0, 120.0, "all", "kahan"),
    (0.0556, 0.1, 0.3, 150.0, 120.0, "all", "chunk64"),
], ids=["C-190m-exact", "X-5cm-exact", "C-190m-exact-kahan", "C-190m-exact-chunk64"])
def test_nearest_tie_queue_mid_tile_drains(sb, lam, dr, px, ground, height, table, accum):
    """Wide fp32 tie bands on 128 x 128 pixels and 2048 pulses of a seeded random echo: some
    workgroups queue more tie rechecks than a chunk leaves room for, so the queue is resolved
    between chunks as well as at the tile's end (the host check counts those drains).  On the X-band
    geometry some resolutions mark more pulses than the LDS set-up table holds and repeat each
    word's set-ups instead, so both ways of resolving the queue are exercised; the compensated
    and chunk-fp64 accumulators take the corrections between chunks as well.  The image
    must equal the sum of the 2048 single-pulse images -- each of which resolves its own queue
    at its tile's end, and whose every bin the index probes pin to the oracle's -- up to the
    order of the fp32 additions.  A correction dropped, applied twice or given to another
    lane moves a pixel by about one echo sample (~1 here, against a bound of 1e-4 of the
    image's largest magnitude, ~0.02)."""
    import torch

    na, n, nr = 2048, 128, 8192
    rc = math.hypot(ground, height)
    rng = np.random.Generator(np.random.PCG64(11))
    echo = synth.complex_normal(rng, (na, nr), 1.0).astype(np.complex64)
    s = synth.Scene(name="ties", seed=11, na=na, nr=nr, nx=n, ny=n, x0=-(n // 2) * px, y0=-(n // 2) * px, z0=0.0,
                    dx=px, dy=px, r0=rc - (nr // 2) * dr, dr=dr, wavelength=lam, interp="nearest",
                    positions=_probe_track(na, ground, height), echo=echo, raw=None,
                    targets=np.zeros((0, 2), np.int64))
    rep = sb.sarbp_check_indices(sb.make_params(**s.params()), s.positions)
    assert rep["tie_queue_drains"] > 0 and rep["nearest_escapes"] == 0 and rep["fp64_ranges"] == 0, rep
    assert rep["tie_queue_tables"] > 0 and (rep["tie_queue_table_misses"] > 0) == (table == "some"), rep
    _say(f"[nearest tie queue, mid-tile] lambda {lam} dr {dr} pixel {px}: {rep['tie_queue_words']} queued words, "
         f"{rep['tie_queue_tile_max']} in one tile, {rep['tie_queue_drains']} mid-tile drains, "
         f"{rep['tie_queue_tables']} resolutions by set-up table, {rep['tie_queue_table_misses']} by replay")
    with sb.Plan.for_scene(s, accum=accum) as plan:
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(echo).cuda()
        whole = plan.backproject(pos, ech)
        acc = plan.new_image()
        for p in range(na):
            plan.backproject(pos[p:p + 1], ech[p:p + 1], image=acc, accumulate=1)
        torch.cuda.synchronize()
        got = whole.cpu().numpy().astype(np.complex128)
        want = acc.cpu().numpy().astype(np.complex128)
    err = np.abs(got - want)
    assert err.max() <= 1e-4 * np.abs(want).max(), (err.max(), np.abs(want).max(),
                                                     np.unravel_index(err.argmax(), err.shape))
    assert rel_l2(got, want) <= 1e-5, rel_l2(got, want)


# ----------------------------------------------------------------------------- range compression

def test_range_compression_matches_oracle(sb):
    import torch

    s = synth.make_scene("e2e", na=64)
    with sb.Plan.for_scene(s, n_fast=s.nr) as plan:
        out = plan.range_compress(torch.from_numpy(s.raw).cuda())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.complex128)
    want = oracle.rc.range_compress(s.raw, s.fs, s.chirp_T, s.chirp_B, s.window)
    assert rel_l2(got, want) < 1e-5, rel_l2(got, want)


@pytest.mark.parametrize("n_fast", [64, 128, 512, 1024, 2048, 4096, 16384])
@pytest.mark.parametrize("window", [0, 1, 2])
def test_range_compression_sizes(sb, n_fast, window):
    import torch

    rng = np.random.Generator(np.random.PCG64(n_fast + window))
    x = (rng.standard_normal((5, n_fast)) + 1j * rng.standard_normal((5, n_fast))).astype(np.complex64)
    T = min(synth.CHIRP_T, 0.5 * n_fast / synth.FS)
    with sb.Plan(n_pulses=1, n_range=n_fast, r0=0.0, dr=1.0, nx=1, ny=1, x0=0, y0=0, z0=0, dx=1, dy=1,
                 wavelength=0.03, interp="linear", n_fast=n_fast, fs=synth.FS, chirp_T=T,
                 chirp_B=synth.BANDWIDTH, window=window) as plan:
        out = plan.range_compress(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.complex128)
    want = oracle.rc.range_compress(x, synth.FS, T, synth.BANDWIDTH, window)
    assert rel_l2(got, want) < 1e-5


def test_range_compression_several_records_per_workgroup(sb):
    """16384-point records fill a CU's LDS, so the launch runs one workgroup per CU and each
    takes several records in turn, loading the next while it transforms the current one:
    600 records (2 or 3 per workgroup on 256 CUs, a ragged last round) against the oracle."""
    import torch

    n_fast, na = 16384, 600
    rng = np.random.Generator(np.random.PCG64(16384))
    x = (rng.standard_normal((na, n_fast)) + 1j * rng.standard_normal((na, n_fast))).astype(np.complex64)
    with sb.Plan(n_pulses=na, n_range=n_fast, r0=0.0, dr=1.0, nx=1, ny=1, x0=0, y0=0, z0=0, dx=1, dy=1,
                 wavelength=0.03, interp="linear", n_fast=n_fast, fs=synth.FS, chirp_T=synth.CHIRP_T,
                 chirp_B=synth.BANDWIDTH, window=1) as plan:
        out = plan.range_compress(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.complex128)
    want = oracle.rc.range_compress(x, synth.FS, synth.CHIRP_T, synth.BANDWIDTH, 1)
    assert rel_l2(got, want) < 1e-5
    # every record on its own, so that a record skipped or written twice cannot hide in the total
    per = np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)
    assert per.max() < 1e-5, (per.max(), int(per.argmax()))


@pytest.mark.parametrize("nbar, sll", [(4, 35.0), (6, 45.0), (3, 25.0)])
def test_range_compression_taylor_parameters(sb, nbar, sll):
    """The Taylor taper's parameters reach the filter (end-to-end scene's chirp, 8192 samples)."""
    import torch

    rng = np.random.Generator(np.random.PCG64(nbar))
    x = (rng.standard_normal((3, 8192)) + 1j * rng.standard_normal((3, 8192))).astype(np.complex64)
    with sb.Plan(n_pulses=1, n_range=8192, r0=0.0, dr=1.0, nx=1, ny=1, x0=0, y0=0, z0=0, dx=1, dy=1,
                 wavelength=0.03, interp="linear", n_fast=8192, fs=synth.FS, chirp_T=synth.CHIRP_T,
                 chirp_B=synth.BANDWIDTH, window=2, taylor_nbar=nbar, taylor_sll=sll) as plan:
        out = plan.range_compress(torch.from_numpy(x).cuda())
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.complex128)
    want = oracle.rc.range_compress(x, synth.FS, synth.CHIRP_T, synth.BANDWIDTH, 2, nbar, sll)
    assert rel_l2(got, want) < 1e-5


# ----------------------------------------------------------------------------- full-size configs

_SCENES = {}


def _scene(name):
    """Full-size scenes, generated once per test session (the hi-fi and large scenes take tens
    of seconds of host time)."""
    import time

    if name not in _SCENES:
        t = time.time()
        _SCENES[name] = synth.make_scene(name)
        s = _SCENES[name]
        _say(f"[{name}] generated {s.na}x{s.nr} echo, {s.nx}x{s.ny} grid in {time.time() - t:.1f}s")
    return _SCENES[name]


def _check_image(s, got, want, label):
    """Whole-image parity: rel-L2 over every pixel, over the clutter alone (outside the target
    windows) and over the target windows; each target's peak pixel and magnitude."""
    wins = target_windows(s)
    mask = np.zeros(want.shape, bool)
    for w in wins:
        mask[w[:, 1], w[:, 0]] = True
    e_all, e_clut, e_tgt = rel_l2(got, want), rel_l2(got[~mask], want[~mask]), rel_l2(got[mask], want[mask])
    db = check_peaks(lambda w: got[w[:, 1], w[:, 0]], lambda w: want[w[:, 1], w[:, 0]], wins, s.interp, label)
    _say(f"[{label}] whole image {got.shape[1]}x{got.shape[0]}: rel-L2 {e_all:.2e} (clutter {e_clut:.2e}, "
         f"target windows {e_tgt:.2e}); {len(wins)} peaks on the oracle's pixels, worst {db:.4f} dB")
    assert e_all <= REL_L2 and e_clut <= REL_L2 and e_tgt <= REL_L2, (e_all, e_clut, e_tgt)


@pytest.mark.parametrize("scene, interp", [("std", None), ("std", "nearest"), ("hifi", None)],
                         ids=["std", "std-nearest", "hifi"])
def test_full_size_whole_image(sb, scene, interp):
    """The standard scene (linear, and nearest on the same echo) and the hi-fi scene (sinc8,
    perturbed track) against the oracle's whole image: 1024 x 1024 pixels x 4096 pulses.
    Nearest also bounds every pixel's error by 2e-3 of the image's peak magnitude (the
    coherent worst case of its fp32 phase bound): its tie rechecks run on a few rows of
    this geometry hundreds of times per tile, and a wrong recheck shows there."""
    import dataclasses
    import time

    import torch

    s = _scene(scene)
    if interp is not None:
        s = dataclasses.replace(s, interp=interp)
    with sb.Plan.for_scene(s) as plan:
        img = plan.backproject(torch.from_numpy(s.positions).cuda(), torch.from_numpy(s.echo).cuda())
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
    t = time.time()
    want = oracle.scene_backproject(s)
    _say(f"[{scene}] oracle image in {time.time() - t:.1f}s on {oracle.threads()} threads")
    _check_image(s, got, want, f"{scene} {s.interp}")
    if s.interp == "nearest":
        err = np.abs(got - want)
        assert err.max() <= 2e-3 * np.abs(want).max(), (err.max(), np.unravel_index(err.argmax(), err.shape))


def test_large_scene_sampled(sb):
    """The large scene (16384 pulses x 8192 bins -> 2048 x 2048): its oracle image would take
    minutes, so 4000 random pixels (clutter) and every target window are compared, each set
    against the bar on its own."""
    import torch

    s = _scene("large")
    with sb.Plan.for_scene(s) as plan:
        img = plan.backproject(torch.from_numpy(s.positions).cuda(), torch.from_numpy(s.echo).cuda())
        torch.cuda.synchronize()
        got = img.cpu().numpy()
    wins = target_windows(s)
    rnd = sample_pixels(s, 4000, 80)
    ij = np.concatenate([rnd] + wins)
    want = oracle.scene_pixels(s, ij)
    g = got[ij[:, 1], ij[:, 0]].astype(np.complex128)
    nr_ = len(rnd)
    e_rnd, e_tgt = rel_l2(g[:nr_], want[:nr_]), rel_l2(g[nr_:], want[nr_:])
    lut = {tuple(p): v for p, v in zip(ij.tolist(), want)}
    db = check_peaks(lambda w: got[w[:, 1], w[:, 0]], lambda w: np.array([lut[tuple(p)] for p in w.tolist()]), wins,
                     s.interp, "large linear")
    _say(f"[large] rel-L2 {e_rnd:.2e} on {nr_} random pixels, {e_tgt:.2e} on {len(ij) - nr_} target-window "
         f"pixels; worst peak {db:.4f} dB")
    assert e_rnd <= REL_L2 and e_tgt <= REL_L2, (e_rnd, e_tgt)


def test_end_to_end_whole_image(sb):
    """Raw LFM echoes -> GPU range compression -> GPU backprojection, against the fp64 oracle
    chain (numpy matched filter, then the C oracle over the whole 1024 x 1024 image)."""
    import torch

    s = _scene("e2e")
    with sb.Plan.for_scene(s, n_fast=s.nr) as plan:
        raw = torch.from_numpy(s.raw).cuda()
        rc = plan.range_compress(raw)
        img = plan.backproject(torch.from_numpy(s.positions).cuda(), rc)
        torch.cuda.synchronize()
        got = img.cpu().numpy().astype(np.complex128)
        rc_got = rc.cpu().numpy()
    rc_want = oracle.rc.range_compress(s.raw, s.fs, s.chirp_T, s.chirp_B, s.window)
    e_rc = rel_l2(rc_got.astype(np.complex128), rc_want)
    _say(f"[e2e] range compression rel-L2 {e_rc:.2e}")
    assert e_rc < 1e-5
    want = oracle.scene_backproject(s, echo=rc_want)
    _check_image(s, got, want, "e2e linear")


# ----------------------------------------------------------------------------- geometry edge cases

def _custom_scene(pos, nr, nx, ny, dx, dy, interp, seed, dr=synth.DR):
    """Random echo on an arbitrary geometry (range record centred on the scene centre)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    Rc = float(np.linalg.norm(pos[len(pos) // 2] - np.array([0.0, 0.0, 0.0])))
    r0 = Rc - (nr // 2) * dr
    echo = (rng.standard_normal((len(pos), nr)) + 1j * rng.standard_normal((len(pos), nr))).astype(np.complex64)
    return synth.Scene(name="custom", seed=seed, na=len(pos), nr=nr, nx=nx, ny=ny, x0=-(nx // 2) * dx,
                       y0=-(ny // 2) * dy, z0=0.0, dx=dx, dy=dy, r0=r0, dr=dr, wavelength=synth.WAVELENGTH,
                       interp=interp, positions=pos, echo=echo, raw=None, targets=np.zeros((0, 2), np.int64))


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_window_beyond_lds_is_unsupported(sb, interp):
    """200 m pixels: one tile's echo window (~32,000 bins, 250 KB or more) cannot be
    staged even one pulse at a time in 150 KiB of LDS, so plan creation reports
    SARBP_EUNSUPPORTED and nothing runs."""
    with pytest.raises(sb.SarbpError) as err:
        sb.Plan(n_pulses=16, n_range=65536, r0=5000.0, dr=synth.DR, nx=64, ny=64, x0=-6400.0, y0=-6400.0,
                z0=0.0, dx=200.0, dy=200.0, wavelength=synth.WAVELENGTH, interp=interp)
    assert err.value.status == sb.SARBP_EUNSUPPORTED


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_coarse_grid_uses_large_lds_windows(sb, interp):
    """3 m pixels sampled at 0.1 m range bins: each 64 x 32 tile spans ~2150 bins, so
    fewer than 8 pulses fit the default LDS budget for every interpolator (17 KB per
    pulse for nearest, 34 KB linear, 138 KB sinc8) and the plan stages pulses in up to
    150 KiB instead.  (The tiles' 107 m half diagonal also puts the plan on fp64 range
    differences.)"""
    pos = synth.track(40)
    s = _custom_scene(pos, 16384, 70, 40, 3.0, 3.0, interp, 31, dr=0.1)
    _say(f"[coarse {interp}] {s.nx}x{s.ny} at 3 m, dr 0.1 m")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


@pytest.mark.parametrize("interp, accum", [("linear", "fp32"), ("nearest", "fp32"), ("sinc8", "fp32"),
                                           ("linear", "kahan"), ("linear", "chunk64")])
@pytest.mark.parametrize("pixel", [0.8, 8.0])
def test_coarse_grid_range_precision(sb, interp, accum, pixel):
    """Fp32 window positions carry about 2^-24 of the window, i.e. of the carrier cycles
    across it, so the plan switches to fp64 range differences once a 64 x 32 tile's
    window spans more than 4096 cycles.  0.8 m pixels (3837 cycles at 3.125 cm and
    0.416 m bins) stay just under it, on the fp32 kernels; 8 m pixels (~37000 cycles,
    where fp32 differences gave a relative error of 4.2e-3) go over, with the
    seven-term series for every pulse at 11 km.  Both must meet the fine grids' bar."""
    pos = synth.track(40)
    s = _custom_scene(pos, 4096, 70, 40, pixel, pixel, interp, 47)
    _say(f"[range precision {interp} {accum}] {s.nx}x{s.ny} at {pixel} m")
    got = _run_bp(sb, s, accum=accum)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


# ----------------------------------------------------------------------------- pulses split over workgroups

def _rel(a, b):
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


@pytest.mark.parametrize("interp, accum", [("linear", "fp32"), ("nearest", "fp32"), ("sinc8", "fp32"),
                                           ("linear", "kahan"), ("linear", "chunk64")])
def test_split_small_grid(sb, interp, accum):
    """The tiny scene (128 x 128 pixels in 16 tiles of 64 x 16, 256 pulses) through
    sarbp_backproject_split: 8 pulse groups of 32, so 128 workgroups instead of 16.  The
    image equals the unsplit call's up to the summation order (1e-5) and the oracle's
    within the bar; then 250 pulses (ragged groups) with accumulate = 1 onto the first
    image equals the unsplit calls' sum."""
    import torch

    s = synth.make_scene("tiny", interp=interp)
    with sb.Plan.for_scene(s, accum=accum) as plan:
        need = plan.split_workspace_bytes(s.na)
        assert need == 8 * s.nx * s.ny * 8, need
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        a = plan.backproject(pos, ech)
        b = plan.backproject(pos, ech, split=True)
        a2 = plan.backproject(pos[:250].contiguous(), ech[:250].contiguous(), image=a.clone(), accumulate=1)
        b2 = plan.backproject(pos[:250].contiguous(), ech[:250].contiguous(), image=b.clone(), accumulate=1,
                              split=True)
        torch.cuda.synchronize()
        a, b, a2, b2 = (t.cpu().numpy().astype(np.complex128) for t in (a, b, a2, b2))
    want = oracle.scene_backproject(s)
    _say(f"[split {interp} {accum}] vs unsplit {_rel(b, a):.1e}, vs oracle {rel_l2(b, want):.1e}, "
         f"accumulated {_rel(b2, a2):.1e}")
    assert _rel(b, a) <= 1e-5
    assert rel_l2(b, want) <= REL_L2
    assert _rel(b2, a2) <= 1e-5


def test_split_terrain_and_volume(sb):
    """Small terrain (150 x 70 pixels, 6 tiles of 64 x 32) and volume (96 x 40 x 3 layers)
    grids, split against unsplit."""
    import torch

    s = synth.make_scene("std", na=300, nr=1024, nx=150, ny=70, interp="linear", n_targets=3, dem_relief=20.0)
    relief = synth.block_relief(s.dem)
    dem = torch.from_numpy(np.ascontiguousarray(s.dem)).cuda()
    with sb.Plan.for_scene(s, dem_relief=relief) as plan:
        assert plan.split_workspace_bytes(s.na) > 0
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        a = plan.backproject(pos, ech, dem=dem)
        b = plan.backproject(pos, ech, dem=dem, split=True)
        torch.cuda.synchronize()
        a, b = a.cpu().numpy(), b.cpu().numpy()
    assert np.isfinite(b).all() and _rel(b, a) <= 1e-5, _rel(b, a)

    v = synth.make_scene("std", na=256, nr=1024, nx=96, ny=40, interp="linear", n_targets=2)
    with sb.Plan.for_scene(v, nz=3, dz=1.5) as plan:
        assert plan.split_workspace_bytes(v.na) > 0
        pos = torch.from_numpy(v.positions).cuda()
        ech = torch.from_numpy(v.echo).cuda()
        a = plan.backproject(pos, ech)
        b = plan.backproject(pos, ech, split=True)
        torch.cuda.synchronize()
        a, b = a.cpu().numpy(), b.cpu().numpy()
    assert b.shape == (3, 40, 96) and _rel(b, a) <= 1e-5, _rel(b, a)


def test_split_workspace_rules(sb):
    """A grid that fills the GPU needs no workspace and runs unsplit (bit for bit the plain
    call); a short or overlapping workspace is refused before anything runs; fewer than 64
    pulses are not split."""
    import torch

    s = synth.make_scene("std", na=64, nr=1024, nx=1024, ny=1024, interp="linear", n_targets=2, clutter=False)
    with sb.Plan.for_scene(s) as plan:
        assert plan.split_workspace_bytes(s.na) == 0
        pos = torch.from_numpy(s.positions).cuda()
        ech = torch.from_numpy(s.echo).cuda()
        a = plan.backproject(pos, ech)
        b = plan.backproject(pos, ech, split=True)
        torch.cuda.synchronize()
        assert torch.equal(a, b)
    t = synth.make_scene("tiny")
    with sb.Plan.for_scene(t) as plan:
        assert plan.split_workspace_bytes(63) == 0 and plan.split_workspace_bytes(64) > 0
        need = plan.split_workspace_bytes(t.na)
        pos = torch.from_numpy(t.positions).cuda()
        ech = torch.from_numpy(t.echo).cuda()
        img = torch.zeros(plan.image_shape, dtype=torch.complex64, device="cuda")
        short = torch.empty(need - 8, dtype=torch.uint8, device="cuda")
        with pytest.raises(sb.SarbpError) as err:
            plan.backproject(pos, ech, image=img, split=True, workspace=short)
        assert err.value.status == sb.SARBP_EINVAL
        big = torch.empty(need + img.numel() * 8, dtype=torch.uint8, device="cuda")
        overlap = big[8:].view(torch.complex64)[: img.numel()].view(plan.image_shape)
        with pytest.raises(sb.SarbpError) as err:
            plan.backproject(pos, ech, image=overlap, split=True, workspace=big)
        assert err.value.status == sb.SARBP_EINVAL


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_most_carrier_cycles_per_bin(sb, interp):
    """3.98 m range bins at 3.125 cm: 254.7 carrier cycles per bin, just under the 255
    that plan creation accepts (the hardware sine and cosine take at most 256 cycles).
    The per-sample rotation then spans almost the whole argument range."""
    s = _custom_scene(synth.track(40), 1024, 70, 40, synth.PIXEL, synth.PIXEL, interp, 53, dr=3.98)
    _say(f"[cycles per bin {interp}] {2 * s.dr / s.wavelength:.1f}")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_anisotropic_squinted_grid(sb, interp):
    """0.15 m x 0.35 m pixels (a 41-bin window, which linear and nearest stage as 42) on
    a grid centred 300 m ahead of the track's middle (a squinted view), random echo:
    the full image against the oracle."""
    import dataclasses

    nx, ny, dx, dy = 150, 70, 0.15, 0.35
    s = _custom_scene(synth.track(160), 4096, nx, ny, dx, dy, interp, 41)
    s = dataclasses.replace(s, x0=300.0 - (nx // 2) * dx)
    _say(f"[anisotropic {interp}] {nx}x{ny} at {dx} x {dy} m, 300 m squint")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
@pytest.mark.parametrize("ny", [1024, 96])
def test_full_image_both_tile_heights(sb, interp, ny):
    """A random echo over a 1024-wide grid: 1024 rows give 512 tiles of 64 x 32 (two
    pixels per lane); 96 rows give too few for two per CU, so the plan takes 64 x 16
    tiles (one pixel per lane).  The full image against the oracle."""
    s = _custom_scene(synth.track(48), 2048, 1024, ny, synth.PIXEL, synth.PIXEL, interp, 43)
    _say(f"[tile heights {interp}] 1024 x {ny}")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)


@pytest.mark.parametrize("ground, height", [(400.0, 300.0), (1600.0, 1200.0)])
@pytest.mark.parametrize("interp", ["linear", "nearest", "sinc8"])
def test_short_range_series_modes(sb, interp, ground, height):
    """500 m and 2 km slant ranges: the tile-centre series needs its exact form or its
    third term there (bounds checked per pulse chunk in the kernel)."""
    na = 48
    t = (np.arange(na) - (na - 1) / 2) / synth.PRF
    pos = np.stack([synth.V_PLATFORM * t, np.full(na, -ground), np.full(na, height)], 1)
    s = _custom_scene(pos, 2048, 96, 64, synth.PIXEL, synth.PIXEL, interp, 37)
    _say(f"[short range {interp}] R = {np.hypot(ground, height):.0f} m")
    got = _run_bp(sb, s)
    want = oracle.scene_backproject(s)
    assert rel_l2(got, want) <= REL_L2, rel_l2(got, want)
