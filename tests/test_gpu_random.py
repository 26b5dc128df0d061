"""GPU parity on seeded random geometries: the HIP library against the oracle over a spread
of problem shapes no fixed workload covers.

Each case draws, from its own seed:
* the interpolator and the accumulator;
* the carrier wavelength (Ka, X, C or L band);
* grid sides of 1-160 x 1-120 pixels with anisotropic spacing of 0.05-6 m, so both
  tile heights, ragged tiles, the fp64-range kernels and the large-LDS windows occur;
* a track of 1-300 pulses at any heading, squinted up to 45 degrees, 0.2-20 km away
  and 0.1-10 km up, with a smooth random wobble;
* range bins of 0.05-2 m (capped so that 2 dr / lambda stays below 250 carrier
  cycles per bin, and widened where a tile's window would not fit in LDS);
* a record of 8-4096 bins placed anywhere from well before to well after the
  scene, so pixels often fall partly or wholly outside it (zero extension);
* for a quarter of the cases, rough terrain of up to 30 m peak to peak (on the fp32
  or, for windows of many carrier cycles, the fp64-range terrain kernels);
* for half of the cases, two calls that split the pulses, the second accumulating;
* for about a tenth (flat ones), a volume of 2-6 layers 0.1-20 m apart.

Every case also runs through sarbp_backproject_split (pulse groups for small grids;
most of these grids are small), against the oracle and against the plain call.

The bar is the fine grids' one (relative L2 error at most REL_L2).  A case whose record
misses the whole scene must give exactly zero.
"""
import math
import sys

import numpy as np
import pytest

import oracle
import synth
from _parity import REL_L2, rel_l2
from _probe import nearest_index_mismatches

N_CASES = 128
WAVELENGTHS = (0.0086, 0.03125, 0.0556, 0.236)


@pytest.fixture(scope="module")
def sb(gpu_device):  # requested by the gpu-marked test only
    from domain_backprojection_amd import sarbp

    return sarbp


def _loguniform(rng, lo, hi):
    return float(math.exp(rng.uniform(math.log(lo), math.log(hi))))


def random_case(seed):
    """One random problem: (scene, accum, split, layers) with split = 0 for a single call,
    else the number of pulses in the first of two calls, and layers = (nz, dz) for a
    volume, else None."""
    rng = np.random.Generator(np.random.PCG64(seed))
    interp = ("nearest", "linear", "sinc8")[int(rng.integers(3))]
    accum = ("fp32", "kahan", "chunk64")[int(rng.integers(3))]
    lam = float(WAVELENGTHS[int(rng.integers(len(WAVELENGTHS)))])
    nx = max(1, int(_loguniform(rng, 1, 161)))
    ny = max(1, int(_loguniform(rng, 1, 121)))
    na = max(1, int(_loguniform(rng, 1, 301)))
    terrain = rng.uniform() < 0.25
    dx, dy = _loguniform(rng, 0.05, 6.0), _loguniform(rng, 0.05, 6.0)
    half_diag = lambda: 0.5 * math.hypot(64 * dx, 32 * dy)

    # Track: broadside point at ground range G, bearing phi from the scene centre; the
    # track runs perpendicular to the line of sight, turned by a squint of up to 45 deg.
    G, H = _loguniform(rng, 200.0, 20000.0), _loguniform(rng, 100.0, 10000.0)
    phi = rng.uniform(0.0, 2.0 * math.pi)
    squint = rng.uniform(-math.pi / 4, math.pi / 4)
    heading = phi + math.pi / 2 + squint
    step = _loguniform(rng, 0.02, 1.0)  # along-track spacing [m]
    s = (np.arange(na) - (na - 1) / 2) * step
    wob = rng.uniform(0.0, 0.5, 3)
    fr = rng.uniform(0.5, 3.0, 3)
    ph = rng.uniform(0.0, 2.0 * math.pi, 3)
    pos = np.stack([G * math.cos(phi) + s * math.cos(heading), G * math.sin(phi) + s * math.sin(heading),
                    np.full(na, H)], axis=1)
    pos += wob * np.sin(2.0 * math.pi * fr * s[:, None] / max(1.0, step * na) + ph)
    x0, y0 = -(nx // 2) * dx, -(ny // 2) * dy
    Rc = float(np.linalg.norm(pos[na // 2]))

    dr = _loguniform(rng, 0.05, 2.0)
    dr = max(dr, 2.0 * half_diag() / 1800.0)  # keep each tile's window within the LDS limit
    dr = min(dr, 125.0 * lam)  # at most 250 carrier cycles per bin
    nr = max(8, int(_loguniform(rng, 8, 4097)))
    r0 = Rc - rng.uniform(-0.3, 1.3) * nr * dr

    dem = None
    if terrain:
        h = rng.uniform(0.0, 15.0)
        dem = rng.uniform(-1.0, 1.0, (ny, nx)).astype(np.float32) * np.float32(h)
    echo = (rng.standard_normal((na, nr)) + 1j * rng.standard_normal((na, nr))).astype(np.complex64)
    scene = synth.Scene(name=f"random{seed}", seed=seed, na=na, nr=nr, nx=nx, ny=ny, x0=x0, y0=y0, z0=0.0,
                        dx=dx, dy=dy, r0=r0, dr=dr, wavelength=lam, interp=interp, positions=pos, echo=echo,
                        raw=None, targets=np.zeros((0, 2), np.int64), dem=dem)
    split = int(rng.integers(1, na)) if (na > 1 and rng.uniform() < 0.5) else 0
    layers = None
    if dem is None and rng.uniform() < 0.15:
        layers = (int(rng.integers(2, 7)), _loguniform(rng, 0.1, 20.0))
    return scene, accum, split, layers


def expected(scene, layers):
    """The oracle's image: the plane (or terrain) definition, or each layer of a volume."""
    if layers is None:
        return oracle.scene_backproject(scene)
    return oracle.backproject_volume(scene.positions, scene.echo, scene.r0, scene.dr, scene.nx, scene.ny, layers[0],
                                     scene.x0, scene.y0, scene.z0, scene.dx, scene.dy, layers[1], scene.wavelength,
                                     scene.interp)


def _run(sb, scene, accum, split, layers=None, groups=False):
    import torch

    kw = dict(accum=accum)
    if layers is not None:
        kw.update(nz=layers[0], dz=layers[1])
    dem_d = None
    if scene.dem is not None:
        kw["dem_relief"] = max(synth.block_relief(scene.dem), 1e-3)
        dem_d = torch.from_numpy(np.ascontiguousarray(scene.dem)).cuda()
    with sb.Plan.for_scene(scene, **kw) as plan:
        pos = torch.from_numpy(np.ascontiguousarray(scene.positions)).cuda()
        ech = torch.from_numpy(np.ascontiguousarray(scene.echo)).cuda()
        if split:
            img = plan.backproject(pos[:split].contiguous(), ech[:split].contiguous(), dem=dem_d, split=groups)
            plan.backproject(pos[split:].contiguous(), ech[split:].contiguous(), image=img, accumulate=1, dem=dem_d,
                             split=groups)
        else:
            img = plan.backproject(pos, ech, dem=dem_d, split=groups)
        torch.cuda.synchronize()
        return img.cpu().numpy().astype(np.complex128)


def test_random_case_generator_is_seeded():
    """The generator itself (no GPU use): the same seed gives the same case."""
    a, acc_a, split_a, lay_a = random_case(5)
    b, acc_b, split_b, lay_b = random_case(5)
    assert (acc_a, split_a, lay_a, a.interp, a.nx, a.ny, a.na) == (acc_b, split_b, lay_b, b.interp, b.nx, b.ny, b.na)
    assert np.array_equal(a.echo, b.echo) and np.array_equal(a.positions, b.positions)


@pytest.mark.gpu
@pytest.mark.parametrize("seed", range(7000, 7000 + N_CASES))
def test_random_geometry_matches_oracle(sb, seed):
    scene, accum, split, layers = random_case(seed)
    print(f"[random {seed}] {scene.interp} {accum} {scene.nx}x{scene.ny} px {scene.dx:.3g}x{scene.dy:.3g} m, "
          f"{scene.na} pulses x {scene.nr} bins of {scene.dr:.3g} m, lambda {scene.wavelength}, "
          f"terrain {scene.dem is not None}, split {split}, layers {layers}", flush=True)
    sys.stdout.flush()
    got = _run(sb, scene, accum, split, layers)
    grouped = _run(sb, scene, accum, split, layers, groups=True)
    want = expected(scene, layers)
    assert np.isfinite(got).all() and np.isfinite(grouped).all()
    if np.linalg.norm(want) == 0.0:
        assert np.all(got == 0) and np.all(grouped == 0)
    else:
        err, err_g = rel_l2(got, want), rel_l2(grouped, want)
        print(f"[random {seed}] rel-L2 {err:.2e} (pulse groups {err_g:.2e})", flush=True)
        assert err <= REL_L2, err
        assert err_g <= REL_L2, err_g
        assert np.linalg.norm(grouped - got) <= 1e-5 * np.linalg.norm(got)
    if scene.interp == "nearest":
        # every pixel of every pulse (at most 64, evenly spaced, first and last included)
        pulses = sorted(set(np.linspace(0, scene.na - 1, min(scene.na, 64)).astype(int).tolist()))
        kw = {}
        if scene.dem is not None:
            kw["dem_relief"] = max(synth.block_relief(scene.dem), 1e-3)
        bad = nearest_index_mismatches(sb, scene, pulses, dem=scene.dem, layers=layers, **kw)
        print(f"[random {seed}] nearest index probe: {len(pulses)} pulses, {bad} mismatches", flush=True)
        assert bad == 0
