"""Pins of the oracle's terrain variant (pixel (i, j) at height z0 + dem[j, i]; the page,
section 3.3, notes that terrain height may have to enter the range history)."""
import numpy as np
import pytest

import oracle
import synth
from test_oracle_pins import _geom, _h


def _dem_bp(g, echo, interp, dem):
    return oracle.backproject(g["pos"], echo, r0=g["r0"], dr=g["dr"], nx=g["nx"], ny=g["ny"], x0=g["x0"],
                              y0=g["y0"], z0=g["z0"], dx=g["dx"], dy=g["dy"], wavelength=synth.WAVELENGTH,
                              interp=interp, dem=dem)


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_flat_dem_is_the_plane(interp):
    g = _geom(na=24, nr=512, nx=20, ny=16)
    rng = np.random.Generator(np.random.PCG64(2))
    echo = (rng.standard_normal((24, 512)) + 1j * rng.standard_normal((24, 512))).astype(np.complex64)
    plane = oracle.backproject(g["pos"], echo, g["r0"], g["dr"], g["nx"], g["ny"], g["x0"], g["y0"], g["z0"],
                               g["dx"], g["dy"], synth.WAVELENGTH, interp)
    flat = _dem_bp(g, echo, interp, np.zeros((g["ny"], g["nx"]), np.float32))
    assert np.array_equal(plane, flat)
    # a constant height h equals the plane z0 + h
    h = np.float32(7.25)
    lifted = _dem_bp(g, echo, interp, np.full((g["ny"], g["nx"]), h, np.float32))
    plane_h = oracle.backproject(g["pos"], echo, g["r0"], g["dr"], g["nx"], g["ny"], g["x0"], g["y0"],
                                 g["z0"] + float(h), g["dx"], g["dy"], synth.WAVELENGTH, interp)
    assert np.array_equal(lifted, plane_h)


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_target_on_terrain_focuses_to_the_closed_form(interp):
    """A unit target on a hill (12.5 m above the plane): on the terrain the image at its
    pixel is real, positive and equals sum_n w(f_n) with the ranges taken to the raised
    point; the flat plane puts the target ~5 m off in range and loses the peak."""
    g = _geom(na=96, nr=512, nx=40, ny=36, perturbed=True)
    i, j = 23, 17
    dem = synth.terrain(g["nx"], g["ny"], g["dx"], g["dy"], np.random.Generator(np.random.PCG64(8)), 8.0)
    dem = dem + np.float32(12.5) - dem[j, i]
    hz = float(dem[j, i])
    pts = np.array([[g["x0"] + i * g["dx"], g["y0"] + j * g["dy"], hz]])
    echo = synth.render_points(g["pos"], g["nr"], g["r0"], g["dr"], pts, [1.0], half=-1)
    img = _dem_bp(g, echo, interp, dem)
    R = np.sqrt((pts[0, 0] - g["pos"][:, 0]) ** 2 + (pts[0, 1] - g["pos"][:, 1]) ** 2 + (hz - g["pos"][:, 2]) ** 2)
    u = (R - g["r0"]) / g["dr"]
    f = u - np.floor(u)
    b = synth.BETA
    if interp == "linear":
        w = (1 - f) * np.sinc(b * f) + f * np.sinc(b * (1 - f))
    elif interp == "nearest":
        w = np.sinc(b * np.abs(f - np.round(f)))
    else:
        w = sum(_h(f - m) * np.sinc(b * (m - f)) for m in range(-3, 5))
    peak = img[j, i]
    assert abs(peak.real - w.sum()) / w.sum() < 1e-12
    assert abs(peak.imag) / peak.real < 1e-8
    # On sloping ground a neighbour can lie almost on the target's iso-range surface,
    # and the linear interpolator's response varies from 0.74 to 1 with the fraction,
    # so the argmax may move one pixel; the target stays within 10 % of the maximum.
    assert abs(peak) >= 0.9 * np.abs(img).max()
    flat = oracle.backproject(g["pos"], echo, g["r0"], g["dr"], g["nx"], g["ny"], g["x0"], g["y0"], g["z0"],
                              g["dx"], g["dy"], synth.WAVELENGTH, interp)
    assert np.abs(flat).max() < 0.2 * abs(peak)


def test_pixels_variant_matches_rows_variant():
    g = _geom(na=16, nr=512, nx=24, ny=20)
    rng = np.random.Generator(np.random.PCG64(4))
    echo = (rng.standard_normal((16, 512)) + 1j * rng.standard_normal((16, 512))).astype(np.complex64)
    dem = synth.terrain(g["nx"], g["ny"], g["dx"], g["dy"], rng, 20.0)
    img = _dem_bp(g, echo, "linear", dem)
    ij = np.array([[0, 0], [5, 7], [23, 19], [11, 3]])
    px = oracle.backproject_pixels(g["pos"], echo, g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"],
                                   synth.WAVELENGTH, "linear", ij, dem=dem)
    assert np.array_equal(px, img[ij[:, 1], ij[:, 0]])


def test_terrain_generator_and_block_bound():
    rng = np.random.Generator(np.random.PCG64(1))
    dem = synth.terrain(200, 100, 0.2, 0.2, rng, 30.0)
    assert dem.dtype == np.float32 and abs(float(dem.max() - dem.min()) - 30.0) < 1e-4
    r = synth.block_relief(dem)
    assert 0 < r <= 30.0
    blk = dem[32:64, 64:128].astype(np.float64)
    assert blk.max() - blk.min() <= r



# --------------------------------------------------------------------------- 3-D (voxel) images

def _volume_case(dh, interp):
    pos = synth.multipass_track(8, 32, dh)
    nr, nx, ny, nz = 512, 24, 20, 12
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    dx = dy = synth.PIXEL
    x0, y0, z0, dz = -(nx // 2) * dx, -(ny // 2) * dy, -1.5, 0.25
    i, j, l = 13, 9, 10
    pt = np.array([[x0 + i * dx, y0 + j * dy, z0 + l * dz]])
    echo = synth.render_points(pos, nr, r0, synth.DR, pt, [1.0], half=-1)
    v = oracle.backproject_volume(pos, echo, r0, synth.DR, nx, ny, nz, x0, y0, z0, dx, dy, dz, synth.WAVELENGTH,
                                  interp)
    return pos, pt[0], r0, v, (l, j, i)


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_volume_target_focuses_in_height(interp):
    """8 parallel passes 40 m apart in height (280 m of elevation aperture): a unit
    target 1 m above the plane focuses at its voxel to the closed form sum_n w(f_n)
    (real, positive) and is the brightest voxel, with the neighbouring layers of its
    column below 0.8 and two layers away below 0.3.  A single pass, with no elevation
    aperture, smears the column (neighbours above 0.9)."""
    pos, pt, r0, v, (l, j, i) = _volume_case(40.0, interp)
    R = np.linalg.norm(pos - pt, axis=1)
    u = (R - r0) / synth.DR
    f = u - np.floor(u)
    b = synth.BETA
    if interp == "linear":
        w = (1 - f) * np.sinc(b * f) + f * np.sinc(b * (1 - f))
    elif interp == "nearest":
        w = np.sinc(b * np.abs(f - np.round(f)))
    else:
        w = sum(_h(f - m) * np.sinc(b * (m - f)) for m in range(-3, 5))
    peak = v[l, j, i]
    assert abs(peak.real - w.sum()) / w.sum() < 1e-12
    assert abs(peak.imag) / peak.real < 1e-8
    assert np.unravel_index(np.argmax(np.abs(v)), v.shape) == (l, j, i)
    col = np.abs(v[:, j, i]) / abs(peak)
    assert col[l - 1] < 0.8 and col[l + 1] < 0.8 and col[l - 2] < 0.3
    _, _, _, v1, _ = _volume_case(0.0, interp)
    c1 = np.abs(v1[:, j, i]) / np.abs(v1[:, j, i]).max()
    assert c1[l - 1] > 0.9 and c1[l + 1] > 0.9


def test_volume_layers_are_planes():
    """Layer l of a volume equals the plane image at z0 + l dz, bit for bit."""
    pos, _, r0, v, _ = _volume_case(40.0, "linear")
    rng = np.random.Generator(np.random.PCG64(3))
    echo = (rng.standard_normal((len(pos), 512)) + 1j * rng.standard_normal((len(pos), 512))).astype(np.complex64)
    vol = oracle.backproject_volume(pos, echo, r0, synth.DR, 8, 6, 3, -0.8, -0.6, 2.0, 0.2, 0.2, 0.5,
                                    synth.WAVELENGTH, "sinc8")
    plane = oracle.backproject(pos, echo, r0, synth.DR, 8, 6, -0.8, -0.6, 2.0 + 2 * 0.5, 0.2, 0.2,
                               synth.WAVELENGTH, "sinc8")
    assert np.array_equal(vol[2], plane)


def test_nearest_index_on_terrain_is_the_ramp_probe():
    """oracle.nearest_index with per-pixel heights equals the bin the terrain definition selects:
    one pulse with echo s[k] = k + 1 gives |I| - 1 = floor(u + 1/2) exactly (the backprojection's
    terrain variant is pinned against the 40-digit brute force); a flat map equals the plane
    index, and a constant height h equals the plane at z0 + h."""
    g = _geom(na=1, nr=512, nx=24, ny=20)
    rng = np.random.Generator(np.random.PCG64(9))
    dem = rng.uniform(-6.0, 9.0, (g["ny"], g["nx"])).astype(np.float32)
    echo = (np.arange(g["nr"]) + 1.0).astype(np.complex128)[None, :]
    img = _dem_bp(g, echo, "nearest", dem)
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    ij = np.stack([ii.ravel(), jj.ravel()], 1)
    k = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"], ij, dem=dem)
    got = np.abs(img).ravel() - 1.0
    assert np.max(np.abs(got - np.rint(got))) < 1e-9
    assert np.array_equal(np.rint(got).astype(np.int64), k)
    assert len(np.unique(k)) > 3  # the heights move the selected bin
    flat = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"], ij,
                                dem=np.zeros_like(dem))
    plane = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"], ij)
    assert np.array_equal(flat, plane)
    h = np.float32(3.5)
    lifted = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"], ij,
                                  dem=np.full_like(dem, h))
    plane_h = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"] + float(h), g["dx"],
                                   g["dy"], ij)
    assert np.array_equal(lifted, plane_h)
