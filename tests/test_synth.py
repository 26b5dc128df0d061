"""Unit tests of the seeded scene generator (CPU)."""
import numpy as np

import synth


def test_same_seed_same_scene():
    a = synth.make_scene("tiny")
    b = synth.make_scene("tiny")
    assert a.sha256() == b.sha256()
    c = synth.make_scene("tiny", seed=5)
    assert c.sha256()["echo"] != a.sha256()["echo"]


def test_thread_count_does_not_change_the_echo():
    pos = synth.track(64)
    r0 = synth.RC_CENTRE - 256 * synth.DR
    rng = np.random.Generator(np.random.PCG64(3))
    pts = np.stack([rng.uniform(-5, 5, 50), rng.uniform(-5, 5, 50), np.zeros(50)], 1)
    amp = rng.standard_normal(50) + 1j * rng.standard_normal(50)
    e1 = synth.render_points(pos, 512, r0, synth.DR, pts, amp, half=4, nthreads=1)
    e4 = synth.render_points(pos, 512, r0, synth.DR, pts, amp, half=4, nthreads=4)
    assert np.array_equal(e1, e4)


def test_tabulated_grid_matches_direct_rendering():
    """The straight-track tabulation (shift invariance in x) reproduces the direct sum."""
    na, nr, nx, ny = 48, 256, 20, 12
    dx = dy = synth.PIXEL
    x0, y0, z0 = -(nx // 2) * dx, -(ny // 2) * dy, 0.0
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    pos = synth.track(na)
    rng = np.random.Generator(np.random.PCG64(4))
    sigma = synth.complex_normal(rng, (ny, nx), 1.0)
    a = np.zeros((na, nr), np.complex128)
    synth.render_grid_straight(na, nr, r0, synth.DR, nx, ny, x0, y0, z0, dx, dy, sigma, 4, a)
    jj, ii = np.meshgrid(np.arange(ny), np.arange(nx), indexing="ij")
    cells = np.stack([x0 + ii.ravel() * dx, y0 + jj.ravel() * dy, np.zeros(ii.size)], 1)
    b = synth.render_points(pos, nr, r0, synth.DR, cells, sigma.ravel(), half=4)
    assert np.max(np.abs(a - b)) < 1e-9 * np.max(np.abs(b))


def test_truncated_profile_equals_full_profile_near_peak():
    pos = synth.track(8)
    r0 = synth.RC_CENTRE - 256 * synth.DR
    pts = np.array([[1.3, -2.1, 0.0]])
    full = synth.render_points(pos, 512, r0, synth.DR, pts, [1.0], half=-1)
    trunc = synth.render_points(pos, 512, r0, synth.DR, pts, [1.0], half=4)
    nz = np.abs(trunc) > 0
    assert nz.sum() == 8 * 9
    assert np.max(np.abs(full[nz] - trunc[nz])) < 1e-12


def test_echo_sample_formula_spot_check():
    """A few samples of a one-target echo against the model written in numpy."""
    pos = synth.track(4)
    r0 = synth.RC_CENTRE - 256 * synth.DR
    p = np.array([0.8, -1.4, 0.0])
    e = synth.render_points(pos, 512, r0, synth.DR, p[None], [0.5 - 0.25j], half=-1)
    for n in range(4):
        R = np.linalg.norm(p - pos[n])
        u = (R - r0) / synth.DR
        for k in (int(u) - 3, int(u), int(u) + 5):
            want = (0.5 - 0.25j) * np.sinc(synth.BETA * (k - u)) * np.exp(-1j * 4 * np.pi * R / synth.WAVELENGTH)
            assert abs(e[n, k] - want) < 1e-10  # fp64 rounding of a 4.5e6 rad phase


def test_raw_chirp_spot_check():
    pos = synth.track(2)
    nfast = 4096
    r0 = synth.RC_CENTRE - (nfast // 2) * synth.DR
    p = np.array([2.0, 3.0, 0.0])
    raw = synth.render_chirp(pos, nfast, r0, p[None], [1.0])
    t0 = 2 * r0 / synth.C_LIGHT
    K = synth.BANDWIDTH / synth.CHIRP_T
    for n in range(2):
        R = np.linalg.norm(p - pos[n])
        tau = 2 * R / synth.C_LIGHT
        nz = np.nonzero(raw[n])[0]
        assert len(nz) == round(synth.CHIRP_T * synth.FS)
        for m in (nz[0], nz[len(nz) // 2], nz[-1]):
            t = t0 + m / synth.FS - tau
            want = np.exp(-1j * 4 * np.pi * R / synth.WAVELENGTH) * np.exp(1j * np.pi * K * t * t)
            assert -synth.CHIRP_T / 2 <= t < synth.CHIRP_T / 2
            assert abs(raw[n, m] - want) < 1e-9


def test_targets_are_central_and_separated():
    rng = np.random.Generator(np.random.PCG64(1))
    for k, side in ((5, 128), (25, 1024), (64, 2048)):
        t = synth.target_pixels(side, side, k, rng)
        assert len(t) == k and len({tuple(x) for x in t}) == k
        assert t.min() >= 0.1 * side - 1 and t.max() <= 0.9 * side
        d = np.sqrt(((t[:, None, :] - t[None, :, :]) ** 2).sum(-1)) + np.eye(k) * 1e9
        assert d.min() > 0.8 * side / np.ceil(np.sqrt(k)) * 0.5 - 1


def test_noise_power():
    a = synth.make_scene("tiny")
    b = synth.make_scene("tiny", noise_var=0.0)
    n = (a.echo.astype(np.complex128) - b.echo.astype(np.complex128)).ravel()
    var = np.mean(np.abs(n) ** 2)
    se = 0.01 / np.sqrt(n.size)
    assert abs(var - 0.01) < 4 * se


def test_perturbed_track_is_smooth_and_bounded():
    rng = np.random.Generator(np.random.PCG64(2))
    p = synth.track(4096, rng, perturbed=True)
    s = synth.track(4096)
    d = p - s
    assert np.max(np.abs(d)) <= 0.5 + 1e-12
    assert np.max(np.abs(d)) > 0.05
    assert np.max(np.abs(np.diff(d, axis=0))) < 2 * np.pi * 0.5 * 0.5 / synth.PRF + 1e-9


def test_config_geometry():
    s = synth.make_scene("tiny")
    assert s.positions.shape == (256, 3) and s.echo.shape == (256, 512) and s.echo.dtype == np.complex64
    # scene centre (pixel nx/2, ny/2) is the origin; the record is centred on its range
    x, y = s.pixel_xy(s.nx // 2, s.ny // 2)
    assert x == 0.0 and y == 0.0
    assert abs(s.r0 + (s.nr // 2) * s.dr - synth.RC_CENTRE) < 1e-9
    rho_az, rho_rg = synth.resolution(s)
    assert abs(rho_az - 3.41) < 0.01 and abs(rho_rg - 0.559) < 0.001
