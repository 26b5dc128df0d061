"""Pins of the CPU oracle to things other than itself (closed forms, textbook
impulse-response figures, special cases, invariants, the page's printed numbers).

Each pin is chosen so that a plausible mistake in the oracle fails at least one:

* wrong phase sign / dropped range term / wrong pixel coordinates / transposed image
  -> single-target closed form and peak location
* swapped linear weights, off-by-one bin, wrong r0 -> ramp and delta echoes
* misaligned sinc8 taps -> half-sample symmetry and continuity
* skipped or repeated pulses -> closed-form peak value (a sum over every pulse)
* missing conj / wrong window / wrong normalisation in range compression -> RC pins
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = json.load(open(os.path.join(HERE, "golden", "pages_numbers.json"), encoding="utf-8"))


def _geom(na=32, nr=512, nx=24, ny=20, perturbed=False, seed=7):
    rng = np.random.Generator(np.random.PCG64(seed))
    pos = synth.track(na, rng, perturbed=perturbed)
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    dx = dy = synth.PIXEL
    x0, y0 = -(nx // 2) * dx, -(ny // 2) * dy
    return dict(pos=pos, nr=nr, r0=r0, dr=synth.DR, nx=nx, ny=ny, x0=x0, y0=y0, z0=0.0, dx=dx, dy=dy)


def _bp(g, echo, interp, pos=None, **kw):
    p = g["pos"] if pos is None else pos
    a = dict(r0=g["r0"], dr=g["dr"], nx=g["nx"], ny=g["ny"], x0=g["x0"], y0=g["y0"], z0=g["z0"],
             dx=g["dx"], dy=g["dy"], wavelength=synth.WAVELENGTH, interp=interp)
    a.update(kw)
    return oracle.backproject(p, echo, **a)


def _u(g, pos, i, j):
    """Fractional bin position of pixel (i, j) for every pulse, computed with numpy."""
    x = g["x0"] + np.asarray(i) * g["dx"]
    y = g["y0"] + np.asarray(j) * g["dy"]
    R = np.sqrt((x - pos[:, 0]) ** 2 + (y - pos[:, 1]) ** 2 + (g["z0"] - pos[:, 2]) ** 2)
    return (R - g["r0"]) / g["dr"], R


def _h(t):
    t = np.asarray(t, dtype=np.float64)
    return np.where(np.abs(t) < 4, np.sinc(t) * (0.54 + 0.46 * np.cos(np.pi * t / 4)), 0.0)


# --------------------------------------------------------------------------- focusing

@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_single_target_closed_form_peak(interp):
    """Noise-free unit target on a pixel: the image there is real, positive and equals
    sum_n w(f_n) for the interpolator's response w to a sampled sinc."""
    g = _geom(na=96, nr=512, nx=40, ny=36, perturbed=True)
    i, j = 23, 17
    pts = np.array([[g["x0"] + i * g["dx"], g["y0"] + j * g["dy"], 0.0]])
    echo = synth.render_points(g["pos"], g["nr"], g["r0"], g["dr"], pts, [1.0], half=-1)
    img = _bp(g, echo, interp)
    u, _ = _u(g, g["pos"], i, j)
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
    assert np.unravel_index(np.argmax(np.abs(img)), img.shape) == (j, i)


def _cut_width_and_pslr(x, mag):
    """-3 dB width (linear interpolation of the crossing) and peak sidelobe ratio [dB]."""
    p = int(np.argmax(mag))
    m = mag / mag[p]
    half = 1 / np.sqrt(2)
    lo = p
    while m[lo] > half:
        lo -= 1
    hi = p
    while m[hi] > half:
        hi += 1
    xl = x[lo] + (half - m[lo]) * (x[lo + 1] - x[lo]) / (m[lo + 1] - m[lo])
    xh = x[hi - 1] + (half - m[hi - 1]) * (x[hi] - x[hi - 1]) / (m[hi] - m[hi - 1])
    # first nulls: walk down from the peak to the first local minima
    a = p
    while a > 0 and m[a - 1] < m[a]:
        a -= 1
    b = p
    while b < len(m) - 1 and m[b + 1] < m[b]:
        b += 1
    side = max(m[:a].max() if a > 0 else 0, m[b + 1:].max() if b < len(m) - 1 else 0)
    return xh - xl, 20 * np.log10(side)


def test_point_spread_function_matches_textbook():
    """Mainlobe widths and sidelobes of an isolated target on the tiny geometry (256
    pulses): azimuth -3 dB width 0.886*lambda*R/(2L) and uniform-aperture sidelobes near
    -13.26 dB (linear interpolation); ground-range width 0.886*(c/2B)/sin(theta) with the
    near-ideal sinc8 interpolator (linear interpolation of a 1.2x-oversampled profile is not
    band-limited and narrows the range response to ~0.35 m, so it is not a textbook case)."""
    na, nr = 256, 512
    pos = synth.track(na)
    r0 = synth.RC_CENTRE - (nr // 2) * synth.DR
    pts = np.array([[0.0, 0.0, 0.0]])
    echo = synth.render_points(pos, nr, r0, synth.DR, pts, [1.0], half=-1)
    L = synth.V_PLATFORM * na / synth.PRF
    rho_az = 0.886 * synth.WAVELENGTH * synth.RC_CENTRE / (2 * L)
    rho_rg = 0.886 * synth.C_LIGHT / (2 * synth.BANDWIDTH) * synth.RC_CENTRE / synth.GROUND_RANGE
    # azimuth cut: fine grid along x through the target
    ddx, nxa = 0.05, 801
    az = oracle.backproject(pos, echo, r0, synth.DR, nxa, 1, -(nxa // 2) * ddx, 0.0, 0.0, ddx, 1.0,
                            synth.WAVELENGTH, "linear")[0]
    xa = (np.arange(nxa) - nxa // 2) * ddx
    w_az, pslr_az = _cut_width_and_pslr(xa, np.abs(az))
    # range cut: fine grid along y
    ddy, nyr = 0.01, 801
    rg = oracle.backproject(pos, echo, r0, synth.DR, 1, nyr, 0.0, -(nyr // 2) * ddy, 0.0, 1.0, ddy,
                            synth.WAVELENGTH, "sinc8")[:, 0]
    yr = (np.arange(nyr) - nyr // 2) * ddy
    w_rg, pslr_rg = _cut_width_and_pslr(yr, np.abs(rg))
    assert abs(w_az / rho_az - 1) < 0.10, (w_az, rho_az)
    assert abs(w_rg / rho_rg - 1) < 0.10, (w_rg, rho_rg)
    assert abs(pslr_az + 13.26) < 1.0, pslr_az
    assert abs(pslr_rg + 13.26) < 1.5, pslr_rg
    assert np.argmax(np.abs(az)) == nxa // 2 and np.argmax(np.abs(rg)) == nyr // 2


# --------------------------------------------------------------------------- special cases

def _single_pulse_geom():
    g = _geom(na=1, nr=4096, nx=48, ny=40)
    g["pos"] = np.array([[3.0, -synth.GROUND_RANGE, synth.ALTITUDE]])
    return g


def test_index_probe_nearest():
    """One pulse, echo s[k] = k + 1 (real): |I(p)| - 1 is exactly the chosen bin floor(u + 1/2),
    which also equals oracle.nearest_index and the numpy formula."""
    g = _single_pulse_geom()
    echo = (np.arange(g["nr"]) + 1.0).astype(np.complex128)[None, :]
    img = _bp(g, echo, "nearest")
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    u, _ = _u(g, g["pos"], ii[..., None], jj[..., None])
    k_np = np.floor(u[..., 0] + 0.5)
    got = np.abs(img) - 1.0
    assert np.max(np.abs(got - np.rint(got))) < 1e-9
    assert np.array_equal(np.rint(got), k_np)
    ij = np.stack([ii.ravel(), jj.ravel()], 1)
    k_or = oracle.nearest_index(g["pos"][0], g["r0"], g["dr"], g["x0"], g["y0"], g["z0"], g["dx"], g["dy"], ij)
    assert np.array_equal(k_or, k_np.ravel().astype(np.int64))


def test_delta_echo_selects_one_bin():
    """One pulse, s = delta at k*: I(p) = exp(j 4 pi R / lambda) where floor(u + 1/2) = k*, else 0."""
    g = _single_pulse_geom()
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    u, R = _u(g, g["pos"], ii[..., None], jj[..., None])
    kstar = int(np.floor(np.median(u)) )
    echo = np.zeros((1, g["nr"]), np.complex128)
    echo[0, kstar] = 1.0
    img = _bp(g, echo, "nearest")
    sel = np.floor(u[..., 0] + 0.5) == kstar
    assert sel.any() and (~sel).any()
    expect = np.where(sel, np.exp(1j * 4 * np.pi * R[..., 0] / synth.WAVELENGTH), 0)
    assert np.max(np.abs(img - expect)) < 1e-12


def test_ramp_echo_is_reproduced_by_linear():
    """One pulse, s[k] = k (real): linear interpolation returns u exactly, so |I(p)| = u(p)."""
    g = _single_pulse_geom()
    echo = np.arange(g["nr"], dtype=np.complex128)[None, :]
    img = _bp(g, echo, "linear")
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    u, R = _u(g, g["pos"], ii[..., None], jj[..., None])
    assert np.max(np.abs(np.abs(img) - u[..., 0]) / u[..., 0]) < 1e-12
    ph = np.angle(img * np.exp(-1j * 4 * np.pi * R[..., 0] / synth.WAVELENGTH))
    assert np.max(np.abs(ph)) < 1e-8


@pytest.mark.parametrize("interp", ["nearest", "linear"])
def test_constant_echo_partition_of_unity(interp):
    """One pulse, s = 1: nearest and linear weights sum to one, so |I| = 1 inside the record."""
    g = _single_pulse_geom()
    echo = np.ones((1, g["nr"]), np.complex128)
    img = _bp(g, echo, interp)
    assert np.max(np.abs(np.abs(img) - 1.0)) < 1e-12


def test_zero_extension_outside_record():
    """Samples beyond the record are zero: a pixel whose bin is far off contributes nothing,
    and a pixel between the last bin and the next gets (1 - f) of the last sample."""
    g = _single_pulse_geom()
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    u, R = _u(g, g["pos"], ii[..., None], jj[..., None])
    u = u[..., 0]
    # shift r0 so that the grid's bins straddle the end of a short record
    nr = 64
    kmid = np.floor(np.median(u))
    shift = kmid - (nr - 1)
    g2 = dict(g, nr=nr, r0=g["r0"] + shift * g["dr"])
    echo = np.ones((1, nr), np.complex128)
    img = _bp(g2, echo, "linear")
    u2 = u - shift
    inside = u2 <= nr - 1
    tail = (u2 > nr - 1) & (u2 < nr)
    far = u2 >= nr
    assert inside.any() and tail.any() and far.any()
    assert np.max(np.abs(np.abs(img[inside]) - 1)) < 1e-9
    f = u2[tail] - np.floor(u2[tail])
    assert np.max(np.abs(np.abs(img[tail]) - (1 - f))) < 1e-9
    assert np.max(np.abs(img[far])) == 0.0


# --------------------------------------------------------------------------- invariants

def _random_echo(na, nr, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return rng.standard_normal((na, nr)) + 1j * rng.standard_normal((na, nr))


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_linearity(interp):
    g = _geom(na=24, nr=512, nx=16, ny=12)
    s1, s2 = _random_echo(24, 512, 1), _random_echo(24, 512, 2)
    a, b = 0.7 - 0.2j, -1.3 + 0.4j
    lhs = _bp(g, a * s1 + b * s2, interp)
    rhs = a * _bp(g, s1, interp) + b * _bp(g, s2, interp)
    assert np.linalg.norm(lhs - rhs) / np.linalg.norm(rhs) < 1e-12


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_pulse_order_invariance(interp):
    g = _geom(na=24, nr=512, nx=16, ny=12, perturbed=True)
    s = _random_echo(24, 512, 3)
    perm = np.random.Generator(np.random.PCG64(9)).permutation(24)
    a = _bp(g, s, interp)
    b = _bp(g, s[perm], interp, pos=g["pos"][perm])
    assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-12


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_global_phase_covariance(interp):
    g = _geom(na=16, nr=512, nx=12, ny=10)
    s = _random_echo(16, 512, 4)
    th = np.exp(1j * 0.937)
    a = _bp(g, s * th, interp)
    b = _bp(g, s, interp) * th
    assert np.linalg.norm(a - b) / np.linalg.norm(b) < 1e-12


def test_translation_invariance():
    """Moving antennas and grid by one vector leaves every range, hence the image, unchanged."""
    g = _geom(na=16, nr=512, nx=12, ny=10, perturbed=True)
    s = _random_echo(16, 512, 5)
    t = np.array([1.0e5, -3.0e4, 250.0])
    a = _bp(g, s, "linear")
    b = _bp(g, s, "linear", pos=g["pos"] + t, x0=g["x0"] + t[0], y0=g["y0"] + t[1], z0=g["z0"] + t[2])
    assert np.linalg.norm(a - b) / np.linalg.norm(a) < 1e-7


# --------------------------------------------------------------------------- sinc8 kernel

def test_sinc8_kernel_interpolating_and_symmetric():
    assert oracle.sinc8_weight(0.0) == 1.0
    for m in range(1, 5):
        assert abs(oracle.sinc8_weight(m)) < 1e-15 and abs(oracle.sinc8_weight(-m)) < 1e-15
    for t in np.linspace(0.01, 3.99, 37):
        assert oracle.sinc8_weight(t) == oracle.sinc8_weight(-t)
    assert oracle.sinc8_weight(4.0) == 0.0 and oracle.sinc8_weight(4.5) == 0.0


def test_sinc8_half_sample_symmetry_and_continuity():
    """Taps k-3..k+4 around u = k + f: an echo mirrored about k + 1/2 gives a real result at
    f = 1/2 for a symmetric-phase pulse, and the interpolant is continuous across integer u."""
    g = _single_pulse_geom()
    s = _random_echo(1, g["nr"], 6)
    jj, ii = np.meshgrid(np.arange(g["ny"]), np.arange(g["nx"]), indexing="ij")
    u, R = _u(g, g["pos"], ii[..., None], jj[..., None])
    u = u[..., 0]
    k = np.floor(u).astype(int)
    f = u - k
    img = _bp(g, s, "sinc8") * np.exp(-1j * 4 * np.pi * R[..., 0] / synth.WAVELENGTH)
    # direct evaluation of the taps in numpy for every pixel
    expect = sum(s[0, k + m] * _h(f - m) for m in range(-3, 5))
    assert np.max(np.abs(img - expect)) < 1e-12
    # mirrored echo about kc + 1/2: v(kc + 1/2) must equal the sum over symmetric pairs
    kc = int(np.median(k))
    sym = np.zeros(g["nr"], np.complex128)
    for m in range(0, 4):
        sym[kc - m] = sym[kc + 1 + m] = 1.0 + m
    w = [_h(0.5 - m) for m in range(-3, 5)]
    v_mid = sum(sym[kc + m] * w[m + 3] for m in range(-3, 5))
    assert abs(v_mid.imag) == 0.0
    assert np.allclose(w, w[::-1], rtol=0, atol=1e-15)
    # continuity: the tap sum at u -> k+1 from below equals the tap sum at u = k+1
    below = sum(sym[kc + m] * _h(1 - 1e-12 - m) for m in range(-3, 5))
    at = sum(sym[kc + 1 + m] * _h(0.0 - m) for m in range(-3, 5))
    assert abs(below - at) < 1e-9


# --------------------------------------------------------------------------- range compression

def _raw_single(nfast, delay_bins, amp=1.0 + 0j):
    """Raw chirp echo of one unit target whose delay is exactly ``delay_bins`` samples."""
    r0 = synth.RC_CENTRE - (nfast // 2) * synth.DR
    R = r0 + delay_bins * synth.DR
    pos = np.array([[0.0, -np.sqrt(R * R - synth.ALTITUDE ** 2), synth.ALTITUDE]])
    pts = np.array([[0.0, 0.0, 0.0]])
    raw = synth.render_chirp(pos, nfast, r0, pts, [amp])
    return raw, R


def test_rc_matches_direct_dft():
    nfast = 256
    rng = np.random.Generator(np.random.PCG64(11))
    x = rng.standard_normal((4, nfast)) + 1j * rng.standard_normal((4, nfast))
    T = 40 / synth.FS  # 40-sample chirp so it fits the short record
    y = oracle.rc.range_compress(x, synth.FS, T, synth.BANDWIDTH, window=1)
    n = np.arange(nfast)
    F = np.exp(-2j * np.pi * np.outer(n, n) / nfast)
    ref = oracle.rc.chirp_reference(nfast, synth.FS, T, synth.BANDWIDTH)
    Wn = oracle.rc.window_band(nfast, synth.FS, synth.BANDWIDTH, 1)
    Hd = np.conj(F @ ref) * Wn
    yd = (np.conj(F) @ ((F @ x.T) * Hd[:, None]) / nfast).T
    assert np.linalg.norm(y - yd) / np.linalg.norm(yd) < 1e-12


def test_rc_compressed_peak_closed_form():
    """Unit chirp at an integer delay k*: unwindowed output peaks at k* with value exactly
    L = T fs (the chirp energy) and the carrier phase -4 pi R / lambda."""
    nfast, kstar = 8192, 4100
    raw, R = _raw_single(nfast, kstar)
    y = oracle.rc.range_compress(raw, synth.FS, synth.CHIRP_T, synth.BANDWIDTH, window=0)[0]
    L = round(synth.CHIRP_T * synth.FS)
    assert int(np.argmax(np.abs(y))) == kstar
    assert abs(abs(y[kstar]) - L) < 1e-6 * L
    ph = np.angle(y[kstar] * np.exp(1j * 4 * np.pi * R / synth.WAVELENGTH))
    assert abs(ph) < 1e-6


def _rc_profile(window, up=32):
    nfast, kstar = 8192, 4096
    raw, _ = _raw_single(nfast, kstar)
    y = oracle.rc.range_compress(raw, synth.FS, synth.CHIRP_T, synth.BANDWIDTH, window=window)[0]
    # band-limited upsampling of the compressed pulse around the peak (zero-padded spectrum)
    seg = y[kstar - 64:kstar + 64]
    Y = np.fft.fftshift(np.fft.fft(seg))
    pad = np.zeros(len(seg) * up, complex)
    c = len(pad) // 2 - len(seg) // 2
    pad[c:c + len(seg)] = Y
    z = np.fft.ifft(np.fft.ifftshift(pad)) * up
    x = np.arange(len(z)) / up
    return x, np.abs(z)


def test_rc_mainlobe_and_sidelobes_match_theory_and_page():
    """Unwindowed: -3 dB width 0.886 fs/B samples and peak sidelobe near -13 dB (the page's
    figure for an unweighted matched filter).  Hamming: mainlobe 1.3-1.5x wider (the page's
    range) with sidelobes below -35 dB."""
    xg, mg = _rc_profile(0)
    w0, p0 = _cut_width_and_pslr(xg, mg)
    xh, mh = _rc_profile(1)
    w1, p1 = _cut_width_and_pslr(xh, mh)
    gold = GOLDEN["unwindowed_matched_filter_sidelobe_db"]
    assert abs(w0 / (0.886 * synth.FS / synth.BANDWIDTH) - 1) < 0.03, w0
    assert abs(p0 - gold["value"]) < gold["abs_tol_db"] + 0.3, p0
    widen = w1 / w0
    hw = GOLDEN["hamming_mainlobe_widening"]
    assert hw["min"] <= widen <= hw["max"], widen
    assert p1 < -35.0, p1


@pytest.mark.parametrize("nbar, sll", [(4, 35.0), (5, 40.0), (3, 25.0), (8, 50.0)])
def test_taylor_taper_matches_scipy(nbar, sll):
    """The oracle's Taylor taper against scipy.signal.windows.taylor (an independent
    implementation of the same classical formula), sampled at scipy's points
    x_k = (k - M/2 + 1/2) / M and normalised to 1 at the centre."""
    from scipy.signal.windows import taylor

    M = 301
    x = (np.arange(M) - M / 2 + 0.5) / M
    want = taylor(M, nbar=nbar, sll=sll, norm=True)
    got = oracle.rc.taylor_taper(x, nbar, sll)
    assert np.max(np.abs(got - want)) < 1e-12


def test_rc_taylor_sidelobes_and_mainlobe():
    """Taylor-weighted compression of a unit chirp: peak sidelobe at the design level
    (-35 dB, nbar = 4) within 1.5 dB, and a mainlobe narrower than Hamming's while still
    wider than unweighted -- the page's comparison of the two windows."""
    xg, mg = _rc_profile(0)
    w0, _ = _cut_width_and_pslr(xg, mg)
    xh, mh = _rc_profile(1)
    w1, _ = _cut_width_and_pslr(xh, mh)
    xt, mt = _rc_profile(2)
    w2, p2 = _cut_width_and_pslr(xt, mt)
    assert abs(p2 + 35.0) < 1.5, p2
    assert w0 < w2 < w1, (w0, w2, w1)


# --------------------------------------------------------------------------- page numbers

def test_page_work_model_numbers():
    for case in GOLDEN["work_model"]["cases"]:
        upd = case["na"] * case["nx"] * case["ny"]
        assert abs(upd / case["approx_updates"] - 1) < case["rel_tol"]
    s2 = synth.SCENES["std"]
    s3 = synth.SCENES["large"]
    assert s2["na"] * s2["nx"] * s2["ny"] == 4096 * 1024 * 1024
    assert s3["na"] * s3["nx"] * s3["ny"] == 16384 * 2048 * 2048
    t = GOLDEN["threads_for_1024_square"]
    assert 1024 * 1024 == t["pixels"]
    lg = GOLDEN["launch_grid_for_16x16_blocks"]
    assert [lg["image"] // lg["block"]] * 2 == lg["grid"]


def test_grid_spacing_rule_holds_for_the_configs():
    """The page's rule: pixel spacing 1/3 to 1/2 of the range resolution (0.15-0.2 m for 0.5 m)."""
    rule = GOLDEN["grid_spacing_rule"]
    lo, hi = rule["fraction_of_resolution"]
    slant_res = synth.C_LIGHT / (2 * synth.BANDWIDTH)
    assert lo * slant_res - 1e-9 <= synth.PIXEL <= hi * slant_res + 1e-9
    assert rule["spacing_m"][0] <= synth.PIXEL <= rule["spacing_m"][1]
