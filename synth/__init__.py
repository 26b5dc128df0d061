"""Seeded synthetic spotlight-SAR scenes: the inputs both the oracle and the HIP library consume.

This module is an input generator only.  It builds antenna tracks, pixel grids
and echoes (a forward model: scene -> echo) and holds none of the
backprojection arithmetic.  It imports neither ``oracle`` nor the HIP package.

Geometry and parameters follow the workload of the page
"基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR backprojection):
a straight-line spotlight pass whose beam stays on one scene centre (section
3.2), pixel spacing at 1/2-1/3 of the resolution (section 3.2; 0.2 m for a
0.5 m range resolution), 4096 pulses onto 1024 x 1024 pixels and 16384 pulses
onto 2048 x 2048 pixels as the two workload sizes (section 1.2), simulated
point targets for validation (section 4.2), and an LFM pulse that is range
compressed by FFT matched filtering with a Hamming window (section 3.1).

Conventions (x along track, y ground range, z up; scene centre at the origin):

* pixel (i, j) centre = (x0 + i*dx, y0 + j*dy, z0), x0 = -(nx/2)*dx, y0 = -(ny/2)*dy, z0 = 0
* antenna n = (v*t_n, -Y0, H) + optional smooth deviation, t_n = (n - (na-1)/2) / PRF
* range bin k is at r0 + k*dr, dr = c / (2 fs), r0 = Rc - (nr/2)*dr, Rc = |(0, Y0, H)|
* range-compressed echo of a unit scatterer: sinc(beta*(k - u)) * exp(-j 4 pi R / lambda),
  beta = B / fs, u = (R - r0) / dr

Randomness: numpy PCG64 seeded with 1000 + config number, drawn in a fixed
order: track deviation, targets, clutter (row-major), noise (pulse-major).
"""
from __future__ import annotations

import ctypes
import dataclasses
import hashlib
import os
import subprocess
import threading

import numpy as np

C_LIGHT = 299_792_458.0
WAVELENGTH = 0.03125  # carrier wavelength [m] (X band)
BANDWIDTH = 300e6  # chirp bandwidth B [Hz]
FS = 360e6  # range sampling rate [Hz]
V_PLATFORM = 100.0  # [m/s]
PRF = 500.0  # [Hz]
ALTITUDE = 5000.0  # H [m]
GROUND_RANGE = 10000.0  # Y0 [m]
PIXEL = 0.2  # grid spacing [m]
CHIRP_T = 2e-6  # pulse length [s]

DR = C_LIGHT / (2.0 * FS)
BETA = BANDWIDTH / FS
RC_CENTRE = float(np.hypot(GROUND_RANGE, ALTITUDE))

# Configurations: (name, pulses, range bins or raw samples, grid side, interpolation,
# targets, clutter, noise variance, noise location, track)
SCENES = {
    "tiny": dict(seed=1001, na=256, nr=512, nx=128, ny=128, interp="linear", n_targets=5,
                 clutter=False, noise_var=0.01, noise_on="rc", track="straight", raw=False),
    "std": dict(seed=1002, na=4096, nr=4096, nx=1024, ny=1024, interp="linear", n_targets=25,
                clutter=True, noise_var=0.0, noise_on="rc", track="straight", raw=False),
    "large": dict(seed=1003, na=16384, nr=8192, nx=2048, ny=2048, interp="linear", n_targets=64,
                  clutter=True, noise_var=0.0, noise_on="rc", track="straight", raw=False),
    "hifi": dict(seed=1004, na=4096, nr=4096, nx=1024, ny=1024, interp="sinc8", n_targets=25,
                 clutter=True, noise_var=0.0, noise_on="rc", track="perturbed", raw=False),
    "e2e": dict(seed=1005, na=4096, nr=8192, nx=1024, ny=1024, interp="linear", n_targets=25,
                clutter=False, noise_var=0.1, noise_on="raw", track="straight", raw=True),
}

CLUTTER_VAR = 0.01  # per-cell reflectivity variance: -20 dB relative to a unit target
CLUTTER_HALF_TAPS = 4  # clutter range profile truncated to +-4 bins (generator choice)
TARGET_HALF_TAPS = 256  # target range profile truncated to +-256 bins (full record when nr <= 512)
TRACK_DEV_AMP = 0.5  # [m] total amplitude of the 3-sinusoid deviation, per axis

INTERP_CODE = {"nearest": 0, "linear": 1, "sinc8": 2}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_render.so")
_lib = None
_lib_lock = threading.Lock()


def build_renderer(force: bool = False) -> str:
    """Compile the C renderer (gcc, OpenMP) next to this file and return its path."""
    src = os.path.join(_HERE, "render.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O3", "-march=x86-64-v3", "-ffp-contract=off", "-fno-math-errno", "-fPIC", "-shared", "-fopenmp", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lib_lock:
        if _lib is None:
            lib = ctypes.CDLL(build_renderer())
            dp = ctypes.POINTER(ctypes.c_double)
            i, d = ctypes.c_int, ctypes.c_double
            lib.synth_render_sinc.argtypes = [i, i, dp, d, d, d, d, i, dp, dp, i, dp, i]
            lib.synth_render_sinc_grid_straight.argtypes = [
                i, i, d, d, d, d, d, d, d, i, i, d, d, d, d, d, dp, i, dp, i]
            lib.synth_render_chirp.argtypes = [i, i, dp, d, d, d, d, d, d, i, dp, dp, dp, i]
            for f in (lib.synth_render_sinc, lib.synth_render_sinc_grid_straight, lib.synth_render_chirp):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def _dp(a: np.ndarray):
    assert a.dtype == np.float64 and a.flags.c_contiguous
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(n, 16))


@dataclasses.dataclass
class Scene:
    """One seeded synthetic workload.  Arrays are host numpy arrays."""

    name: str
    seed: int
    na: int
    nr: int
    nx: int
    ny: int
    x0: float
    y0: float
    z0: float
    dx: float
    dy: float
    r0: float
    dr: float
    wavelength: float
    interp: str
    positions: np.ndarray  # (na, 3) float64
    echo: np.ndarray | None  # (na, nr) complex64, range compressed
    raw: np.ndarray | None  # (na, nr) complex64 raw LFM samples (end-to-end config)
    targets: np.ndarray  # (K, 2) int64 pixel indices (i, j)
    fs: float = FS
    chirp_T: float = CHIRP_T
    chirp_B: float = BANDWIDTH
    window: int = 1
    dem: np.ndarray | None = None  # (ny, nx) float32 pixel heights above z0, or None (the plane z = z0)

    @property
    def updates(self) -> int:
        """Pixel-pulse updates of one image: na * nx * ny."""
        return self.na * self.nx * self.ny

    def pixel_xy(self, i, j):
        return self.x0 + np.asarray(i) * self.dx, self.y0 + np.asarray(j) * self.dy

    def sha256(self) -> dict:
        out = {"positions": hashlib.sha256(self.positions.tobytes()).hexdigest()}
        if self.echo is not None:
            out["echo"] = hashlib.sha256(self.echo.tobytes()).hexdigest()
        if self.raw is not None:
            out["raw"] = hashlib.sha256(self.raw.tobytes()).hexdigest()
        return out

    def params(self) -> dict:
        """Scalar parameters in the C-ABI's vocabulary."""
        return dict(n_pulses=self.na, n_range=self.nr, r0=self.r0, dr=self.dr, nx=self.nx,
                    ny=self.ny, x0=self.x0, y0=self.y0, z0=self.z0, dx=self.dx, dy=self.dy,
                    wavelength=self.wavelength, interp=self.interp)


def track_model(rng: np.random.Generator | None = None, perturbed: bool = False):
    """Draw the seeded deviation of a track: frequencies f and phases psi, (3 axes, 3 terms)
    each, or None for a straight track."""
    if not perturbed:
        return None
    assert rng is not None
    f = rng.uniform(0.02, 0.5, size=(3, 3))
    psi = rng.uniform(0.0, 2.0 * np.pi, size=(3, 3))
    return f, psi


def track_at(t: np.ndarray, model=None) -> np.ndarray:
    """Antenna phase centres (len(t), 3) at slow times t [s]: straight line at constant
    speed through the origin's broadside point at t = 0, plus the drawn deviation per
    axis, sum over m=1..3 of (0.5/3 m) sin(2 pi f_m t + psi_m)."""
    t = np.asarray(t, dtype=np.float64)
    pos = np.empty((t.size, 3), dtype=np.float64)
    pos[:, 0] = V_PLATFORM * t
    pos[:, 1] = -GROUND_RANGE
    pos[:, 2] = ALTITUDE
    if model is not None:
        f, psi = model
        for ax in range(3):
            dev = np.zeros(t.size)
            for m in range(3):
                dev += (TRACK_DEV_AMP / 3.0) * np.sin(2.0 * np.pi * f[ax, m] * t + psi[ax, m])
            pos[:, ax] += dev
    return pos


def pulse_times(na: int) -> np.ndarray:
    """Slow time of each pulse, centred on the aperture: (n - (na-1)/2) / PRF."""
    return (np.arange(na, dtype=np.float64) - (na - 1) / 2.0) / PRF


def track(na: int, rng: np.random.Generator | None = None, perturbed: bool = False) -> np.ndarray:
    """Antenna phase centres (na, 3) at the pulse times: straight line at constant speed,
    plus an optional seeded smooth deviation per axis, sum over m=1..3 of
    (0.5/3 m) sin(2 pi f_m t + psi_m), f_m ~ U[0.02, 0.5] Hz, psi_m ~ U[0, 2 pi)."""
    return track_at(pulse_times(na), track_model(rng, perturbed))


def terrain(nx: int, ny: int, dx: float, dy: float, rng: np.random.Generator, relief: float,
            hills: int = 8) -> np.ndarray:
    """Smooth terrain heights (ny, nx) float32 above the reference plane: a sum of
    seeded Gaussian hills and dips (centres over the scene, widths 15-40 % of its
    smaller side), shifted and scaled to a peak-to-peak `relief` centred on zero."""
    X, Y = np.meshgrid((np.arange(nx) - nx / 2) * dx, (np.arange(ny) - ny / 2) * dy)
    side = min(nx * dx, ny * dy)
    h = np.zeros((ny, nx))
    for _ in range(hills):
        cx, cy = rng.uniform(-0.5, 0.5) * nx * dx, rng.uniform(-0.5, 0.5) * ny * dy
        sig = rng.uniform(0.15, 0.4) * side
        h += rng.uniform(-1.0, 1.0) * np.exp(-((X - cx) ** 2 + (Y - cy) ** 2) / (2.0 * sig * sig))
    h = (h - h.min()) / max(h.max() - h.min(), 1e-30) * relief - 0.5 * relief
    return h.astype(np.float32)


def block_relief(dem: np.ndarray, bx: int = 64, by: int = 32) -> float:
    """Largest height range (max - min) within the bx x by blocks aligned to pixel (0, 0):
    the bound a terrain plan needs."""
    ny, nx = dem.shape
    worst = 0.0
    for j in range(0, ny, by):
        for i in range(0, nx, bx):
            b = dem[j:j + by, i:i + bx].astype(np.float64)
            worst = max(worst, float(b.max() - b.min()))
    return worst


def multipass_track(passes: int, na_per_pass: int, dh: float) -> np.ndarray:
    """Antenna positions (passes * na_per_pass, 3) of parallel straight passes at heights
    ALTITUDE + (k - (passes - 1) / 2) dh: an aperture with extent in elevation, so that
    backprojection onto a volume resolves height (a single pass does not)."""
    one = track(na_per_pass)
    out = []
    for k in range(passes):
        p = one.copy()
        p[:, 2] += (k - (passes - 1) / 2.0) * dh
        out.append(p)
    return np.concatenate(out)


def target_pixels(nx: int, ny: int, k: int, rng: np.random.Generator) -> np.ndarray:
    """K well-separated pixels: a ceil(sqrt K)^2 lattice over the central 80 % of the grid,
    K cells chosen at random, one pixel drawn from the middle half of each chosen cell."""
    g = int(np.ceil(np.sqrt(k)))
    cells = rng.permutation(g * g)[:k] if k < g * g else np.arange(g * g)
    cells = np.sort(cells)
    lo_x, hi_x = 0.1 * nx, 0.9 * nx
    lo_y, hi_y = 0.1 * ny, 0.9 * ny
    wx, wy = (hi_x - lo_x) / g, (hi_y - lo_y) / g
    out = np.empty((k, 2), dtype=np.int64)
    for t, c in enumerate(cells):
        cx, cy = c % g, c // g
        ax = lo_x + cx * wx
        ay = lo_y + cy * wy
        i = int(np.floor(rng.uniform(ax + wx / 4, ax + 3 * wx / 4)))
        j = int(np.floor(rng.uniform(ay + wy / 4, ay + 3 * wy / 4)))
        out[t] = (min(max(i, 0), nx - 1), min(max(j, 0), ny - 1))
    return out


def render_points(positions, nr, r0, dr, pts, amp, half=-1, out=None, wavelength=WAVELENGTH,
                  beta=BETA, nthreads=None):
    """Add the range-compressed echoes of point scatterers to ``out`` (na, nr) complex128."""
    lib = _load()
    positions = np.ascontiguousarray(positions, dtype=np.float64)
    na = positions.shape[0]
    if out is None:
        out = np.zeros((na, nr), dtype=np.complex128)
    pts = np.ascontiguousarray(pts, dtype=np.float64).reshape(-1, 3)
    amp = np.ascontiguousarray(np.asarray(amp, dtype=np.complex128).reshape(-1).view(np.float64))
    ov = out.view(np.float64)
    rc = lib.synth_render_sinc(na, nr, _dp(positions), r0, dr, wavelength, beta, pts.shape[0],
                               _dp(pts), _dp(amp), int(half), _dp(ov), nthreads or _threads())
    if rc != 0:
        raise ValueError("synth_render_sinc rejected its arguments")
    return out


def render_grid_straight(na, nr, r0, dr, nx, ny, x0, y0, z0, dx, dy, sigma, half, out,
                         wavelength=WAVELENGTH, beta=BETA, nthreads=None):
    """Add one scatterer per grid cell (reflectivity ``sigma`` (ny, nx)) for the straight
    track of :func:`track` (pulse spacing v/PRF must equal dx)."""
    lib = _load()
    dxa = V_PLATFORM / PRF
    if abs(dxa - dx) > 1e-12:
        raise ValueError("tabulated clutter rendering needs pulse spacing == pixel spacing")
    ax0 = V_PLATFORM * (-(na - 1) / 2.0) / PRF
    sig = np.ascontiguousarray(np.asarray(sigma, dtype=np.complex128)).view(np.float64)
    ov = out.view(np.float64)
    rc = lib.synth_render_sinc_grid_straight(na, nr, ax0, -GROUND_RANGE, ALTITUDE, r0, dr, wavelength,
                                             beta, nx, ny, x0, y0, z0, dx, dy, _dp(sig), int(half),
                                             _dp(ov), nthreads or _threads())
    if rc != 0:
        raise ValueError("synth_render_sinc_grid_straight rejected its arguments")
    return out


def render_chirp(positions, nfast, r0, pts, amp, out=None, wavelength=WAVELENGTH, fs=FS,
                 chirp_T=CHIRP_T, chirp_B=BANDWIDTH, nthreads=None):
    """Add raw LFM echoes (before range compression); sample m is at range r0 + m*c/(2 fs)."""
    lib = _load()
    positions = np.ascontiguousarray(positions, dtype=np.float64)
    na = positions.shape[0]
    if out is None:
        out = np.zeros((na, nfast), dtype=np.complex128)
    pts = np.ascontiguousarray(pts, dtype=np.float64).reshape(-1, 3)
    amp = np.ascontiguousarray(np.asarray(amp, dtype=np.complex128).reshape(-1).view(np.float64))
    t0 = 2.0 * r0 / C_LIGHT
    rc = lib.synth_render_chirp(na, nfast, _dp(positions), t0, fs, wavelength, C_LIGHT, chirp_T,
                                chirp_B / chirp_T, pts.shape[0], _dp(pts), _dp(amp),
                                _dp(out.view(np.float64)), nthreads or _threads())
    if rc != 0:
        raise ValueError("synth_render_chirp rejected its arguments")
    return out


def complex_normal(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    """CN(0, var) samples, real and imaginary parts drawn interleaved."""
    g = rng.standard_normal(tuple(shape) + (2,))
    return (g[..., 0] + 1j * g[..., 1]) * np.sqrt(var / 2.0)


def make_scene(name: str, seed: int | None = None, **over) -> Scene:
    """Build the scene ``name`` (a key of SCENES).  Keyword overrides (na, nr, nx, ny, interp,
    n_targets, clutter, noise_var, track, clutter_half) give reduced variants for tests;
    ``dem_relief`` (metres, peak to peak) puts the grid, targets and clutter on seeded
    terrain (drawn right after the targets)."""
    spec = dict(SCENES[name])
    clutter_half = over.pop("clutter_half", CLUTTER_HALF_TAPS)
    dem_relief = over.pop("dem_relief", None)
    spec.update(over)
    seed = spec["seed"] if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    na, nr, nx, ny = spec["na"], spec["nr"], spec["nx"], spec["ny"]
    dx = dy = PIXEL
    x0, y0, z0 = -(nx // 2) * dx, -(ny // 2) * dy, 0.0
    r0 = RC_CENTRE - (nr // 2) * DR
    positions = track(na, rng, perturbed=(spec["track"] == "perturbed"))
    tg = target_pixels(nx, ny, spec["n_targets"], rng)
    dem = None if dem_relief is None else terrain(nx, ny, dx, dy, rng, float(dem_relief))
    tz = np.full(len(tg), z0) if dem is None else z0 + dem[tg[:, 1], tg[:, 0]].astype(np.float64)
    pts = np.stack([x0 + tg[:, 0] * dx, y0 + tg[:, 1] * dy, tz], axis=1)
    amp = np.ones(len(tg), dtype=np.complex128)
    echo = raw = None
    if spec["raw"]:
        acc = render_chirp(positions, nr, r0, pts, amp)
        if spec["noise_var"] > 0:
            acc += complex_normal(rng, (na, nr), spec["noise_var"])
        raw = acc.astype(np.complex64)
    else:
        half = -1 if nr <= 2 * TARGET_HALF_TAPS else TARGET_HALF_TAPS
        acc = render_points(positions, nr, r0, DR, pts, amp, half=half)
        if spec["clutter"]:
            sigma = complex_normal(rng, (ny, nx), CLUTTER_VAR)
            if spec["track"] == "straight" and dem is None:
                render_grid_straight(na, nr, r0, DR, nx, ny, x0, y0, z0, dx, dy, sigma, clutter_half, acc)
            else:
                jj, ii = np.meshgrid(np.arange(ny), np.arange(nx), indexing="ij")
                cz = np.full(ii.size, z0) if dem is None else z0 + dem.ravel().astype(np.float64)
                cells = np.stack([x0 + ii.ravel() * dx, y0 + jj.ravel() * dy, cz], axis=1)
                render_points(positions, nr, r0, DR, cells, sigma.ravel(), half=clutter_half, out=acc)
        if spec["noise_var"] > 0:
            acc += complex_normal(rng, (na, nr), spec["noise_var"])
        echo = acc.astype(np.complex64)
    return Scene(name=name, seed=seed, na=na, nr=nr, nx=nx, ny=ny, x0=x0, y0=y0,
                 z0=z0, dx=dx, dy=dy, r0=r0, dr=DR, wavelength=WAVELENGTH, interp=spec["interp"],
                 positions=positions, echo=echo, raw=raw, targets=tg, dem=dem)


def resolution(scene: Scene) -> tuple[float, float]:
    """Nominal (azimuth, ground-range) resolution [m]: lambda*Rc/(2L) with L = v*na/PRF,
    and c/(2B) projected to the ground."""
    L = V_PLATFORM * scene.na / PRF
    rho_az = scene.wavelength * RC_CENTRE / (2.0 * L)
    rho_rg = C_LIGHT / (2.0 * BANDWIDTH) * RC_CENTRE / GROUND_RANGE
    return rho_az, rho_rg
