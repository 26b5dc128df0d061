"""CPU oracle for time-domain SAR backprojection and matched-filter range compression.

TEST INFRASTRUCTURE ONLY: tests/, ``__graft_entry__.smoke()`` and bench.py's
``cpu_baseline`` leg are the only code allowed to import this package.  The HIP
library and its binding never import, link or call it, and share no code with it.

* :func:`backproject` / :func:`backproject_pixels` / :func:`nearest_index` wrap
  ``bp_oracle.c`` (plain IEEE double precision, gcc ``-O2 -ffp-contract=off``,
  OpenMP over image rows), the definition stated in that file's header.
* :mod:`oracle.rc` holds the fp64 FFT matched filter (numpy).
* :mod:`oracle.track` interpolates antenna positions from navigation samples (numpy).

Pins: every function here is checked in ``tests/test_oracle_pins.py`` against
closed forms, textbook impulse-response figures, special cases and invariants
(see that file).  The sinc8 kernel *shape* is a reading of the page (which names
sinc interpolation without defining it) and is pinned only by its interpolating,
symmetry and continuity properties and the closed-form peak.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from . import rc  # noqa: F401  (re-export)
from . import track  # noqa: F401  (re-export)

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "_bp_oracle.so")
_lib = None
_lock = threading.Lock()

INTERP = {"nearest": 0, "linear": 1, "sinc8": 2}


def build(force: bool = False) -> str:
    """Compile ``bp_oracle.c`` with gcc (no FMA contraction, no fast-math)."""
    src = os.path.join(_HERE, "bp_oracle.c")
    if force or not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(src):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-fPIC", "-shared", "-o", tmp, src, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is None:
            lib = ctypes.CDLL(build())
            dp = ctypes.POINTER(ctypes.c_double)
            lp = ctypes.POINTER(ctypes.c_int64)
            i, d = ctypes.c_int, ctypes.c_double
            lib.oracle_backproject_rows.argtypes = [i, i, dp, dp, d, d, i, i, d, d, d, d, d, d, i, i, i, dp, i]
            lib.oracle_backproject_pixels.argtypes = [i, i, dp, dp, d, d, d, d, d, d, d, d, i, i, lp, dp, i]
            lib.oracle_nearest_index.argtypes = [dp, d, d, d, d, d, d, d, i, lp, lp]
            fp_ = ctypes.POINTER(ctypes.c_float)
            lib.oracle_nearest_index_dem.argtypes = [dp, d, d, d, d, d, d, d, i, i, fp_, i, lp, lp]
            fp = ctypes.POINTER(ctypes.c_float)
            lib.oracle_backproject_rows_dem.argtypes = [i, i, dp, dp, d, d, i, i, d, d, d, d, d, fp, d, i, i, i,
                                                        dp, i]
            lib.oracle_backproject_pixels_dem.argtypes = [i, i, dp, dp, d, d, d, d, d, d, d, i, fp, d, i, i, lp,
                                                          dp, i]
            lib.oracle_sinc8_weight.argtypes = [d]
            lib.oracle_sinc8_weight.restype = d
            for f in (lib.oracle_backproject_rows, lib.oracle_backproject_pixels, lib.oracle_nearest_index,
                      lib.oracle_nearest_index_dem,
                      lib.oracle_backproject_rows_dem, lib.oracle_backproject_pixels_dem):
                f.restype = ctypes.c_int
            _lib = lib
    return _lib


def threads() -> int:
    """Host threads the oracle uses: the CPUs this process may run on."""
    return max(1, len(os.sched_getaffinity(0)))


def _f64(a):
    a = np.ascontiguousarray(a, dtype=np.float64)
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _echo128(echo):
    e = np.ascontiguousarray(echo, dtype=np.complex128)  # complex64 -> complex128 is exact
    return e, e.view(np.float64).ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _interp(interp):
    return INTERP[interp] if isinstance(interp, str) else int(interp)


def _dem32(dem, ny, nx):
    d = np.ascontiguousarray(dem, dtype=np.float32)
    if d.shape != (ny, nx):
        raise ValueError("dem must be (ny, nx)")
    return d, d.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def backproject(positions, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy, wavelength, interp,
                rows=None, nthreads=None, dem=None) -> np.ndarray:
    """Image (ny, nx) complex128, or rows [j0, j1) of it when ``rows=(j0, j1)``.  With
    ``dem`` (float32 (ny, nx)), pixel (i, j) lies at height z0 + dem[j, i]."""
    lib = _load()
    pos, pp = _f64(positions)
    e, ep = _echo128(echo)
    na, nr = e.shape
    assert pos.shape == (na, 3)
    j0, j1 = (0, ny) if rows is None else rows
    out = np.zeros((j1 - j0, nx), dtype=np.complex128)
    op = out.view(np.float64).ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    if dem is None:
        rc_ = lib.oracle_backproject_rows(na, nr, pp, ep, r0, dr, nx, ny, x0, y0, z0, dx, dy, wavelength,
                                          _interp(interp), j0, j1, op, nthreads or threads())
    else:
        d, dp_ = _dem32(dem, ny, nx)
        rc_ = lib.oracle_backproject_rows_dem(na, nr, pp, ep, r0, dr, nx, ny, x0, y0, z0, dx, dy, dp_, wavelength,
                                              _interp(interp), j0, j1, op, nthreads or threads())
    if rc_ != 0:
        raise ValueError("oracle_backproject_rows rejected its arguments")
    return out


def backproject_pixels(positions, echo, r0, dr, x0, y0, z0, dx, dy, wavelength, interp, ij,
                       nthreads=None, dem=None) -> np.ndarray:
    """Values at grid pixels ``ij`` ((P, 2) int: i along x, j along y), complex128 (P,).
    With ``dem`` (float32 (ny, nx)), pixel (i, j) lies at height z0 + dem[j, i]."""
    lib = _load()
    pos, pp = _f64(positions)
    e, ep = _echo128(echo)
    na, nr = e.shape
    ij = np.ascontiguousarray(ij, dtype=np.int64).reshape(-1, 2)
    out = np.zeros(ij.shape[0], dtype=np.complex128)
    ijp = ij.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    op = out.view(np.float64).ctypes.data_as(ctypes.POINTER(ctypes.c_double))
    if dem is None:
        rc_ = lib.oracle_backproject_pixels(na, nr, pp, ep, r0, dr, x0, y0, z0, dx, dy, wavelength,
                                            _interp(interp), ij.shape[0], ijp, op, nthreads or threads())
    else:
        d = np.ascontiguousarray(dem, dtype=np.float32)
        if ij.size and (ij[:, 0].max() >= d.shape[1] or ij[:, 1].max() >= d.shape[0] or ij.min() < 0):
            raise ValueError("pixel outside the dem")
        rc_ = lib.oracle_backproject_pixels_dem(na, nr, pp, ep, r0, dr, x0, y0, z0, dx, dy, d.shape[1],
                                                d.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), wavelength,
                                                _interp(interp), ij.shape[0], ijp, op, nthreads or threads())
    if rc_ != 0:
        raise ValueError("oracle_backproject_pixels rejected its arguments")
    return out


def nearest_index(antenna, r0, dr, x0, y0, z0, dx, dy, ij, dem=None) -> np.ndarray:
    """floor(u + 1/2) for one antenna position at grid pixels ``ij``: int64 (P,).  With ``dem``
    (float32 (ny, nx)), pixel (i, j) lies at height z0 + dem[j, i]."""
    lib = _load()
    a, ap = _f64(np.asarray(antenna).reshape(3))
    ij = np.ascontiguousarray(ij, dtype=np.int64).reshape(-1, 2)
    out = np.zeros(ij.shape[0], dtype=np.int64)
    ijp = ij.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    op = out.ctypes.data_as(ctypes.POINTER(ctypes.c_int64))
    if dem is None:
        rc_ = lib.oracle_nearest_index(ap, r0, dr, x0, y0, z0, dx, dy, ij.shape[0], ijp, op)
    else:
        d = np.ascontiguousarray(dem, dtype=np.float32)
        ny, nx = d.shape
        rc_ = lib.oracle_nearest_index_dem(ap, r0, dr, x0, y0, z0, dx, dy, nx, ny,
                                           d.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), ij.shape[0], ijp, op)
    if rc_ != 0:
        raise ValueError("oracle_nearest_index rejected its arguments")
    return out


def sinc8_weight(t: float) -> float:
    """The oracle's 8-tap kernel h(t)."""
    return float(_load().oracle_sinc8_weight(float(t)))


def backproject_volume(positions, echo, r0, dr, nx, ny, nz, x0, y0, z0, dx, dy, dz, wavelength, interp,
                       nthreads=None) -> np.ndarray:
    """Voxel image (nz, ny, nx) complex128: voxel (i, j, l) at (x0 + i dx, y0 + j dy, z0 + l dz)
    -- the plane definition at each layer height (3-D backprojection, the page's section 5)."""
    return np.stack([backproject(positions, echo, r0, dr, nx, ny, x0, y0, z0 + float(l) * dz, dx, dy, wavelength,
                                 interp, nthreads=nthreads) for l in range(nz)])


def scene_backproject(scene, echo=None, rows=None, nthreads=None) -> np.ndarray:
    """:func:`backproject` with the geometry of a ``synth.Scene`` (and its dem, if any)."""
    return backproject(scene.positions, scene.echo if echo is None else echo, scene.r0, scene.dr,
                       scene.nx, scene.ny, scene.x0, scene.y0, scene.z0, scene.dx, scene.dy,
                       scene.wavelength, scene.interp, rows=rows, nthreads=nthreads,
                       dem=getattr(scene, "dem", None))


def scene_pixels(scene, ij, echo=None, nthreads=None) -> np.ndarray:
    """:func:`backproject_pixels` with the geometry of a ``synth.Scene`` (and its dem, if any)."""
    return backproject_pixels(scene.positions, scene.echo if echo is None else echo, scene.r0, scene.dr,
                              scene.x0, scene.y0, scene.z0, scene.dx, scene.dy, scene.wavelength,
                              scene.interp, ij, nthreads=nthreads, dem=getattr(scene, "dem", None))
