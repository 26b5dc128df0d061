"""Antenna positions interpolated from navigation samples -- oracle, TEST INFRASTRUCTURE ONLY.

The page "基于GPU的SAR后向投影成像优化与CUDA加速实践" (GPU-based SAR backprojection
imaging and CUDA acceleration), section 3.3, notes that in practice the radar position
of each pulse may have to be interpolated from the flight track; it names no method.

Reading: cubic (4-point) Lagrange interpolation, per axis, through the navigation
samples around each pulse time, in double precision:

* the samples' times t_0 < t_1 < ... < t_{M-1} are strictly increasing (M >= 4);
* for a pulse time t with t_0 <= t <= t_{M-1}, i is the interval with t_i <= t < t_{i+1}
  (i = M-2 when t = t_{M-1}); the stencil is the 4 samples j0 .. j0+3 with
  j0 = min(max(i - 1, 0), M - 4), i.e. two on each side where the record allows;
* p(t) = sum_k p_{j0+k} * prod_{m != k} (t - t_{j0+m}) / (t_{j0+k} - t_{j0+m});
* a time outside [t_0, t_{M-1}] (or not finite) has no position: NaN.

Linear interpolation would be the plainer reading, but it misplaces a smoothly
perturbed track (0.5 m deviations at up to 0.5 Hz, samples at 100 Hz) by ~2e-5 m,
i.e. 8e-3 rad of phase at a 3 cm wavelength; the cubic's error there is ~4e-9 m.
"""
from __future__ import annotations

import numpy as np


def stencil_start(nav_t: np.ndarray, t: float) -> int:
    """First of the 4 samples used for time t (t inside the samples' span)."""
    M = len(nav_t)
    i = int(np.searchsorted(nav_t, t, side="right")) - 1
    i = min(max(i, 0), M - 2)
    return min(max(i - 1, 0), M - 4)


def interpolate_track(nav_t, nav_xyz, t) -> np.ndarray:
    """Positions (len(t), 3) at times t from samples nav_xyz (M, 3) at nav_t (M,)."""
    nav_t = np.asarray(nav_t, dtype=np.float64)
    nav_xyz = np.asarray(nav_xyz, dtype=np.float64)
    t = np.atleast_1d(np.asarray(t, dtype=np.float64))
    if nav_t.ndim != 1 or len(nav_t) < 4 or nav_xyz.shape != (len(nav_t), 3):
        raise ValueError("need M >= 4 samples: nav_t (M,), nav_xyz (M, 3)")
    if not np.all(np.diff(nav_t) > 0):
        raise ValueError("navigation times must increase strictly")
    out = np.full((t.size, 3), np.nan)
    for n, tn in enumerate(t):
        if not (np.isfinite(tn) and nav_t[0] <= tn <= nav_t[-1]):
            continue
        j0 = stencil_start(nav_t, tn)
        ts = nav_t[j0:j0 + 4]
        acc = np.zeros(3)
        for k in range(4):
            w = 1.0
            for m in range(4):
                if m != k:
                    w *= (tn - ts[m]) / (ts[k] - ts[m])
            acc += w * nav_xyz[j0 + k]
        out[n] = acc
    return out
