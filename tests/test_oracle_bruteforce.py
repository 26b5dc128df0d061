"""Brute-force pin of the backprojection oracle: the definition written out again in
40-digit mpmath arithmetic, independently of the oracle's C code, on tiny random
cases with every interpolator (time-domain backprojection, sections 1.1 and 2.2 of
the page: per pixel and pulse, range, bin position, interpolated sample, phase
term exp(+j 4 pi R / lambda), coherent sum).

The geometries put some pixel-pulse pairs within the interpolators' reach of both
ends of the record, so the zero extension outside it is exercised too.

Tolerances come from the oracle's own fp64 arithmetic: its phase 4 pi R / lambda is
rounded to ~2^-53 of its size (plus the rounding of R and u, of the same order), so
each term is accurate to a few 2^-53 * 4 pi R / lambda: the bound used is four of
those, 3.6e-11 at 200 m and 2.0e-9 at 11 km.
"""
import mpmath as mp
import numpy as np
import pytest

import oracle

mp.mp.dps = 40
LAM = 0.03125


def _h(t):
    """Windowed sinc of the 8-tap option: sinc(t) (0.54 + 0.46 cos(pi t / 4)), |t| < 4."""
    if abs(t) >= 4:
        return mp.mpf(0)
    s = mp.mpf(1) if t == 0 else mp.sin(mp.pi * t) / (mp.pi * t)
    return s * (mp.mpf("0.54") + mp.mpf("0.46") * mp.cos(mp.pi * t / 4))


def _brute(pos, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy, interp, dem=None):
    na, nr = echo.shape
    S = [[mp.mpc(complex(echo[n, k])) for k in range(nr)] for n in range(na)]

    def s(n, k):
        return S[n][k] if 0 <= k < nr else mp.mpc(0)

    out = np.zeros((ny, nx), dtype=np.complex128)
    r0, dr = mp.mpf(r0), mp.mpf(dr)
    for j in range(ny):
        for i in range(nx):
            x = mp.mpf(x0) + i * mp.mpf(dx)
            y = mp.mpf(y0) + j * mp.mpf(dy)
            z = mp.mpf(z0) + (0 if dem is None else mp.mpf(float(dem[j, i])))
            acc = mp.mpc(0)
            for n in range(na):
                ax, ay, az = (mp.mpf(float(c)) for c in pos[n])
                R = mp.sqrt((x - ax) ** 2 + (y - ay) ** 2 + (z - az) ** 2)
                u = (R - r0) / dr
                if interp == "nearest":
                    v = s(n, int(mp.floor(u + mp.mpf("0.5"))))
                elif interp == "linear":
                    k = int(mp.floor(u))
                    f = u - k
                    v = (1 - f) * s(n, k) + f * s(n, k + 1)
                else:
                    k = int(mp.floor(u))
                    v = mp.fsum(s(n, k + m) * _h(u - k - m) for m in range(-3, 5))
                acc += v * mp.expjpi(4 * R / LAM)
            out[j, i] = complex(acc)
    return out


def _case(R_centre, seed):
    """5 pulses, 32-bin record, 3 x 4 pixels spread so that bin positions run from
    below the record's start to past its end."""
    rng = np.random.Generator(np.random.PCG64(seed))
    na, nr, nx, ny = 5, 32, 3, 4
    dr = 0.41637
    H = 0.6 * R_centre
    G = 0.8 * R_centre
    pos = np.stack([rng.uniform(-3, 3, na), -G + rng.uniform(-0.5, 0.5, na), H + rng.uniform(-0.5, 0.5, na)], 1)
    r0 = R_centre - 16 * dr
    dx, dy = 0.37, 6.25  # rows at +-3.1 and +-9.4 m of ground range: bins ~ -2 .. 34
    x0, y0 = -dx, -1.5 * dy
    echo = (rng.standard_normal((na, nr)) + 1j * rng.standard_normal((na, nr))).astype(np.complex64)
    return pos, echo, r0, dr, nx, ny, x0, y0, 0.0, dx, dy


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
@pytest.mark.parametrize("R_centre", [200.0, 11180.0])
def test_oracle_matches_40_digit_definition(interp, R_centre):
    tol = 4 * 2.0 ** -53 * 4 * np.pi * R_centre / LAM
    pos, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy = _case(R_centre, 11 if interp == "linear" else 12)
    # the case reaches both ends of the record (zero extension exercised)
    x = x0 + np.arange(nx) * dx
    y = y0 + np.arange(ny) * dy
    X, Y = np.meshgrid(x, y)
    u = (np.sqrt((X[..., None] - pos[:, 0]) ** 2 + (Y[..., None] - pos[:, 1]) ** 2 + pos[:, 2] ** 2) - r0) / dr
    nr = echo.shape[1]
    assert np.any((u >= -4) & (u < 0)) and np.any((u > nr - 1) & (u < nr + 3))
    want = _brute(pos, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy, interp)
    got = oracle.backproject(pos, echo, r0=r0, dr=dr, nx=nx, ny=ny, x0=x0, y0=y0, z0=z0, dx=dx, dy=dy,
                             wavelength=LAM, interp=interp)
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err <= tol, err


@pytest.mark.parametrize("interp", ["nearest", "linear", "sinc8"])
def test_oracle_terrain_matches_40_digit_definition(interp):
    """The same with a random terrain height per pixel (float32, +-5 m) at 11 km."""
    pos, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy = _case(11180.0, 13)
    dem = np.random.Generator(np.random.PCG64(14)).uniform(-5, 5, (ny, nx)).astype(np.float32)
    want = _brute(pos, echo, r0, dr, nx, ny, x0, y0, z0, dx, dy, interp, dem=dem)
    got = oracle.backproject(pos, echo, r0=r0, dr=dr, nx=nx, ny=ny, x0=x0, y0=y0, z0=z0, dx=dx, dy=dy,
                             wavelength=LAM, interp=interp, dem=dem)
    err = np.linalg.norm(got - want) / np.linalg.norm(want)
    assert err <= 4 * 2.0 ** -53 * 4 * np.pi * 11180.0 / LAM, err
