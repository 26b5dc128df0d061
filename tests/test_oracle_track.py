"""Pins of the oracle's track interpolation (cubic 4-point Lagrange through the
navigation samples around each pulse time; reading of the page's remark, section 3.3,
that pulse positions may have to be interpolated from the track)."""
import numpy as np
import pytest

import oracle
import synth


def _nav(M=40, seed=3, uniform=False):
    rng = np.random.Generator(np.random.PCG64(seed))
    if uniform:
        t = np.linspace(-2.0, 2.0, M)
    else:
        t = np.sort(rng.uniform(-2.0, 2.0, M))
        t[0], t[-1] = -2.0, 2.0
    return t, rng


def test_cubic_trajectories_are_reproduced_exactly():
    """A cubic polynomial per axis lies in the interpolant's space: exact to rounding."""
    t, rng = _nav()
    c = rng.standard_normal((4, 3)) * np.array([1e3, 10.0, 5.0])
    f = lambda tt: np.stack([np.polyval(c[:, a], tt) for a in range(3)], 1)
    q = np.linspace(-2.0, 2.0, 777)
    got = oracle.track.interpolate_track(t, f(t), q)
    assert np.max(np.abs(got - f(q))) < 1e-9


def test_nodes_and_library_lagrange():
    """At a sample time it returns that sample; between samples it equals scipy's
    Lagrange polynomial through the same 4 stencil samples."""
    from scipy.interpolate import lagrange

    t, rng = _nav(M=25, seed=9)
    p = rng.standard_normal((25, 3))
    got = oracle.track.interpolate_track(t, p, t)
    assert np.max(np.abs(got - p)) < 1e-12
    for tn in rng.uniform(-2.0, 2.0, 50):
        j0 = oracle.track.stencil_start(t, tn)
        for a in range(3):
            want = lagrange(t[j0:j0 + 4] - tn, p[j0:j0 + 4, a])(0.0)
            assert abs(oracle.track.interpolate_track(t, p, [tn])[0, a] - want) < 1e-9


def test_stencil_is_centred_and_clamped():
    t = np.arange(10.0)
    assert oracle.track.stencil_start(t, 4.5) == 3   # samples 3,4,5,6 around interval [4,5)
    assert oracle.track.stencil_start(t, 0.2) == 0   # clamped at the start
    assert oracle.track.stencil_start(t, 8.7) == 6   # clamped at the end
    assert oracle.track.stencil_start(t, 9.0) == 6   # last sample time


def test_fourth_order_convergence_on_the_perturbed_track():
    """The hi-fi scene's smooth deviation (0.5 m, up to 0.5 Hz): halving the sample
    interval divides the error by ~16, and at 100 Hz it is below 1e-8 m."""
    model = synth.track_model(np.random.Generator(np.random.PCG64(1004)), perturbed=True)
    q = synth.pulse_times(4096)
    exact = synth.track_at(q, model)
    errs = []
    for rate in (25.0, 50.0, 100.0):
        tn = np.arange(q[0] - 0.05, q[-1] + 0.05 + 1e-9, 1.0 / rate)
        got = oracle.track.interpolate_track(tn, synth.track_at(tn, model), q)
        errs.append(np.max(np.abs(got - exact)))
    assert 10 < errs[0] / errs[1] < 22 and 10 < errs[1] / errs[2] < 22, errs
    assert errs[2] < 1e-8, errs


def test_outside_the_samples_is_nan_and_bad_input_raises():
    t, _ = _nav(M=8)
    p = np.zeros((8, 3))
    got = oracle.track.interpolate_track(t, p, [-2.5, 2.5, np.nan, 0.0])
    assert np.isnan(got[:3]).all() and np.isfinite(got[3]).all()
    with pytest.raises(ValueError):
        oracle.track.interpolate_track(t[::-1], p, [0.0])
    with pytest.raises(ValueError):
        oracle.track.interpolate_track(t[:3], p[:3], [0.0])
