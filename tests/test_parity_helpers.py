"""Host-side checks of the parity helpers' acceptance logic (no GPU)."""
import numpy as np
import pytest

from _parity import PEAK_TIE, TIES, check_peaks, rel_l2


def _win():
    return np.array([[10, 20], [10, 21], [10, 22], [10, 23]])


def test_peak_on_an_oracle_plateau_is_accepted_and_reported():
    w = _win()
    want = np.array([1.0, 218.92128, 218.92176, 218.92223])  # nearest-interpolation plateau (relative gap 2e-6)
    got = want.copy()
    got[2] *= 1 + 1e-5  # the GPU picks another pixel of the plateau
    n = len(TIES)
    check_peaks(lambda p: got, lambda p: want, [w], "nearest", "plateau")
    assert len(TIES) == n + 1 and TIES[-1]["accepted"] and TIES[-1]["gpu"] == [10, 22]
    assert TIES[-1]["gap"] == pytest.approx(2.15e-6, rel=0.02)


def test_tie_needs_nearest():
    """Linear and sinc8 are continuous in the range: a moved peak fails even within the GPU error."""
    w = _win()
    want = np.array([1.0, 218.92128, 218.92176, 218.92223])
    got = want.copy()
    got[2] *= 1 + 1e-5
    for interp in ("linear", "sinc8"):
        with pytest.raises(AssertionError, match="peak moved"):
            check_peaks(lambda p: got, lambda p: want, [w], interp)
    assert not TIES[-1]["accepted"]


def test_tie_beyond_the_window_error_is_rejected():
    """A gap (here 5.6e-5, under PEAK_TIE) larger than the GPU's largest error in the window
    (3e-5: both pixels moved towards each other) is not a tie of the definition."""
    w = _win()
    want = np.array([1.0, 200.0, 218.91, 218.92223])
    got = want.copy()
    got[2] *= 1 + 3e-5
    got[3] *= 1 - 3e-5
    assert np.argmax(np.abs(got)) == 2
    with pytest.raises(AssertionError, match="peak moved"):
        check_peaks(lambda p: got, lambda p: want, [w], "nearest")
    assert not TIES[-1]["accepted"] and TIES[-1]["gap"] < PEAK_TIE


def test_peak_moved_off_the_plateau_is_rejected():
    w = _win()
    want = np.array([1.0, 200.0, 218.9, 210.0])
    got = want.copy()
    got[3] = 219.5
    with pytest.raises(AssertionError, match="peak moved"):
        check_peaks(lambda p: got, lambda p: want, [w], "nearest")


def test_peak_magnitude_bound():
    w = _win()
    want = np.array([1.0, 2.0, 100.0, 3.0])
    assert check_peaks(lambda p: want * 1.005, lambda p: want, [w], "linear") == pytest.approx(0.0433, abs=1e-3)
    with pytest.raises(AssertionError, match="dB"):
        check_peaks(lambda p: want * 1.01, lambda p: want, [w], "linear")  # 0.086 dB


def test_tie_band_and_rel_l2():
    assert 0 < PEAK_TIE <= 1e-3
    a = np.ones(100, complex)
    assert rel_l2(a * (1 + 1e-3), a) == pytest.approx(1e-3)
