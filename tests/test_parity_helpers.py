"""Host-side checks of the parity helpers' acceptance logic (no GPU)."""
import numpy as np
import pytest

from _parity import PEAK_TIE, check_peaks, rel_l2


def _win():
    return np.array([[10, 20], [10, 21], [10, 22], [10, 23]])


def test_peak_on_an_oracle_plateau_is_accepted():
    w = _win()
    want = np.array([1.0, 218.92128, 218.92176, 218.92223])  # nearest-interpolation plateau (relative gap 2e-6)
    got = want.copy()
    got[2] *= 1 + 1e-5  # the GPU picks another pixel of the plateau
    check_peaks(lambda p: got, lambda p: want, [w])


def test_peak_moved_off_the_plateau_is_rejected():
    w = _win()
    want = np.array([1.0, 200.0, 218.9, 210.0])
    got = want.copy()
    got[3] = 219.5
    with pytest.raises(AssertionError, match="peak moved"):
        check_peaks(lambda p: got, lambda p: want, [w])


def test_peak_magnitude_bound():
    w = _win()
    want = np.array([1.0, 2.0, 100.0, 3.0])
    check_peaks(lambda p: want * 1.005, lambda p: want, [w])  # 0.043 dB
    with pytest.raises(AssertionError, match="dB"):
        check_peaks(lambda p: want * 1.01, lambda p: want, [w])  # 0.086 dB


def test_tie_band_and_rel_l2():
    assert 0 < PEAK_TIE <= 1e-3
    a = np.ones(100, complex)
    assert rel_l2(a * (1 + 1e-3), a) == pytest.approx(1e-3)
