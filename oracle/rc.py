"""fp64 range compression by FFT matched filtering -- oracle, TEST INFRASTRUCTURE ONLY.

Follows section 3.1 of the page "基于GPU的SAR后向投影成像优化与CUDA加速实践"
(GPU-based SAR backprojection imaging and CUDA acceleration): per pulse, FFT
along range, multiply by the matched filter's frequency response and a Hamming
window, inverse FFT; all pulses are independent (a batch of 1-D transforms).

Definitions (the page leaves them open; the readings are):

* chirp p(t) = exp(j pi K t^2) for -T/2 <= t < T/2, K = B / T (up-chirp)
* reference ref[m mod N] = p(m / fs) for m = -L/2 .. L/2 - 1, L = round(T fs), centred at t = 0
* window W[m] = 0.54 + 0.46 cos(2 pi f_m / B) for |f_m| <= B/2, else 0, f_m = fftfreq(N, 1/fs)[m]
* y_n = IFFT_N( FFT_N(x_n) * conj(FFT_N(ref)) * W ), numpy normalisation (1/N on the inverse)
* output bin k lies at range r0 + k c / (2 fs), the range of raw sample k

numpy's pocketfft serves as the FFT step (a library primitive); the pins in the
tests compare it with a direct O(N^2) DFT and with closed forms.
"""
from __future__ import annotations

import numpy as np


def chirp_reference(n_fast: int, fs: float, chirp_T: float, chirp_B: float) -> np.ndarray:
    L = int(round(chirp_T * fs))
    if L <= 0 or L > n_fast:
        raise ValueError("chirp longer than the record")
    K = chirp_B / chirp_T
    m = np.arange(-(L // 2), L - L // 2)
    t = m / fs
    ref = np.zeros(n_fast, dtype=np.complex128)
    ref[m % n_fast] = np.exp(1j * np.pi * K * t * t)
    return ref


def window_band(n_fast: int, fs: float, chirp_B: float, window: int) -> np.ndarray:
    """Frequency-domain weights: 1 (window=0) or Hamming over |f| <= B/2 (window=1)."""
    if window == 0:
        return np.ones(n_fast)
    f = np.fft.fftfreq(n_fast, 1.0 / fs)
    return np.where(np.abs(f) <= chirp_B / 2.0, 0.54 + 0.46 * np.cos(2.0 * np.pi * f / chirp_B), 0.0)


def filter_response(n_fast: int, fs: float, chirp_T: float, chirp_B: float, window: int) -> np.ndarray:
    """conj(FFT(ref)) * W: the per-bin multiplier of the matched filter."""
    return np.conj(np.fft.fft(chirp_reference(n_fast, fs, chirp_T, chirp_B))) * window_band(
        n_fast, fs, chirp_B, window)


def range_compress(raw: np.ndarray, fs: float, chirp_T: float, chirp_B: float, window: int = 1) -> np.ndarray:
    """Range-compress raw (n_pulses, n_fast) samples; complex128 result of the same shape."""
    x = np.asarray(raw, dtype=np.complex128)
    H = filter_response(x.shape[-1], fs, chirp_T, chirp_B, window)
    return np.fft.ifft(np.fft.fft(x, axis=-1) * H, axis=-1)
