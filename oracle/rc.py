"""fp64 range compression by FFT matched filtering -- oracle, TEST INFRASTRUCTURE ONLY.

Follows section 3.1 of the page "基于GPU的SAR后向投影成像优化与CUDA加速实践"
(GPU-based SAR backprojection imaging and CUDA acceleration): per pulse, FFT
along range, multiply by the matched filter's frequency response and a Hamming
or Taylor window, inverse FFT; all pulses are independent (a batch of 1-D
transforms).

Definitions (the page leaves them open; the readings are):

* chirp p(t) = exp(j pi K t^2) for -T/2 <= t < T/2, K = B / T (up-chirp)
* reference ref[m mod N] = p(m / fs) for m = -L/2 .. L/2 - 1, L = round(T fs), centred at t = 0
* window W[m] = w(f_m / B) for |f_m| <= B/2, else 0, f_m = fftfreq(N, 1/fs)[m], with
  - Hamming: w(x) = 0.54 + 0.46 cos(2 pi x)
  - Taylor (the page names it as the alternative with less mainlobe widening, without
    parameters; the reading is the standard Taylor taper with nbar = 4 nearly equal
    sidelobes at SLL = 35 dB below the peak, both adjustable):
    w(x) = 1 + 2 sum_{m=1}^{nbar-1} F_m cos(2 pi m x), scaled so that w(0) = 1, where
    A = acosh(10^(SLL/20)) / pi, sigma^2 = nbar^2 / (A^2 + (nbar - 1/2)^2) and
    F_m = (-1)^(m+1) / 2 * prod_{n=1}^{nbar-1} (1 - m^2 / (sigma^2 (A^2 + (n - 1/2)^2)))
                          / prod_{n=1, n != m}^{nbar-1} (1 - m^2 / n^2)
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


def taylor_taper(x: np.ndarray, nbar: int = 4, sll_db: float = 35.0) -> np.ndarray:
    """Taylor taper at normalised positions x in [-1/2, 1/2] (1 at x = 0)."""
    A = np.arccosh(10.0 ** (sll_db / 20.0)) / np.pi
    sigma2 = nbar * nbar / (A * A + (nbar - 0.5) ** 2)
    w = np.ones_like(np.asarray(x, dtype=np.float64))
    centre = 1.0
    for m in range(1, nbar):
        num = 1.0
        den = 1.0
        for n in range(1, nbar):
            num *= 1.0 - m * m / (sigma2 * (A * A + (n - 0.5) ** 2))
            if n != m:
                den *= 1.0 - m * m / (n * n)
        F = (-1) ** (m + 1) / 2.0 * num / den
        w = w + 2.0 * F * np.cos(2.0 * np.pi * m * np.asarray(x, dtype=np.float64))
        centre += 2.0 * F
    return w / centre


def window_band(n_fast: int, fs: float, chirp_B: float, window: int, nbar: int = 4,
                sll_db: float = 35.0) -> np.ndarray:
    """Frequency-domain weights over |f| <= B/2: 1 (window=0), Hamming (1) or Taylor (2)."""
    if window == 0:
        return np.ones(n_fast)
    f = np.fft.fftfreq(n_fast, 1.0 / fs)
    x = f / chirp_B
    w = 0.54 + 0.46 * np.cos(2.0 * np.pi * x) if window == 1 else taylor_taper(x, nbar, sll_db)
    return np.where(np.abs(f) <= chirp_B / 2.0, w, 0.0)


def filter_response(n_fast: int, fs: float, chirp_T: float, chirp_B: float, window: int, nbar: int = 4,
                    sll_db: float = 35.0) -> np.ndarray:
    """conj(FFT(ref)) * W: the per-bin multiplier of the matched filter."""
    return np.conj(np.fft.fft(chirp_reference(n_fast, fs, chirp_T, chirp_B))) * window_band(
        n_fast, fs, chirp_B, window, nbar, sll_db)


def range_compress(raw: np.ndarray, fs: float, chirp_T: float, chirp_B: float, window: int = 1, nbar: int = 4,
                   sll_db: float = 35.0) -> np.ndarray:
    """Range-compress raw (n_pulses, n_fast) samples; complex128 result of the same shape."""
    x = np.asarray(raw, dtype=np.complex128)
    H = filter_response(x.shape[-1], fs, chirp_T, chirp_B, window, nbar, sll_db)
    return np.fft.ifft(np.fft.fft(x, axis=-1) * H, axis=-1)
