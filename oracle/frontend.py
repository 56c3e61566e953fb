"""Oracle front end: sizes, window, mel filter bank, DFT magnitude, log-mel.

TEST INFRASTRUCTURE (see the package docstring). float64 throughout.
Source: egemma2_audio.rs (cortiq-engine 0.8.49), module documentation
steps 1-2, constants, ``num_frames``, ``num_tokens``, ``linspace``,
``mel_filter_bank``, ``MelFrontend::new`` and ``MelFrontend::log_mel``.
"""
from __future__ import annotations

import numpy as np

SAMPLE_RATE = 16000
MAX_SAMPLES = 480000      # 30 s cut
FRAME = 320               # 20 ms window
HOP = 160                 # 10 ms hop
N_FFT = 512
N_MELS = 128
MEL_FLOOR = 1e-3


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def num_frames(n: int) -> int:
    """Frames of an n-sample clip: 0 if n <= 160, else ceil((n-160)/160),
    after the 30 s cut (egemma2_audio.rs, ``num_frames``)."""
    n = min(int(n), MAX_SAMPLES)
    return 0 if n <= HOP else _ceil_div(n - HOP, HOP)


def num_tokens(n: int) -> int:
    """Soft tokens: the frame count halved (rounding up) twice, one halving
    per stride-2 convolution (egemma2_audio.rs, ``num_tokens``)."""
    return _ceil_div(_ceil_div(num_frames(n), 2), 2)


def hann_window() -> np.ndarray:
    """Periodic Hann of length 320: 0.5 - 0.5 cos(2 pi n / 320)
    (egemma2_audio.rs, ``MelFrontend::new``)."""
    n = np.arange(FRAME, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * n / FRAME)


def linspace(a: float, b: float, n: int) -> np.ndarray:
    """a + i*step with the last point set to b exactly (egemma2_audio.rs,
    ``linspace``)."""
    step = (b - a) / (n - 1)
    v = a + np.arange(n, dtype=np.float64) * step
    v[-1] = b
    return v


def hz_to_mel(f):
    return 2595.0 * np.log10(1.0 + np.asarray(f, dtype=np.float64) / 700.0)


def mel_to_hz(m):
    return 700.0 * (10.0 ** (np.asarray(m, dtype=np.float64) / 2595.0) - 1.0)


def mel_filter_bank() -> np.ndarray:
    """HTK triangles without normalisation, [257 freq][128 mel] float64
    (egemma2_audio.rs, ``mel_filter_bank``): 130 points evenly spaced on the
    HTK mel scale over 0..8 kHz, 257 FFT frequencies over 0..8 kHz, and
    W[k][m] = max(0, min(rising edge, falling edge))."""
    n_freq = N_FFT // 2 + 1
    mels = linspace(float(hz_to_mel(0.0)), float(hz_to_mel(8000.0)), N_MELS + 2)
    ff = mel_to_hz(mels)
    fft_f = linspace(0.0, SAMPLE_RATE / 2, n_freq)
    W = np.zeros((n_freq, N_MELS), dtype=np.float64)
    for k, f in enumerate(fft_f):
        for m in range(N_MELS):
            down = -(ff[m] - f) / (ff[m + 1] - ff[m])
            up = (ff[m + 2] - f) / (ff[m + 2] - ff[m + 1])
            W[k, m] = max(0.0, min(down, up))
    return W


def frames_of(wave: np.ndarray) -> np.ndarray:
    """Windowed frames zero-padded to 512, [F, 512] float64.

    Frame i takes samples wave[160 i - 160 + j], j < 320 (160 zeros stand in
    front of the clip, the "semicausal" padding), times the window; entries
    320..511 are zero (egemma2_audio.rs, ``MelFrontend::log_mel``).
    """
    wave = np.asarray(wave, dtype=np.float64)[:MAX_SAMPLES]
    F = num_frames(len(wave))
    w = hann_window()
    out = np.zeros((F, N_FFT), dtype=np.float64)
    j = np.arange(FRAME)
    for i in range(F):
        p = i * HOP + j - HOP
        inside = p >= 0
        out[i, j[inside]] = wave[p[inside]] * w[inside]
    return out


def dft_magnitude(frames: np.ndarray) -> np.ndarray:
    """|X_k| = |sum_n x_n exp(-2 pi i k n / 512)| for k = 0..256, by the
    direct DFT as a matrix product (the definition; no FFT)."""
    n = np.arange(N_FFT)
    k = np.arange(N_FFT // 2 + 1)
    ang = 2.0 * np.pi * ((np.outer(n, k) % N_FFT) / N_FFT)
    re = frames @ np.cos(ang)
    im = -(frames @ np.sin(ang))
    return np.hypot(re, im)


def log_mel(wave: np.ndarray) -> np.ndarray:
    """[F, 128] log-mel: ln(sum_k |X_k| W[k][b] + 1e-3)
    (egemma2_audio.rs, ``MelFrontend::log_mel``)."""
    mag = dft_magnitude(frames_of(wave))
    return np.log(mag @ mel_filter_bank() + MEL_FLOOR)
