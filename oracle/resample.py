"""Oracle for the step ahead of the log-mel: channel mixdown and band-limited
resampling to 16 kHz.

TEST INFRASTRUCTURE (see the package docstring). float64 except where the
page fixes float32 (the mixdown, and the final cast of each output).
Source: egemma2_audio.rs (cortiq-engine 0.8.49), ``to_mono_16k``,
``resample_hq``, ``bessel_i0`` and the resampler constants above them.

The resampler, stated as a definition: with r = from/to and
c = min(1, to/from) * 0.958 (the cut-off as a fraction of the lower of the
two Nyquist rates, expressed in cycles per input sample times two),

    y[m] = sum_n x[n] h(n - m r),
    h(d) = c sinc(c d) I0(12.8 sqrt(1 - (c d / 64)^2)) / I0(12.8)   if |c d| < 64,
    h(d) = 0                                                         otherwise,

sinc(t) = sin(pi t) / (pi t), summed in float64 over the input samples
(samples outside the clip are absent), for m = 0 .. ceil(N to / from) - 1,
each output rounded to float32. Equal rates return the input unchanged.
The page evaluates h per output phase over the span of taps where it can be
nonzero; taps outside that span are zero, so the sum is the same.
"""
from __future__ import annotations

import math

import numpy as np

ZERO_CROSSINGS = 64.0   # sinc zero crossings on each side of the centre
ROLLOFF = 0.958         # cut-off as a fraction of the lower Nyquist rate
KAISER_BETA = 12.8
TARGET_RATE = 16000


def bessel_i0(x):
    """Modified Bessel function of the first kind, order 0, by its power
    series sum_k ((x/2)^2)^k / (k!)^2, summed until a term falls below
    1e-17 of the sum (egemma2_audio.rs, ``bessel_i0``). Elementwise."""
    x = np.asarray(x, dtype=np.float64)
    q = x * x / 4.0
    term = np.ones_like(q)
    total = np.ones_like(q)
    for k in range(1, 400):
        term = term * q / float(k * k)
        total = total + term
        if np.all(term < total * 1e-17):
            break
    return total


def resampled_length(n: int, from_rate: int, to_rate: int) -> int:
    """Output length: unchanged for equal rates, else ceil(to * n / from)
    (egemma2_audio.rs, ``resample_hq``; reducing the ratio by the gcd
    first leaves the ceiling unchanged)."""
    n = int(n)
    if from_rate == to_rate or n == 0:
        return n
    return -(-(to_rate * n) // from_rate)


def cutoff(from_rate: int, to_rate: int) -> float:
    """c = min(1, to/from) * 0.958: the kernel's sinc argument per input
    sample (egemma2_audio.rs, ``resample_hq``: base / o)."""
    g = math.gcd(from_rate, to_rate)
    o, nw = from_rate // g, to_rate // g
    return min(o, nw) / o * ROLLOFF


def kernel(d, c: float):
    """h(d) for offsets d in input samples (see the module docstring):
    Kaiser-windowed sinc with 64 zero crossings a side, beta 12.8, scaled by
    c so that the filter has unit gain at DC."""
    d = np.asarray(d, dtype=np.float64)
    t = d * c
    inside = np.abs(t) < ZERO_CROSSINGS
    r = np.where(inside, t / ZERO_CROSSINGS, 0.0)
    win = bessel_i0(KAISER_BETA * np.sqrt(1.0 - r * r)) / bessel_i0(KAISER_BETA)
    pt = np.pi * t
    with np.errstate(invalid="ignore", divide="ignore"):
        sinc = np.where(pt == 0.0, 1.0, np.sin(pt) / np.where(pt == 0.0, 1.0, pt))
    return np.where(inside, c * sinc * win, 0.0)


def resample_f64(x, from_rate: int, to_rate: int) -> np.ndarray:
    """The sums y[m] in float64, before the final cast.

    Output m = f * nw + j (nw = to/g, o = from/g) sits at input position
    f * o + j * o / nw, so every output of phase j uses the same taps
    h(d - j o / nw) at the integer offsets d around it; those rows of taps
    are applied to strided windows of x with a matrix product."""
    x = np.asarray(x, dtype=np.float32).astype(np.float64)
    n = len(x)
    if from_rate == to_rate or n == 0:
        return x.copy()
    g = math.gcd(from_rate, to_rate)
    o, nw = from_rate // g, to_rate // g
    m_total = resampled_length(n, from_rate, to_rate)
    c = cutoff(from_rate, to_rate)
    half = ZERO_CROSSINGS / c
    y = np.zeros(m_total, dtype=np.float64)
    for j in range(min(nw, m_total)):
        e = j * o / nw
        d = np.arange(math.floor(e - half), math.ceil(e + half) + 1)
        taps = kernel(d - e, c)
        outs = np.arange(j, m_total, nw)
        f = (outs - j) // nw
        for s in range(0, len(f), 4096):
            fb = f[s:s + 4096]
            idx = fb[:, None] * o + d[None, :]
            ok = (idx >= 0) & (idx < n)
            xs = np.where(ok, x[np.clip(idx, 0, n - 1)], 0.0)
            y[outs[s:s + 4096]] = xs @ taps
    return y


def resample(x, from_rate: int, to_rate: int) -> np.ndarray:
    """Band-limited resampling, float32 out (egemma2_audio.rs,
    ``resample_hq``)."""
    return resample_f64(x, from_rate, to_rate).astype(np.float32)


def mixdown(channels) -> np.ndarray:
    """Average of the channels, sample by sample: the channel values added
    in float32 in channel order, then divided by the channel count in
    float32 (egemma2_audio.rs, ``to_mono_16k``). No channels give an empty
    signal; one channel is returned as is."""
    chans = [np.asarray(ch, dtype=np.float32) for ch in channels]
    if not chans:
        return np.zeros(0, dtype=np.float32)
    if len(chans) == 1:
        return chans[0].copy()
    acc = chans[0].copy()
    for ch in chans[1:]:
        acc = (acc + ch).astype(np.float32)
    return (acc / np.float32(len(chans))).astype(np.float32)


def to_mono_16k(channels, rate: int) -> np.ndarray:
    """Mixdown, then resampling to 16 kHz (egemma2_audio.rs,
    ``to_mono_16k``)."""
    return resample(mixdown(channels), rate, TARGET_RATE)
