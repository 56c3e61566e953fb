"""Pins for the oracle's mixdown and resampler.

Each pin comes from outside the oracle: the values and bounds of the
egemma2_audio.rs page's own unit tests (tests/golden/resample_printed.json),
scipy's Bessel function, exact integer arithmetic, brute-force evaluation of
the defining sum, and invariants of the kernel (evenness, support, DC gain).
"""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

from oracle import resample as rs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "resample_printed.json")))


def test_bessel_i0_matches_scipy():
    x = np.array([0.0, 0.25, 1.0, 3.0, 7.5, 12.8, 20.0, 40.0])
    np.testing.assert_allclose(rs.bessel_i0(x), scipy.special.i0(x), rtol=1e-14, atol=0)


def test_length_is_exact_ceiling():
    rates = [8000, 11025, 16000, 22050, 24000, 32000, 44100, 44099, 48000, 96000, 7]
    for fr in rates:
        for n in [0, 1, 2, 3, 159, 160, 161, 999, 44099, 48000, 123457]:
            want = n if fr == 16000 else math.ceil(Fraction(16000 * n, fr))
            assert rs.resampled_length(n, fr, 16000) == want, (fr, n)


def test_equal_rates_are_the_identity():
    x = np.random.default_rng(3).standard_normal(1000).astype(np.float32)
    y = rs.resample(x, 16000, 16000)
    assert y.dtype == np.float32 and np.array_equal(x, y)
    assert len(rs.resample(np.zeros(0, np.float32), 48000, 16000)) == 0


def test_mixdown_printed_example():
    g = GOLD["mixdown"]
    y = rs.to_mono_16k([np.array(c, np.float32) for c in g["channels"]], g["rate"])
    assert y.tolist() == g["expected"]


def test_mixdown_is_float32_sum_then_divide():
    rng = np.random.default_rng(5)
    ch = [rng.standard_normal(257).astype(np.float32) for _ in range(3)]
    want = np.array([(np.float32(np.float32(a + b) + c)) / np.float32(3)
                     for a, b, c in zip(*ch)], np.float32)
    assert np.array_equal(rs.mixdown(ch), want)
    one = rs.mixdown([ch[0]])
    assert np.array_equal(one, ch[0])
    assert len(rs.mixdown([])) == 0


def test_constant_at_48k_printed():
    g = GOLD["constant"]
    y = rs.to_mono_16k([np.full(g["samples"], g["value"], np.float32)], g["rate"])
    assert len(y) == g["out_len"]
    assert abs(float(y[g["probe"]]) - g["value"]) < g["tol"]


@pytest.mark.parametrize("pair", GOLD["tones"]["pairs"])
def test_tones_keep_shape_and_length_printed(pair):
    g = GOLD["tones"]
    fr, f0 = int(pair[0]), float(pair[1])
    x = np.sin(2 * np.pi * f0 * np.arange(fr) / fr).astype(np.float32)
    y = rs.resample(x, fr, 16000)
    assert len(y) == g["out_len"]
    i = np.arange(*g["window"])
    err = np.abs(y[i].astype(np.float64) - np.sin(2 * np.pi * f0 * i / 16000.0)).max()
    assert err < g["max_err"], (fr, err)


def test_tone_above_new_nyquist_is_removed_printed():
    g = GOLD["alias"]
    fr = g["rate"]
    x = np.sin(2 * np.pi * g["freq_hz"] * np.arange(fr) / fr).astype(np.float32)
    y = rs.resample(x, fr, 16000)
    w = y[g["window"][0]:g["window"][1]].astype(np.float64)
    assert math.sqrt(np.mean(w * w)) < g["max_rms"]


def test_coprime_rate_length_and_brute_force_printed():
    g = GOLD["coprime"]
    x = ((np.arange(g["samples"]) % g["period"]).astype(np.float32) / np.float32(g["period"])
         - np.float32(0.5)).astype(np.float32)
    y = rs.resample_f64(x, g["rate"], 16000)
    assert len(y) == g["out_len"]
    c = rs.cutoff(g["rate"], 16000)
    n = np.arange(len(x))
    for m in [0, 1, 7919, 15998, 15999]:
        direct = float(np.dot(x.astype(np.float64), rs.kernel(n - m * g["rate"] / 16000.0, c)))
        assert abs(direct - y[m]) < 1e-12, m


@pytest.mark.parametrize("fr", [48000, 44100, 22050, 8000, 32000, 11025, 44099, 96000, 12000])
def test_phase_bookkeeping_matches_the_defining_sum(fr):
    """y[m] = sum_n x[n] h(n - m from/to), evaluated term by term."""
    x = np.random.default_rng(fr).uniform(-1, 1, 301).astype(np.float32)
    y = rs.resample_f64(x, fr, 16000)
    c = rs.cutoff(fr, 16000)
    assert len(y) == rs.resampled_length(len(x), fr, 16000)
    ms = sorted(set([0, 1, 2, len(y) // 2, len(y) - 2, len(y) - 1] +
                    list(np.random.default_rng(1).integers(0, len(y), 24))))
    for m in ms:
        pos = Fraction(int(m) * fr, 16000)
        offs = [float(k - pos) for k in range(len(x))]
        terms = x.astype(np.float64) * rs.kernel(np.array(offs), c)
        assert abs(math.fsum(terms) - y[m]) < 1e-12, (fr, m)


def test_kernel_is_even_with_bounded_support_and_unit_peak():
    for fr in [48000, 8000, 44100]:
        c = rs.cutoff(fr, 16000)
        d = np.linspace(-70 / c, 70 / c, 2001)
        h = rs.kernel(d, c)
        np.testing.assert_allclose(h, rs.kernel(-d, c), rtol=0, atol=1e-18)
        assert np.all(h[np.abs(d * c) >= 64.0] == 0.0)
        assert float(rs.kernel(0.0, c)) == pytest.approx(c, rel=1e-15)
        # the window falls to 1/I0(beta) at the edge of the support
        edge = 63.999999 / c
        ratio = float(rs.kernel(edge, c)) / (c * np.sinc(63.999999))
        assert ratio == pytest.approx(1.0 / float(scipy.special.i0(12.8)), rel=1e-3)


def test_dc_gain_is_one():
    """Sum of the taps a phase applies: the filter's response at DC, which a
    windowed sinc scaled by its cut-off keeps at 1 up to its stopband level."""
    for fr in [48000, 44100, 8000, 22050]:
        c = rs.cutoff(fr, 16000)
        half = 64 / c
        for e in [0.0, 0.137, 0.5, 0.861]:
            d = np.arange(math.floor(-half) - 2, math.ceil(half) + 3)
            assert abs(rs.kernel(d - e, c).sum() - 1.0) < 1e-6, (fr, e)


def test_cutoff_is_the_lower_nyquist_fraction():
    assert rs.cutoff(48000, 16000) == pytest.approx(16000 / 48000 * 0.958, rel=1e-15)
    assert rs.cutoff(8000, 16000) == pytest.approx(0.958, rel=1e-15)
    assert rs.cutoff(44099, 16000) == pytest.approx(16000 / 44099 * 0.958, rel=1e-15)
