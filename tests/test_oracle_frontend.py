"""Pins for the oracle's front end (sizes, window, DFT, mel bank, log-mel).

Each pin comes from outside the oracle: values printed on the
egemma2_audio.rs page (tests/golden/printed_values.json), closed forms,
library routines (numpy.fft, numpy.interp) or brute force.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import frontend as fe

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "printed_values.json")))


# ------------------------------------------------------------------ sizes

def test_counts_match_printed_triples():
    for n, f, t in GOLD["token_counts"]["triples"]:
        assert oracle.num_frames(n) == f, n
        assert oracle.num_tokens(n) == t, n


def test_counts_brute_force_every_length():
    """Frame i is kept iff its window ends before the last sample
    (160 i + 160 <= N' - 1); a stride-2 conv with padding 1 has an output for
    every even input index. Counted literally for every N <= 500000."""
    N = np.arange(500001)
    Np = np.minimum(N, 480000)
    frames = np.zeros_like(N)
    for i in range(3001):
        frames += (160 * i + 160 <= Np - 1)
    t1 = np.zeros_like(N)
    for t in range(1501):
        t1 += (2 * t < frames)
    tok = np.zeros_like(N)
    for t in range(751):
        tok += (2 * t < t1)
    # spot-check the oracle's integer functions against the literal counts
    for n in list(range(0, 2000)) + list(range(478000, 482000)) + list(range(0, 500001, 997)):
        assert oracle.num_frames(n) == frames[n], n
        assert oracle.num_tokens(n) == tok[n], n


def test_frame_rows_match_count():
    for n in (0, 160, 161, 320, 321, 480, 481, 1000, 16000):
        assert fe.frames_of(np.zeros(n, np.float32)).shape == (oracle.num_frames(n), 512)


# ----------------------------------------------------------------- window

def test_periodic_hann_closed_form():
    w = oracle.hann_window()
    assert w.shape == (320,)
    assert w[0] == 0.0
    assert abs(w[160] - 1.0) < 1e-15
    assert abs(w[80] - 0.5) < 1e-15 and abs(w[240] - 0.5) < 1e-15
    for n in range(1, 320):
        assert abs(w[n] - w[320 - n]) < 1e-15
    # a periodic Hann of length N sums to N/2 exactly
    assert abs(w.sum() - 160.0) < 1e-12


# -------------------------------------------------------------------- DFT

def test_dft_matches_numpy_fft():
    rng = np.random.default_rng(7)
    x = rng.standard_normal((6, 512))
    ref = np.abs(np.fft.rfft(x, axis=1))
    got = oracle.dft_magnitude(x)
    assert np.max(np.abs(got - ref)) < 1e-10 * np.max(ref)


def test_dft_parseval():
    rng = np.random.default_rng(8)
    x = rng.standard_normal((4, 512))
    X = oracle.dft_magnitude(x)
    e = (X[:, 0] ** 2 + X[:, 256] ** 2 + 2 * (X[:, 1:256] ** 2).sum(axis=1)) / 512
    assert np.allclose(e, (x ** 2).sum(axis=1), rtol=1e-12)


@pytest.mark.parametrize("freq,bin_", [(440.0, 14), (1000.0, 32), (7000.0, 224)])
def test_tone_peaks_in_its_bin(freq, bin_):
    n = np.arange(512)
    x = np.zeros(512)
    x[:320] = np.sin(2 * np.pi * freq * n[:320] / 16000) * oracle.hann_window()
    assert int(np.argmax(oracle.dft_magnitude(x[None])[0])) == bin_


# --------------------------------------------------------------- mel bank

def test_mel_bank_printed_values():
    g = GOLD["mel_bank"]
    W = oracle.mel_filter_bank()
    assert list(W.shape) == g["shape"]
    assert abs(W[1, 1] - g["W_1_1"]) < g["tol"]
    assert abs(W[1, 2] - g["W_1_2"]) < g["tol"]
    assert np.all(W[0] == 0.0)           # DC row
    assert np.all(W[:, 0] == 0.0)        # band 0 empty
    assert np.all((W >= 0.0) & (W <= 1.0))


def test_mel_bank_is_interpolated_hat():
    """Each band is the piecewise-linear hat through (f_m, 0), (f_{m+1}, 1),
    (f_{m+2}, 0) on HTK-spaced edges: rebuilt with numpy.interp."""
    W = oracle.mel_filter_bank()
    mmax = 2595.0 * math.log10(1.0 + 8000.0 / 700.0)
    edges = np.array([700.0 * (10 ** (mmax * i / 129 / 2595.0) - 1.0) for i in range(130)])
    freqs = np.arange(257) * (8000.0 / 256)
    for m in range(128):
        hat = np.interp(freqs, edges[m:m + 3], [0.0, 1.0, 0.0], left=0.0, right=0.0)
        assert np.max(np.abs(hat - W[:, m])) < 1e-9, m


def test_mel_bank_partition_of_unity_and_edges():
    W = oracle.mel_filter_bank()
    mels = fe.linspace(float(fe.hz_to_mel(0.0)), float(fe.hz_to_mel(8000.0)), 130)
    ff = fe.mel_to_hz(mels)
    assert abs(ff[0]) < 2e-12 and abs(ff[129] - 8000.0) < 2e-12
    freqs = np.arange(257) * 31.25
    inside = (freqs >= ff[1]) & (freqs <= ff[128])
    assert np.allclose(W[inside].sum(axis=1), 1.0, atol=1e-12)
    # at most two bands touch any bin; each band's support is contiguous
    assert np.all((W > 0).sum(axis=1) <= 2)
    for m in range(128):
        nz = np.nonzero(W[:, m] > 0)[0]
        if len(nz):
            assert np.all(np.diff(nz) == 1)


# ---------------------------------------------------------------- log-mel

def test_silence_is_the_floor():
    g = GOLD["silence"]
    m = oracle.log_mel(np.zeros(g["samples"], np.float32))
    assert m.shape == (g["frames"], 128)
    assert np.all(np.abs(m - math.log(1e-3)) < g["tol"])


def test_band_zero_is_always_the_floor():
    x = np.random.default_rng(3).uniform(-1, 1, 4000).astype(np.float32)
    m = oracle.log_mel(x)
    assert np.all(m[:, 0] == math.log(1e-3))


def _centre(b):
    mmax = 2595.0 * math.log10(1.0 + 8000.0 / 700.0)
    return 700.0 * (10 ** (mmax * (b + 1) / 129 / 2595.0) - 1.0)


@pytest.mark.parametrize("freq", [1000.0, 440.0, 3000.0])
def test_tone_lands_in_its_band(freq):
    g = GOLD["tone"]
    n = np.arange(g["samples"])
    x = (g["amplitude"] * np.sin(2 * np.pi * freq * n / 16000)).astype(np.float32)
    m = oracle.log_mel(x)
    best = int(np.argmax(m[len(m) // 2]))
    assert abs(_centre(best) - freq) < g["max_centre_error_hz"]


def test_impulse_fixes_frame_offset_and_window():
    """An impulse at sample 0 sits at j = 160 of frame 0 (window 1: a flat
    unit spectrum) and at j = 0 of frame 1 (window 0); at sample 80 it sits
    at j = 240 of frame 0 and j = 80 of frame 1 (window 0.5 in both)."""
    W = oracle.mel_filter_bank()
    floor = math.log(1e-3)
    x = np.zeros(1000, np.float32)
    x[0] = 1.0
    m = oracle.log_mel(x)
    assert np.allclose(m[0], np.log(W.sum(axis=0) + 1e-3), atol=1e-12)
    assert np.allclose(m[1:], floor, atol=1e-12)
    x = np.zeros(1000, np.float32)
    x[80] = 1.0
    m = oracle.log_mel(x)
    for i in (0, 1):
        assert np.allclose(m[i], np.log(0.5 * W.sum(axis=0) + 1e-3), atol=1e-12)
    assert np.allclose(m[2:], floor, atol=1e-12)


def test_truncation_at_30_s():
    x = np.random.default_rng(4).uniform(-1, 1, 480000 + 3000).astype(np.float32)
    a = oracle.log_mel(x)
    assert a.shape == (2999, 128)
    # frames near the end only see samples below 480000
    b = oracle.log_mel(x[:480000])
    assert np.array_equal(a[-5:], b[-5:])
