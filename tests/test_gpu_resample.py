"""GPU parity of the mixdown and the resampler (the step ahead of the
log-mel) against the oracle, through the C ABI.

Bars: the mixdown is float32 arithmetic in a fixed order, so it must be
bit-exact. A resampled value is a float64 sum rounded to float32; the HIP
path and the oracle add the same terms in different orders. With terms of
magnitude at most 1 (samples in [-1, 1] times taps below 1) and at most
~4000 of them, the two sums differ by less than 4000 * 2^-53 < 1e-12, so
elementwise the float32 results may differ by one float32 ulp (where the
sums straddle a rounding boundary) or by 1e-12 absolute (outputs whose
exact value is zero, e.g. a tone's zero crossings), whichever is larger;
and outputs above 1e-6 in magnitude must be bit-identical in all but 2%.
Lengths are exact integers. Full-size batches compare sampled outputs
against the defining sum evaluated on the tap window.
"""
import math

import numpy as np
import pytest

from oracle import resample as ors
from log_mel_conformer_amd import synth
from _util import say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from log_mel_conformer_amd import ae  # noqa: E402

RATES = [48000, 44100, 22050, 8000, 32000, 11025, 24000, 96000, 12000, 44099, 384000]


def cuda(x):
    return torch.as_tensor(np.ascontiguousarray(x)).to("cuda", torch.float32)


def within_ulp(g, o, what):
    g = np.asarray(g, np.float32)
    o = np.asarray(o, np.float32)
    assert g.shape == o.shape, (what, g.shape, o.shape)
    if g.size == 0:
        return
    ulp = np.maximum(np.spacing(np.abs(o)), np.spacing(np.abs(g))).astype(np.float64)
    d = np.abs(g.astype(np.float64) - o.astype(np.float64))
    bad = d > np.maximum(ulp, 1e-12)
    assert not bad.any(), f"{what}: {bad.sum()} values beyond one ulp, worst {d.max():.3e}"
    big = np.abs(o) > 1e-6
    if big.any():
        same = float(np.mean(g[big] == o[big]))
        assert same > 0.98, f"{what}: only {same:.4f} bit-identical"


def test_mixdown_is_bit_exact():
    rng = np.random.default_rng(21)
    for ch in (1, 2, 3, 6):
        say(f"[gpu] mixdown: {ch} channels")
        x = rng.standard_normal((4099, ch)).astype(np.float32)
        g = ae.mixdown(cuda(x), ch).cpu().numpy()
        o = ors.mixdown([x[:, c] for c in range(ch)])
        assert np.array_equal(g, o), ch


@pytest.mark.parametrize("fr", RATES)
def test_resample_matches_oracle_ragged(fr):
    say(f"[gpu] resample {fr} -> 16000: ragged batch with empty and tiny clips")
    rng = np.random.default_rng(fr)
    lens = [0, 1, 2, 7, 333, int(0.25 * fr), 0, 1234]
    clips = [rng.uniform(-1, 1, n).astype(np.float32) for n in lens]
    wave, off = synth.pack(clips)
    r = ae.Resampler(fr, 16000)
    try:
        y = ae.resample(r, cuda(wave), off).cpu().numpy()
        oo = r.out_offsets(off)
        assert int(oo[-1]) == sum(ors.resampled_length(n, fr, 16000) for n in lens)
        for i, x in enumerate(clips):
            within_ulp(y[oo[i]:oo[i + 1]], ors.resample(x, fr, 16000), f"{fr} clip {i}")
    finally:
        r.close()


def test_equal_rates_copy():
    say("[gpu] resample 16000 -> 16000 is a copy")
    x = np.random.default_rng(2).standard_normal(5000).astype(np.float32)
    r = ae.Resampler(16000, 16000)
    try:
        y = ae.resample(r, cuda(x), np.array([0, 3000, 5000])).cpu().numpy()
    finally:
        r.close()
    assert np.array_equal(y, x)


def test_printed_tones_alias_and_constant():
    say("[gpu] the page's tone, alias and constant cases")
    for fr, f0 in [(8000, 1000.0), (44100, 3000.0), (48000, 7000.0), (22050, 440.0)]:
        x = np.sin(2 * np.pi * f0 * np.arange(fr) / fr).astype(np.float32)
        r = ae.Resampler(fr, 16000)
        try:
            y = ae.resample(r, cuda(x), np.array([0, fr])).cpu().numpy()
        finally:
            r.close()
        assert len(y) == 16000
        i = np.arange(2000, 14000)
        assert np.abs(y[i] - np.sin(2 * np.pi * f0 * i / 16000.0)).max() < 1e-4, fr
        within_ulp(y, ors.resample(x, fr, 16000), f"tone {fr}")
    x = np.sin(2 * np.pi * 9000.0 * np.arange(48000) / 48000).astype(np.float32)
    r = ae.Resampler(48000, 16000)
    try:
        y = ae.resample(r, cuda(x), np.array([0, 48000])).cpu().numpy().astype(np.float64)
        assert math.sqrt(np.mean(y[2000:14000] ** 2)) < 1e-4
        c = np.full((4800, 1), 0.25, np.float32)
        m = ae.to_mono_16k(r, cuda(c), np.array([0, 4800]), 1).cpu().numpy()
    finally:
        r.close()
    assert len(m) == 1600 and abs(float(m[800]) - 0.25) < 1e-4


def test_to_mono_16k_stereo_ragged():
    say("[gpu] to_mono_16k: 5 stereo clips at 44.1 kHz, ragged")
    clips = [synth.recorded_clip(s, 44100, sec) for s, sec in
             enumerate([0.3, 0.01, 1.0, 0.0, 0.77])]
    data, off = synth.pack_frames(clips)
    r = ae.Resampler(44100, 16000)
    try:
        y = ae.to_mono_16k(r, cuda(data), off, 2).cpu().numpy()
        oo = r.out_offsets(off)
    finally:
        r.close()
    for i, c in enumerate(clips):
        within_ulp(y[oo[i]:oo[i + 1]], ors.to_mono_16k([c[:, 0], c[:, 1]], 44100), f"clip {i}")


def _definition_at(x64, m, fr, to, c):
    """The defining sum for output m, over the taps where h can be nonzero."""
    pos = m * fr / to
    half = 64.0 / c
    lo, hi = max(0, math.floor(pos - half) - 1), min(len(x64), math.ceil(pos + half) + 2)
    n = np.arange(lo, hi)
    return float(np.dot(x64[lo:hi], ors.kernel(n - pos, c)))


def test_full_size_48k_stereo_sampled():
    """32 clips x 30 s of stereo at 48 kHz, one launch as the benchmark
    runs it; sampled outputs of clips 0 and 31 against the definition."""
    say("[gpu] to_mono_16k: 32 x 30 s stereo 48 kHz, sampled outputs of clips 0 and 31")
    clips = synth.recorded_batch(32, 48000, 30.0)
    data, off = synth.pack_frames(clips)
    r = ae.Resampler(48000, 16000)
    try:
        y = ae.to_mono_16k(r, cuda(data), off, 2).cpu().numpy()
        oo = r.out_offsets(off)
    finally:
        r.close()
    assert len(y) == 32 * 480000 and np.all(np.diff(oo) == 480000)
    c = ors.cutoff(48000, 16000)
    rng = np.random.default_rng(0)
    for ci in (0, 31):
        mono = ors.mixdown([clips[ci][:, 0], clips[ci][:, 1]]).astype(np.float64)
        ms = [0, 1, 2, 479997, 479998, 479999] + list(rng.integers(0, 480000, 58))
        got = y[oo[ci] + np.array(ms)]
        want = np.array([_definition_at(mono, m, 48000, 16000, c) for m in ms], np.float32)
        within_ulp(got, want, f"clip {ci}")


def test_errors_are_reported():
    say("[gpu] resampler error paths")
    r = ae.Resampler(48000, 22050)
    try:
        x = cuda(np.zeros((100, 2), np.float32))
        with pytest.raises(ae.AeError) as e:
            ae.to_mono_16k(r, x, np.array([0, 100]), 2)
        assert e.value.status == ae.AE_ERR_INVALID
    finally:
        r.close()
    r = ae.Resampler(48000, 16000)
    try:
        x = cuda(np.zeros(480, np.float32))
        y = torch.empty(160, dtype=torch.float32, device="cuda")
        small = torch.empty(8, dtype=torch.uint8, device="cuda")
        off, op = ae._i64([0, 480])
        st = ae.lib().ae_resample(r.handle, ae._ptr(x), op, 1, ae._ptr(y), ae._ptr(small), 8,
                                  ae._stream())
        assert st == ae.AE_ERR_CAPACITY
    finally:
        r.close()
    with pytest.raises(ae.AeError) as e:
        ae.Resampler(0, 16000)
    assert e.value.status == ae.AE_ERR_INVALID
