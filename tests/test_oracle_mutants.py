"""Planted mistakes in a copy of the oracle must each fail a pin.

Each case replaces one exact piece of an oracle module's source
(``oracle/tower.py`` or ``oracle/frontend.py``) with a plausible misreading
of the page (egemma2_audio.rs, cortiq-engine 0.8.49), loads the result as a
separate module and runs the pins against it: ``tower_pins.py`` and
``test_oracle_tower.py`` for the tower, ``test_oracle_frontend.py`` for the
front end. The real oracle passes every pin; a mutant that passes them all
would mean a pin is missing.
"""
import inspect
import types

import numpy as np
import pytest

from oracle import frontend as fe
from oracle import tower as tw
from tower_pins import PINS

# (name, original source fragment, planted replacement)
TOWER_MUTANTS = [
    ("per-dimension query scale repeated instead of tiled over heads",
     "np.tile(q_dim, d // hd)", "np.repeat(q_dim, d // hd)"),
    ("softplus of per_dim_scale dropped",
     'q_dim = softplus(L["per_dim_scale"])', 'q_dim = _f64(L["per_dim_scale"])'),
    ("key scale applied to the query instead of the key",
     'k = k * c["k_scale"]', 'q = q * c["k_scale"]'),
    ("query scale without the 1/ln 2 factor",
     "q_scale=head_dim ** -0.5 / math.log(2.0)", "q_scale=head_dim ** -0.5"),
    ("relative keys as PE W instead of PE W^T",
     "rel_pos_table(n_dist, rel_k.shape[1]) @ rel_k.T", "rel_pos_table(n_dist, rel_k.shape[1]) @ rel_k"),
    ("relative table with cos before sin",
     "np.concatenate([np.sin(t), np.cos(t)], axis=1)", "np.concatenate([np.cos(t), np.sin(t)], axis=1)"),
    ("SiLU before W1's output clamp",
     'u = silu(clip_linear(a, L[f + "_w1"], L[f + "_w1_clip"]))',
     'lo_i, hi_i, lo_o, hi_o = L[f + "_w1_clip"]\n'
     '    u = np.clip(silu(np.clip(a, lo_i, hi_i) @ _f64(L[f + "_w1"]).T), lo_o, hi_o)'),
    ("FFN post norm dropped",
     'residual_weight * rms_norm(y, L[f + "_post"])', 'residual_weight * y'),
    ("light conv: SiLU then RMS norm",
     'c = silu(rms_norm(c, L["lc_norm"]))', 'c = rms_norm(silu(c), L["lc_norm"])'),
    ("GLU gate on the first half",
     "return g[:, :d] * sigmoid(g[:, d:])", "return g[:, d:] * sigmoid(g[:, :d])"),
    ("depthwise taps not reversed in time",
     "back = K - 1 - kk", "back = kk"),
    ("attention and light conv swapped",
     "    h = attention_block(h, L, pos, heads, R)\n    h = light_conv(h, L, pos)\n",
     "    h = light_conv(h, L, pos)\n    h = attention_block(h, L, pos, heads, R)\n"),
    ("FFN 2 run first",
     'h = ffn(h, L, "ff1", residual_weight)', 'h = ffn(h, L, "ff2", residual_weight)'),
    ("norm_out skipped",
     'return rms_norm(h, L["norm_out"])', "return h"),
    ("no soft cap",
     "s[dist] = softcap * math.tanh(logit / softcap)", "s[dist] = logit"),
    ("relative term indexed by the key's position, not the distance",
     "q[t, sl] @ R[dist, sl]", "q[t, sl] @ R[(t - dist) % R.shape[0], sl]"),
    ("subsampler flattened channel-major",
     "x = y1.reshape(y1.shape[0], -1)", "x = y1.transpose(0, 2, 1).reshape(y1.shape[0], -1)"),
    ("convolution without the leading zero pad",
     "xp[1:T + 1, 1:F + 1] = x", "xp[0:T, 0:F] = x"),
    ("LayerNorm without the mean",
     "return np.maximum((x - mean) / np.sqrt(var + EPS) * _f64(g), 0.0)",
     "return np.maximum(x / np.sqrt(var + EPS) * _f64(g), 0.0)"),
    ("no ReLU after the LayerNorm",
     "return np.maximum((x - mean) / np.sqrt(var + EPS) * _f64(g), 0.0)",
     "return (x - mean) / np.sqrt(var + EPS) * _f64(g)"),
    ("conv kernel taps transposed (time along df)",
     "out += patch @ w[:, :, dt, df].T", "out += patch @ w[:, :, df, dt].T"),
]

FRONTEND_MUTANTS = [
    ("symmetric instead of periodic Hann",
     "np.cos(2.0 * np.pi * n / FRAME)", "np.cos(2.0 * np.pi * n / (FRAME - 1))"),
    ("no 160 zeros in front of the clip (frame i starts at 160 i)",
     "p = i * HOP + j - HOP", "p = i * HOP + j"),
    ("frame count rounded down",
     "_ceil_div(n - HOP, HOP)", "(n - HOP) // HOP"),
    ("log10 instead of ln",
     "return np.log(mag @ mel_filter_bank() + MEL_FLOOR)",
     "return np.log10(mag @ mel_filter_bank() + MEL_FLOOR)"),
    ("power instead of magnitude",
     "return np.hypot(re, im)", "return re * re + im * im"),
    ("floor added after the log",
     "return np.log(mag @ mel_filter_bank() + MEL_FLOOR)",
     "return np.log(mag @ mel_filter_bank()) + MEL_FLOOR"),
    ("mel scale with a natural exponent",
     "10.0 ** (np.asarray(m, dtype=np.float64) / 2595.0)",
     "np.exp(np.asarray(m, dtype=np.float64) / 2595.0)"),
    ("129 mel edges instead of 130",
     "N_MELS + 2)", "N_MELS + 1)"),
    ("FFT frequencies up to 16 kHz",
     "fft_f = linspace(0.0, SAMPLE_RATE / 2, n_freq)", "fft_f = linspace(0.0, SAMPLE_RATE, n_freq)"),
    ("no 30 s cut",
     "n = min(int(n), MAX_SAMPLES)", "n = int(n)"),
    ("window applied to frame positions shifted by one",
     "out[i, j[inside]] = wave[p[inside]] * w[inside]",
     "out[i, j[inside]] = wave[p[inside]] * np.roll(w, 1)[inside]"),
]


def _load_mutant(base, old, new):
    src = inspect.getsource(base)
    assert src.count(old) == 1, f"fragment not found exactly once: {old!r}"
    mod = types.ModuleType(base.__name__ + "_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), f"<{base.__name__} mutant>", "exec"), mod.__dict__)
    return mod


def _cases(fn):
    """Argument sets of a pin: one empty set, or its parametrize values;
    None for pins that need fixtures."""
    params = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if params:
        names = [a.strip() for a in params[0].args[0].split(",")]
        return [dict(zip(names, v if isinstance(v, tuple) else (v,))) for v in params[0].args[1]]
    return [{}] if not inspect.signature(fn).parameters else None


def _first_failing_pin(testmod, swaps, extra=()):
    """Run every argument-free or parametrized test of `testmod` (and the
    callables in `extra`) with its module globals swapped; the name of the
    first one that fails, or None."""
    saved = {k: getattr(testmod, k) for k in swaps}
    for k, v in swaps.items():
        setattr(testmod, k, v)
    try:
        for pin in extra:
            try:
                pin()
            except Exception:
                return pin.__name__
        for name in sorted(n for n in dir(testmod) if n.startswith("test_")):
            fn = getattr(testmod, name)
            cases = _cases(fn)
            if cases is None:
                continue
            for c in cases:
                try:
                    fn(**c)
                except Exception:
                    return name
    finally:
        for k, v in saved.items():
            setattr(testmod, k, v)
    return None


def _tower_failure(mod):
    import test_oracle_tower as t
    return _first_failing_pin(t, {"tw": mod}, extra=[lambda pin=p: pin(mod) for p in PINS])


def _frontend_failure(mod):
    import test_oracle_frontend as t
    ns = types.SimpleNamespace(**{n: getattr(mod, n) for n in (
        "num_frames", "num_tokens", "log_mel", "mel_filter_bank", "dft_magnitude", "hann_window")})
    return _first_failing_pin(t, {"fe": mod, "oracle": ns})


@pytest.mark.parametrize("name,old,new", TOWER_MUTANTS, ids=[m[0] for m in TOWER_MUTANTS])
def test_planted_tower_mistake_fails_a_pin(name, old, new):
    mod = _load_mutant(tw, old, new)
    with np.errstate(all="ignore"):
        assert _tower_failure(mod), f"planted mistake '{name}' passes every pin"


@pytest.mark.parametrize("name,old,new", FRONTEND_MUTANTS, ids=[m[0] for m in FRONTEND_MUTANTS])
def test_planted_frontend_mistake_fails_a_pin(name, old, new):
    mod = _load_mutant(fe, old, new)
    with np.errstate(all="ignore"):
        assert _frontend_failure(mod), f"planted mistake '{name}' passes every pin"


def test_unmutated_copies_pass_every_pin():
    with np.errstate(all="ignore"):
        assert _tower_failure(_load_mutant(tw, "EPS = 1e-6", "EPS = 1e-6")) is None
        assert _frontend_failure(_load_mutant(fe, "MEL_FLOOR = 1e-3", "MEL_FLOOR = 1e-3")) is None
