"""Shared helpers of the test suite: parity metrics and cached inputs."""
import functools
import sys

import numpy as np

from log_mel_conformer_amd import synth


def rel_l2(got, want):
    """||got - want||_2 / ||want||_2 in float64."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    den = np.linalg.norm(w)
    return float(np.linalg.norm(g - w) / (den if den > 0 else 1.0))


def rel_max(got, want):
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    den = np.max(np.abs(w)) if w.size else 1.0
    return float(np.max(np.abs(g - w)) / (den if den > 0 else 1.0)) if w.size else 0.0


def say(msg):
    """Progress line that survives output capture and a lost box."""
    sys.__stderr__.write(msg + "\n")
    sys.__stderr__.flush()


@functools.lru_cache(maxsize=4)
def weights(layers, bf16=False):
    return synth.make_weights(layers=layers, bf16=bf16)


# bf16 gates. Per clip: rel-L2 <= 2e-2 on the final embeddings (the stated
# bar). Per token: each row's rel-L2 <= 5e-2, and over the clip
# max|g - o| / max|o| <= 5e-2, so that one bad token cannot hide inside a
# clip's norm (a token 50% off in a 750-token clip moves the clip's rel-L2
# by only about 0.5 / sqrt(750) = 0.018).
BF16_CLIP_TOL = 2e-2
BF16_TOKEN_TOL = 5e-2
BF16_MAX_TOL = 5e-2


def token_rel_l2(got, want):
    """The largest per-row ||g_t - o_t||_2 / ||o_t||_2 (0 for no rows)."""
    g = np.asarray(got, dtype=np.float64)
    w = np.asarray(want, dtype=np.float64)
    if w.shape[0] == 0:
        return 0.0
    den = np.linalg.norm(w, axis=1)
    den = np.where(den > 0, den, 1.0)
    return float(np.max(np.linalg.norm(g - w, axis=1) / den))


def bf16_gate(got, want, what):
    """Assert the three bf16 bars on one clip's rows; print the figures."""
    assert np.asarray(got).shape == np.asarray(want).shape, (what, np.shape(got), np.shape(want))
    r, t, m = rel_l2(got, want), token_rel_l2(got, want), rel_max(got, want)
    say(f"    {what}: rel {r:.3e}, worst token {t:.3e}, max-rel {m:.3e}")
    assert np.all(np.isfinite(got)), what
    assert r <= BF16_CLIP_TOL, (what, "clip rel-L2", r)
    assert t <= BF16_TOKEN_TOL, (what, "token rel-L2", t)
    assert m <= BF16_MAX_TOL, (what, "max-rel", m)
