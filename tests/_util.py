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
