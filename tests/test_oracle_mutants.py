"""Planted mistakes in a copy of the oracle tower must each fail a pin.

Each case replaces one exact piece of ``oracle/tower.py``'s source with a
plausible misreading of the page (egemma2_audio.rs, cortiq-engine 0.8.49),
loads the result as a separate module and runs the pins of
``tower_pins.py`` and ``test_oracle_tower.py`` against it. The real oracle
passes every pin (``test_oracle_tower_pins.py``); a mutant that passes them
all would mean a pin is missing.
"""
import inspect
import types

import numpy as np
import pytest

from oracle import tower as tw
from tower_pins import PINS

# (name, original source fragment, planted replacement)
MUTANTS = [
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
]


def _load_mutant(old, new):
    src = inspect.getsource(tw)
    assert src.count(old) == 1, f"fragment not found exactly once: {old!r}"
    mod = types.ModuleType("oracle._tower_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "<oracle.tower mutant>", "exec"), mod.__dict__)
    return mod


def _older_pins():
    """The pins of test_oracle_tower.py that take the module's functions
    through ``tw``: run them against a mutant by swapping the name."""
    import test_oracle_tower as t
    names = ["test_rms_norm_closed_form", "test_clip_linear_bounds_in_and_out",
             "test_tower_constants", "test_rel_pos_table_closed_form",
             "test_attention_window_by_perturbation", "test_attention_first_token_is_its_value",
             "test_attention_zero_query_averages_the_span", "test_attention_relative_term_and_softcap",
             "test_attention_block_residual_rms_is_one", "test_ffn_half_residual",
             "test_glu_closed_form", "test_dwconv_impulse_response",
             "test_light_conv_zero_end_is_identity", "test_layer_output_rms_with_unit_gain",
             "test_head_is_affine_norm_then_projection"]
    return t, [getattr(t, n) for n in names]


def _fails_some_pin(mod):
    failed = []
    for pin in PINS:
        try:
            pin(mod)
        except (AssertionError, FloatingPointError, ValueError, IndexError):
            failed.append(pin.__name__)
    t, older = _older_pins()
    saved = t.tw
    t.tw = mod
    try:
        for pin in older:
            try:
                pin()
            except (AssertionError, ValueError, IndexError):
                failed.append(pin.__name__)
    finally:
        t.tw = saved
    return failed


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, old, new):
    mod = _load_mutant(old, new)
    with np.errstate(over="ignore"):
        failed = _fails_some_pin(mod)
    assert failed, f"planted mistake '{name}' passes every pin"


def test_unmutated_copy_passes_every_pin():
    mod = _load_mutant("EPS = 1e-6", "EPS = 1e-6")
    assert _fails_some_pin(mod) == []
