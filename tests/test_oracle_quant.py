"""Pins for the int8 dequantisation oracle: torch's own bf16 cast (library
routine), exactness where the product is representable, and per-row scope
of the scale."""
import numpy as np
import pytest

from oracle import quant

torch = pytest.importorskip("torch")


def test_round_bf16_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(10000) * 10 ** rng.uniform(-3, 3, 10000),
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -(1.0 + 2 ** -8), 0.0, -0.0])])
    x = x.astype(np.float32)   # includes exact ties (1 + 2^-8 rounds to 1, 1 + 3 2^-8 up)
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(quant.round_bf16(x), want)


def test_dequantize_exact_for_power_of_two_scales():
    q = np.arange(-127, 128, dtype=np.int8).reshape(5, 51)
    s = np.array([2.0 ** -7, 2.0 ** -3, 1.0, 0.5, 2.0 ** 4], dtype=np.float32)
    w = quant.dequantize_rows(q, s)
    assert np.array_equal(w, q.astype(np.float64) * s[:, None].astype(np.float64))


def test_scale_applies_to_its_row_only():
    rng = np.random.default_rng(1)
    q = rng.integers(-127, 128, (6, 40)).astype(np.int8)
    s = rng.uniform(1e-3, 1e-2, 6).astype(np.float32)
    w = quant.dequantize_rows(q, s)
    s2 = s.copy()
    s2[3] *= 3
    w2 = quant.dequantize_rows(q, s2)
    assert np.array_equal(np.delete(w, 3, 0), np.delete(w2, 3, 0))
    assert not np.array_equal(w[3], w2[3])
    # and it is the float32 product rounded once to bf16
    want = torch.from_numpy((q.astype(np.float32) * s[:, None])).to(torch.bfloat16).double().numpy()
    assert np.array_equal(w, want)
    with pytest.raises(TypeError):
        quant.dequantize_rows(q.astype(np.int16), s)
