"""GPU: the encoder with int8 projections (ae_model_create_q8).

Two bars: (1) bit-identity with a bf16 model whose matrices are the
widened weights bf16(float32(q) * s), computed by the oracle (same kernels,
same operands, so the same bits); (2) the oracle encoder on the widened
weights, at the bf16 tolerance of the final embeddings (2e-2 relative)."""
import copy

import numpy as np
import pytest

import oracle
from oracle import quant
from log_mel_conformer_amd import synth
from _util import bf16_gate, rel_l2, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from log_mel_conformer_amd import ae  # noqa: E402


def widened(W, S):
    Wd = copy.deepcopy(W)
    for L, sc in zip(Wd["layers"], S):
        for k in synth.Q8_MATRICES:
            L[k] = quant.dequantize_rows(L[k], sc[k]).astype(np.float32)
    return Wd


def test_q8_model_is_bit_identical_to_widened_bf16_model():
    say("[gpu] int8 projections: 2 layers, tone + ragged clips vs the widened bf16 model")
    W, S = synth.make_weights_q8(2)
    m8 = ae.Model(W, "bf16", scales=S)
    m16 = ae.Model(widened(W, S), "bf16")
    rng = np.random.default_rng(3)
    clips = [synth.tone_clip(0), rng.uniform(-0.5, 0.5, 23456).astype(np.float32)]
    wave, so = synth.pack(clips)
    wv = torch.from_numpy(wave).cuda()
    a = ae.encode(m8, wv, so).cpu().numpy()
    b = ae.encode(m16, wv, so).cpu().numpy()
    assert np.array_equal(a, b)
    # one layer through ae_conformer_layer
    h = torch.from_numpy(rng.standard_normal((300, 1024)).astype(np.float32)).cuda()
    pos = torch.arange(300, dtype=torch.int32, device="cuda")
    h8, h16 = h.clone(), h.clone()
    ae.conformer_layer(m8, 1, h8, pos)
    ae.conformer_layer(m16, 1, h16, pos)
    assert torch.equal(h8, h16)


def test_q8_model_vs_oracle_30s_12_layers():
    say("[gpu] int8 projections: 12 layers, one 30 s clip vs the oracle on widened weights")
    W, S = synth.make_weights_q8(12)
    m8 = ae.Model(W, "bf16", scales=S)
    clip = synth.multisine_clip(0)
    wave, so = synth.pack([clip])
    got = ae.encode(m8, torch.from_numpy(wave).cuda(), so).cpu().numpy()
    want = oracle.encode_clips([clip], widened(W, S))[0]
    bf16_gate(got, want, "final embeddings")
