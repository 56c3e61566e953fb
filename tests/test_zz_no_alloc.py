"""ae_encode_static, the encoder entry point that allocates nothing (its
workspace is the library's static device scratch), against ae_encode with a
caller workspace: two calls in a row, the second on a smaller batch, each
bit-identical to ae_encode on the same inputs (same kernels and buffer
layout, only the base address differs), plus one clip against the oracle
and the capacity refusal."""
import numpy as np
import pytest

import oracle
from log_mel_conformer_amd import synth
from _util import bf16_gate, rel_l2, say, weights

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover
    pytest.skip("no GPU", allow_module_level=True)

from log_mel_conformer_amd import ae  # noqa: E402


def test_static_scratch_matches_workspace_encode_twice():
    say("[gpu] encode_static: 30 s + 7 s clips, then one 3 s clip, bf16, vs ae_encode")
    W = weights(12, bf16=True)
    m = ae.Model(W, dtype="bf16")
    first = [synth.multisine_clip(3), synth.pink_clip(4, 7 * 16000)]
    second = [synth.tone_clip(5, 3 * 16000)]
    for k, clips in enumerate((first, second)):
        wave, so = synth.pack(clips)
        pl = ae.plan(np.diff(so))
        need = ae.lib().ae_workspace_bytes(m.handle, len(clips), int(pl["frame_off"][-1]),
                                           int(pl["token_off"][-1]))
        assert need <= ae.STATIC_SCRATCH_BYTES, need
        wd = torch.from_numpy(wave).cuda()
        want = ae.encode(m, wd, so)
        got = ae.encode_static(m, wd, so)
        torch.cuda.synchronize()
        say(f"    call {k + 1}: {got.shape[0]} tokens, workspace {need} bytes")
        assert got.shape == want.shape
        assert torch.equal(got, want), float((got - want).abs().max())
    # the second (smaller) call's clip against the oracle as well
    bf16_gate(got.cpu().numpy(), oracle.encode_clips(second, W)[0], "3 s clip")


def test_static_scratch_fp32_one_clip_and_capacity():
    say("[gpu] encode_static: fp32 one 1 s clip vs oracle; a batch beyond the scratch refused")
    W = weights(1)
    m = ae.Model(W, dtype="f32")
    x = synth.tone_clip(0)
    wave, so = synth.pack([x])
    got = ae.encode_static(m, torch.from_numpy(wave).cuda(), so).cpu().numpy()
    want = oracle.encode_clips([x], W, layers=1)[0]
    assert got.shape == (25, 512) and rel_l2(got, want) <= 1e-4, rel_l2(got, want)
    big = [synth.white_clip(i, 480000) for i in range(4)]
    wave, so = synth.pack(big)
    with pytest.raises(ae.AeError) as e:
        ae.encode_static(m, torch.from_numpy(wave).cuda(), so)
    assert e.value.status == ae.AE_ERR_CAPACITY
