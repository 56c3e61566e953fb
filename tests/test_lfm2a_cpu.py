"""CPU checks of the LFM2A entry points of the C-ABI library: the host-only
size functions agree bit-exactly with the oracle's, and argument errors
are reported before any device work (no call here touches a GPU)."""
import ctypes as C

import numpy as np
import pytest

from oracle import lfm2a as O
from log_mel_conformer_amd import ae, lfm2a

I64 = C.POINTER(C.c_int64)


def test_counts_match_oracle():
    for n in list(range(0, 2000)) + list(range(479000, 481000, 7)) + [10 ** 7]:
        assert lfm2a.num_frames(n) == O.num_frames(n), n
        assert lfm2a.num_tokens(n) == O.num_tokens(n), n
    assert lfm2a.num_frames(-3) == 0 and lfm2a.num_tokens(-3) == 0


def test_plan_prefix_sums_and_refusals():
    lens = [0, 320, 16000, 480000, 7777]
    p = lfm2a.plan(lens)
    assert np.array_equal(p["sample_off"], np.concatenate([[0], np.cumsum(lens)]))
    assert np.array_equal(p["frame_off"],
                          np.concatenate([[0], np.cumsum([O.num_frames(n) for n in lens])]))
    assert np.array_equal(p["token_off"],
                          np.concatenate([[0], np.cumsum([O.num_tokens(n) for n in lens])]))
    for bad, status in (([500, -1], ae.AE_ERR_INVALID), ([16000, 319], ae.AE_ERR_SHAPE),
                        ([1], ae.AE_ERR_SHAPE)):
        with pytest.raises(ae.AeError) as e:
            lfm2a.plan(bad)
        assert e.value.status == status, bad
    # the oracle refuses the same clips: fewer than two statistics frames
    with pytest.raises(O.RefusedClip):
        O.log_mel(np.ones(319))
    O.log_mel(np.ones(320))


def test_default_config():
    c = lfm2a.default_config()
    assert (c.n_mel, c.stem_ch, c.n_embd, c.n_head, c.n_ff, c.n_layer, c.conv_kernel, c.pos_dim,
            c.adapter, c.llm_hidden) == (128, 256, 512, 8, 2048, 17, 9, 512, 2048, 2048)
    assert abs(c.eps - 1e-5) < 1e-12


def _fake_weights(n_layer):
    fake = C.c_void_p(0x10000)
    blocks = (lfm2a.BlockWeights * n_layer)()
    for i in range(n_layer):
        for n in lfm2a.BLOCK_FIELDS:
            setattr(blocks[i], n, fake)
    W = lfm2a.Weights()
    for i in range(5):
        W.stem_w[i] = fake
        W.stem_b[i] = fake
    for f in ("pre_encode_out_w", "pre_encode_out_b", "adapter_norm_w", "adapter_norm_b",
              "adapter_up_w", "adapter_up_b", "adapter_down_w", "adapter_down_b"):
        setattr(W, f, fake)
    W.blocks = blocks
    return W


def _create(cfg, W, dt=ae.AE_BF16):
    h = C.c_void_p()
    return lfm2a.lib().lfm2a_model_create(C.byref(cfg), C.byref(W), dt, None, C.byref(h)), h


def test_model_create_refuses_before_device_work():
    cfg = lfm2a.default_config(n_layer=2)
    st, h = _create(lfm2a.default_config(n_layer=2, n_embd=1024), _fake_weights(2))
    assert st == ae.AE_ERR_UNSUPPORTED and h.value is None
    assert _create(cfg, _fake_weights(2), ae.AE_F32)[0] == ae.AE_ERR_UNSUPPORTED
    W = _fake_weights(2)
    W.blocks[1].pos_bias_v = None
    st, _ = _create(cfg, W)
    assert st == ae.AE_ERR_INVALID and b"block 1" in ae.lib().ae_last_error()
    W = _fake_weights(2)
    W.stem_w[3] = None
    assert _create(cfg, W)[0] == ae.AE_ERR_INVALID
    # weights and biases are read with 16-byte loads: a misaligned one is refused
    W = _fake_weights(2)
    W.blocks[0].ffn_up_b = C.c_void_p(0x10004)
    st, _ = _create(cfg, W)
    assert st == ae.AE_ERR_INVALID and b"16-byte" in ae.lib().ae_last_error()


def test_calls_refuse_before_device_work():
    L = lfm2a.lib()
    fake = C.c_void_p(0x10000)
    so = np.array([0, 16000], np.int64)
    assert L.lfm2a_logmel(fake, so.ctypes.data_as(I64), 1, fake, fake, 8, None) == ae.AE_ERR_CAPACITY
    short = np.array([0, 100], np.int64)
    assert L.lfm2a_logmel(fake, short.ctypes.data_as(I64), 1, fake, fake, 1 << 20,
                          None) == ae.AE_ERR_SHAPE
    bad = np.array([0, 1000, 500], np.int64)
    assert L.lfm2a_logmel(fake, bad.ctypes.data_as(I64), 2, fake, fake, 1 << 20,
                          None) == ae.AE_ERR_INVALID
    empty = np.array([0, 0, 0], np.int64)
    assert L.lfm2a_logmel(None, empty.ctypes.data_as(I64), 2, None, None, 0, None) == ae.AE_OK
    to = np.array([0, 10], np.int64)
    assert L.lfm2a_block(None, 0, fake, to.ctypes.data_as(I64), 1, fake, 1 << 20,
                         None) == ae.AE_ERR_INVALID
    # the attention kernel: t_max below the longest clip, then a short workspace
    assert L.lfm2a_xl_attention(fake, fake, 5, fake, fake, to.ctypes.data_as(I64), 1, fake, fake,
                                1 << 20, None) == ae.AE_ERR_SHAPE
    assert L.lfm2a_xl_attention(fake, fake, 10, fake, fake, to.ctypes.data_as(I64), 1, fake,
                                fake, 4, None) == ae.AE_ERR_CAPACITY
    assert L.lfm2a_attention_workspace_bytes(4) >= 80


def test_timing_classes_cover_the_lfm2a_kernels():
    assert len(ae.KERNEL_CLASSES) == 28 and ae.KERNEL_CLASSES[-1] == "lfm_dwconv"
    assert ae.lib().ae_timing_enable(27) == ae.AE_OK
    assert ae.lib().ae_timing_enable(28) == ae.AE_ERR_INVALID
    assert ae.lib().ae_timing_enable(-1) == ae.AE_OK
