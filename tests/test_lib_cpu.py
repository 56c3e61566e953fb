"""CPU checks of the C-ABI library: it loads, exports every symbol
include/ae.h and include/lfm2a.h declare, its host-only functions agree bit-exactly with the
oracle's integer functions, and argument errors are reported before any
device work (no call here touches a GPU)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

import oracle
from log_mel_conformer_amd import ae

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    names = set()
    inc = os.path.join(ROOT, "include")
    for h in sorted(os.listdir(inc)):
        if h.endswith(".h"):
            src = re.sub(r"/\*.*?\*/", "", open(os.path.join(inc, h)).read(), flags=re.S)
            names |= set(re.findall(r"\b((?:ae|lfm2a)_[a-z_0-9]+)\s*\(", src))
    return sorted(names)


def test_library_exports_every_declared_symbol():
    L = ae.lib()
    names = _declared()
    assert len(names) >= 30 and "lfm2a_encode" in names, names
    for n in names:
        assert hasattr(L, n), n


def test_counts_match_oracle():
    for n in list(range(0, 3000)) + list(range(470000, 490000, 7)) + [10 ** 7, -5]:
        assert ae.num_frames(n) == (oracle.num_frames(n) if n >= 0 else 0), n
        assert ae.num_tokens(n) == (oracle.num_tokens(n) if n >= 0 else 0), n


def test_plan_prefix_sums():
    lens = [100, 161, 16000, 560000, 0, 72825]
    p = ae.plan(lens)
    F = [oracle.num_frames(n) for n in lens]
    T = [oracle.num_tokens(n) for n in lens]
    assert np.array_equal(p["frame_off"], np.concatenate([[0], np.cumsum(F)]))
    assert np.array_equal(p["token_off"], np.concatenate([[0], np.cumsum(T)]))
    assert np.array_equal(p["sample_off"], np.concatenate([[0], np.cumsum(np.minimum(lens, 480000))]))
    assert np.array_equal(p["row_off"], np.concatenate([[0], np.cumsum([-(-f // 2) for f in F])]))
    with pytest.raises(ae.AeError) as e:
        ae.plan([5, -1])
    assert e.value.status == ae.AE_ERR_INVALID


def _fake_weights(cfg):
    """A weight table whose pointers are never dereferenced (validation
    fails before any device work)."""
    layers = (ae.LayerWeights * cfg.layers)()
    fake = C.c_void_p(0x10000)
    for i in range(cfg.layers):
        for name, typ in ae.LAYER_FIELDS:
            if typ is ae.Clip:
                setattr(layers[i], name, ae.Clip(-8, 8, -8, 8))
            else:
                setattr(layers[i], name, fake)
    W = ae.Weights()
    for f in ("conv0", "ln0", "conv1", "ln1", "in_proj", "out_proj", "out_bias", "embed"):
        setattr(W, f, fake)
    W.layers = layers
    return W


def _create(cfg, W):
    h = C.c_void_p()
    st = ae.lib().ae_model_create(C.byref(cfg), C.byref(W), ae.AE_BF16, None, C.byref(h))
    return st, h


def test_model_create_refuses_before_device_work():
    cfg = ae.default_config(layers=1, ctx_right=1)
    st, h = _create(cfg, _fake_weights(cfg))
    assert st == ae.AE_ERR_UNSUPPORTED and h.value is None
    assert b"context_right" in ae.lib().ae_last_error()
    cfg = ae.default_config(layers=1, hidden=512)
    assert _create(cfg, _fake_weights(cfg))[0] == ae.AE_ERR_UNSUPPORTED
    cfg = ae.default_config(layers=1)
    W = _fake_weights(cfg)
    W.layers[0].v = None
    st, _ = _create(cfg, W)
    assert st == ae.AE_ERR_INVALID and b"layer 0: weight v" in ae.lib().ae_last_error()
    W = _fake_weights(cfg)
    W.layers[0].q_clip = ae.Clip(1.0, -1.0, -8, 8)
    assert _create(cfg, W)[0] == ae.AE_ERR_INVALID


def test_logmel_refuses_small_workspace_before_device_work():
    so = np.array([0, 16000], np.int64)
    fake = C.c_void_p(0x10000)
    st = ae.lib().ae_logmel(fake, so.ctypes.data_as(C.POINTER(C.c_int64)), 1, fake, fake, 8, None)
    assert st == ae.AE_ERR_CAPACITY
    bad = np.array([0, 100, 50], np.int64)
    st = ae.lib().ae_logmel(fake, bad.ctypes.data_as(C.POINTER(C.c_int64)), 2, fake, fake, 1 << 20, None)
    assert st == ae.AE_ERR_INVALID
    # clips of <= 160 samples have no frames: nothing to do, not an error
    tiny = np.array([0, 160, 200], np.int64)
    st = ae.lib().ae_logmel(None, tiny.ctypes.data_as(C.POINTER(C.c_int64)), 2, None, None, 0, None)
    assert st == ae.AE_OK


def test_timing_class_validation():
    assert ae.lib().ae_timing_enable(99) == ae.AE_ERR_INVALID
    assert ae.lib().ae_timing_enable(-1) == ae.AE_OK


def test_resampled_length_matches_oracle():
    from oracle import resample as ors
    L = ae.lib()
    for fr in (8000, 11025, 16000, 22050, 44100, 44099, 48000, 96000, 384000, 7):
        for n in (0, 1, 2, 3, 160, 44099, 48000, 1440000, 123457):
            assert L.ae_resampled_length(n, fr, 16000) == ors.resampled_length(n, fr, 16000)
    assert L.ae_resampled_length(-1, 48000, 16000) == -1
    assert L.ae_resampled_length(10, 0, 16000) == -1


def test_resampler_create_refuses_bad_rates_before_any_device_work():
    import ctypes as C
    L = ae.lib()
    h = C.c_void_p()
    for fr, to in ((0, 16000), (48000, -1), (768001, 16000)):
        assert L.ae_resampler_create(fr, to, None, C.byref(h)) == ae.AE_ERR_INVALID
        assert h.value is None
    assert L.ae_resample_workspace_bytes(4, 1000, 1) == 256
    assert L.ae_resample_workspace_bytes(4, 1000, 2) == 256 + 4096


def test_expand_ids_matches_oracle():
    from oracle import placeholders as ph
    rng = np.random.default_rng(4)
    A = ph.AUDIO_TOKEN
    for _ in range(100):
        k = int(rng.integers(0, 4))
        body = list(rng.integers(3, 5000, int(rng.integers(0, 20))))
        for _ in range(k):
            body.insert(int(rng.integers(0, len(body) + 1)), A)
        n = list(rng.integers(0, 800, k))
        want = ph.expand_ids(body, n, bos=2, eos=1, max_tokens=10 ** 6)
        got = ae.expand_ids(body, n, bos=2, eos=1, max_tokens=10 ** 6)
        assert got.tolist() == want


def test_expand_ids_refusals():
    A = ae.RELEASE_AUDIO
    with pytest.raises(ae.AeError) as e:
        ae.expand_ids([5, A], [3, 4], bos=2, eos=1, max_tokens=100)
    assert e.value.status == ae.AE_ERR_SHAPE
    with pytest.raises(ae.AeError) as e:
        ae.expand_ids([A], [98], bos=2, eos=1, max_tokens=100)
    assert e.value.status == ae.AE_ERR_CAPACITY
    assert len(ae.expand_ids([A], [96], bos=2, eos=1, max_tokens=100)) == 100


def test_plan_frames_matches_oracle():
    """ae_plan_frames / lfm2a_plan_frames: conv0-row and token prefix sums
    from frame offsets, bit-exact with the oracle's counts."""
    from log_mel_conformer_amd import lfm2a
    from oracle import lfm2a as olfm
    lens = [100, 161, 16000, 480000, 0, 72825, 641]
    fo = np.concatenate([[0], np.cumsum([oracle.num_frames(n) for n in lens])])
    p = ae.plan_frames(fo)
    assert np.array_equal(p["token_off"], np.concatenate([[0], np.cumsum([oracle.num_tokens(n) for n in lens])]))
    assert np.array_equal(p["row_off"], ae.plan(lens)["row_off"])
    assert np.array_equal(ae.plan_frames([0])["token_off"], [0])
    for bad in ([1, 5], [0, 5, 3], [0, 3000]):
        with pytest.raises(ae.AeError):
            ae.plan_frames(bad)
    llens = [0, 320, 16000, 480000, 12345]
    lfo = np.concatenate([[0], np.cumsum([olfm.num_frames(n) for n in llens])])
    assert np.array_equal(lfm2a.plan_frames(lfo),
                          np.concatenate([[0], np.cumsum([olfm.num_tokens(n) for n in llens])]))
    with pytest.raises(ae.AeError):
        lfm2a.plan_frames([0, 4, 2])


def test_binding_refuses_bad_tensors_before_any_call():
    """Host tensors, the wrong dtype, strided views, short buffers and bad
    offsets raise AeError in the binding, before the library sees a pointer
    (a kernel handed any of them would read or write out of bounds)."""
    import torch
    from log_mel_conformer_amd import lfm2a

    class _Cfg:
        hidden, out_dim, n_embd, llm_hidden = 1024, 512, 512, 2048

    class _M:
        cfg = _Cfg()
        handle = None

    so = np.array([0, 16000])
    cases = [
        lambda: ae.logmel(torch.zeros(16000), so),                               # host tensor
        lambda: ae.logmel(np.zeros(16000, np.float32), so),                      # not a tensor
        lambda: ae.logmel(torch.zeros(16000, dtype=torch.float64), so),          # dtype
        lambda: ae.logmel(torch.zeros(16000), [0, 200, 100]),                    # decreasing
        lambda: ae.logmel(torch.zeros(16000), [5, 16000]),                       # not from 0
        lambda: ae.encode(_M(), torch.zeros(16000), so),
        lambda: ae.encode_static(_M(), torch.zeros(16000), so),
        lambda: ae.subsample(_M(), torch.zeros((99, 128)), [0, 99]),
        lambda: ae.conformer_layer(_M(), 0, torch.zeros((25, 1024)), torch.zeros(25, dtype=torch.int32)),
        lambda: ae.conformer_layer(_M(), 0, torch.zeros(25), torch.zeros(25, dtype=torch.int32)),
        lambda: ae.mixdown(torch.zeros(10), 2),
        lambda: lfm2a.logmel(torch.zeros(16000), so),
        lambda: lfm2a.encode(_M(), torch.zeros(16000), so),
        lambda: lfm2a.adapter(_M(), torch.zeros((4, 512))),
    ]
    for i, f in enumerate(cases):
        with pytest.raises(ae.AeError):
            f()
    # the checks themselves: contiguity, size and shape
    t = torch.zeros((8, 8))
    with pytest.raises(ae.AeError):
        ae._dev(t, "t", torch.float32)                    # host tensor refused first
