"""Pins of the LFM2A oracle (oracle.lfm2a) against things other than itself:
library routines (scipy's window and filter, torch's stft, conv2d, conv1d,
layer_norm, gelu and attention, all on the CPU in float64), closed forms,
brute-force sums and invariants. Source of the method: the docs.rs source
page of cera 0.5.3, src/model/audio_encoder_gpu.rs.
"""
import math

import numpy as np
import pytest
import scipy.signal

from oracle import lfm2a as L

torch = pytest.importorskip("torch")
F = torch.nn.functional


def t64(x):
    return torch.as_tensor(np.asarray(x, dtype=np.float64))


# ------------------------------------------------------------------ sizes

def test_sizes():
    assert [L.num_frames(n) for n in (0, 1, 159, 160, 161, 480000)] == [0, 1, 1, 2, 2, 3001]
    assert [L.effective_frames(n) for n in (0, 159, 160, 480000)] == [0, 0, 1, 3000]
    # 3001 frames -> 1501 -> 751 -> 376 through the three stride-2 layers
    assert L.num_tokens(480000) == 376
    assert L.num_tokens(0) == 0 and L.num_tokens(1) == 1
    # the page's twiddle table, [N_FFT, 2] floats, is 4 KB
    assert L.N_FFT * 2 * 4 == 4096
    # its head geometry: n_embd 512 over 8 heads is 64 per head
    assert L.CONFIG["n_embd"] // L.CONFIG["n_head"] == 64


def test_conv_out_matches_torch():
    for h in (1, 2, 3, 7, 8, 100):
        for k, s, p in ((3, 2, 1), (1, 1, 0), (3, 1, 1)):
            x = torch.zeros(1, 1, h, 5, dtype=torch.float64)
            w = torch.zeros(1, 1, k, 1, dtype=torch.float64)
            assert F.conv2d(x, w, stride=(s, 1), padding=(p, 0)).shape[2] == L.conv_out(h, k, s, p)


# -------------------------------------------------------------- front end

def test_hann_is_scipy_periodic_hann():
    assert np.allclose(L.hann_periodic(400), scipy.signal.get_window("hann", 400, fftbins=True),
                       rtol=0, atol=1e-15)
    w = L.padded_window()
    assert w.shape == (512,) and np.all(w[:56] == 0) and np.all(w[456:] == 0)


def test_preemphasis_is_a_first_order_fir():
    x = np.random.default_rng(0).standard_normal(1000)
    assert np.allclose(L.preemphasis(x), scipy.signal.lfilter([1.0, -0.97], [1.0], x),
                       rtol=0, atol=1e-13)


@pytest.mark.parametrize("n", [1, 159, 160, 400, 4000, 4321])
def test_power_spectrum_matches_torch_stft(n):
    """Frames, centring, window and DFT against torch.stft (center, zero
    padding, the 400-point window centred in 512)."""
    x = np.random.default_rng(n).standard_normal(n)
    got = L.power_spectrum(L.stft_frames(x))
    y = t64(L.preemphasis(x))
    win = torch.hann_window(400, periodic=True, dtype=torch.float64)
    X = torch.stft(y, n_fft=512, hop_length=160, win_length=400, window=win, center=True,
                   pad_mode="constant", return_complex=True)
    want = (X.abs() ** 2).T.numpy()
    assert got.shape == want.shape == (L.num_frames(n), 257)
    assert np.allclose(got, want, rtol=1e-10, atol=1e-10)


def test_power_spectrum_brute_force_and_parseval():
    fr = np.random.default_rng(1).standard_normal((2, 512))
    P = L.power_spectrum(fr)
    n = np.arange(512)
    for k in (0, 1, 77, 255, 256):
        X = np.sum(fr[0] * np.exp(-2j * np.pi * k * n / 512))
        assert abs(P[0, k] - abs(X) ** 2) < 1e-8 * max(1.0, abs(X) ** 2)
    # Parseval for a real signal: sum x^2 = (P0 + 2 sum_{1..255} Pk + P256) / N
    e = (P[1, 0] + 2 * P[1, 1:256].sum() + P[1, 256]) / 512
    assert abs(e - np.sum(fr[1] ** 2)) < 1e-9 * e


def test_slaney_mel_scale_closed_forms():
    assert L.hz_to_mel(0.0) == 0.0
    assert abs(L.hz_to_mel(200.0) - 3.0) < 1e-12
    assert abs(L.hz_to_mel(1000.0) - 15.0) < 1e-12
    assert abs(L.hz_to_mel(6400.0) - 42.0) < 1e-12        # one factor 6.4 above 1 kHz
    f = np.array([0.0, 55.0, 999.0, 1000.0, 1234.5, 8000.0])
    assert np.allclose(L.mel_to_hz(L.hz_to_mel(f)), f, rtol=1e-13, atol=1e-9)


def test_mel_filterbank_triangles():
    fb = L.mel_filterbank()
    assert fb.shape == (128, 257) and np.all(fb >= 0)
    edges = L.mel_to_hz(np.linspace(0.0, L.hz_to_mel(8000.0), 130))
    freqs = np.arange(257) * 16000 / 512
    for m in (0, 1, 5, 40, 90, 127):
        lo, c, hi = edges[m:m + 3]
        # the triangle as a piecewise-linear interpolant through its corners
        want = np.interp(freqs, [lo, c, hi], [0.0, 2.0 / (hi - lo), 0.0], left=0.0, right=0.0)
        assert np.allclose(fb[m], want, rtol=1e-12, atol=1e-15), m
        assert np.count_nonzero(fb[m]) >= 1
    # unit area in Hz: the bin-sampled sum of wide triangles is close to 1
    area = fb[100:].sum(axis=1) * (16000 / 512)
    assert np.all(np.abs(area - 1.0) < 0.02)


def test_log_mel_tone_peaks_at_its_band():
    sr = 16000
    for f0 in (440.0, 1000.0, 3000.0):
        x = np.sin(2 * np.pi * f0 * np.arange(sr) / sr)
        raw = L.log_mel_raw(x)
        edges = L.mel_to_hz(np.linspace(0.0, L.hz_to_mel(8000.0), 130))
        centre = edges[1:-1]
        band = int(np.argmax(raw[50]))
        assert abs(centre[band] - f0) <= 0.5 * (edges[band + 2] - edges[band]), (f0, band)


def test_normalize_per_bin_statistics():
    rng = np.random.default_rng(3)
    mel = rng.standard_normal((50, 128)) * 3 + 7
    out = L.normalize_per_bin(mel, 40)
    sd = mel[:40].std(axis=0, ddof=1)
    assert np.allclose(out[:40].mean(axis=0), 0.0, atol=1e-12)
    assert np.allclose(out[:40].std(axis=0, ddof=1), sd / (sd + 1e-5), rtol=1e-12)
    assert np.all(out[40:] == 0)
    with pytest.raises(L.RefusedClip):
        L.normalize_per_bin(mel, 1)
    with pytest.raises(L.RefusedClip):
        L.log_mel(np.ones(300))             # one statistics frame only


# ------------------------------------------------------------------- stem

@pytest.mark.parametrize("cin,cout,groups,k,s,p,h,w", [
    (1, 6, 1, 3, 2, 1, 9, 10), (4, 4, 4, 3, 2, 1, 7, 8), (5, 3, 1, 1, 1, 0, 4, 6),
    (6, 6, 6, 3, 1, 1, 5, 5), (2, 4, 2, 3, 2, 1, 1, 3)])
def test_conv2d_matches_torch(cin, cout, groups, k, s, p, h, w):
    rng = np.random.default_rng(cin * 100 + cout)
    x = rng.standard_normal((cin, h, w))
    wt = rng.standard_normal((cout, cin // groups, k, k))
    b = rng.standard_normal(cout)
    want = F.conv2d(t64(x)[None], t64(wt), t64(b), stride=s, padding=p, groups=groups)[0]
    assert np.allclose(L.conv2d(x, wt, b, s, p, groups), want.numpy(), rtol=1e-12, atol=1e-12)
    if groups == cin == cout:
        assert np.allclose(L.depthwise_conv2d(x, wt, b, s, p), want.numpy(), rtol=1e-12,
                           atol=1e-12)


def _tiny_stem(rng, n_mel, ch):
    shapes = [(ch, 1, 3, 3), (ch, 1, 3, 3), (ch, ch, 1, 1), (ch, 1, 3, 3), (ch, ch, 1, 1)]
    return [(rng.standard_normal(s) * 0.5, rng.standard_normal(s[0]) * 0.1) for s in shapes]


@pytest.mark.parametrize("frames", [1, 2, 5, 17, 40])
def test_conv_stem_against_torch_ops(frames):
    """The stem as torch conv2d calls with the page's modes, and the
    (channel, time, freq) -> (time, channel freq) flatten."""
    rng = np.random.default_rng(frames)
    n_mel, ch, d = 16, 4, 8
    W = {"stem": _tiny_stem(rng, n_mel, ch),
         "pre_encode_out_w": rng.standard_normal((d, ch * 2)),
         "pre_encode_out_b": rng.standard_normal(d)}
    feat = rng.standard_normal((frames, n_mel))
    x = t64(feat)[None, None]
    for i, (w, b) in enumerate(W["stem"]):
        dw, s, p = L.STEM_LAYER_MODES[i]
        x = F.conv2d(x, t64(w), t64(b), stride=s, padding=p, groups=x.shape[1] if dw else 1)
        if L.STEM_RELU_AFTER[i]:
            x = torch.relu(x)
    x = x[0].permute(1, 0, 2).reshape(x.shape[2], -1)
    want = F.linear(x, t64(W["pre_encode_out_w"]), t64(W["pre_encode_out_b"])).numpy()
    got = L.conv_stem(feat, W)
    assert got.shape == want.shape
    assert got.shape[0] == L.num_tokens((frames - 1) * 160 + 1)   # frames = 1 + n // 160
    assert np.allclose(got, want, rtol=1e-11, atol=1e-11)


# ----------------------------------------------------------------- blocks

def test_elementwise_and_layer_norm_against_torch():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((7, 33)) * 4
    w, b = rng.standard_normal(33), rng.standard_normal(33)
    assert np.allclose(L.layer_norm(x, w, b), F.layer_norm(t64(x), (33,), t64(w), t64(b),
                                                           eps=1e-5).numpy(), rtol=1e-12,
                       atol=1e-12)
    assert np.allclose(L.gelu_erf(x), F.gelu(t64(x)).numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(L.silu(x), F.silu(t64(x)).numpy(), rtol=1e-12, atol=1e-14)
    assert np.allclose(L.sigmoid(x), torch.sigmoid(t64(x)).numpy(), rtol=1e-12, atol=1e-15)


def test_relative_pos_emb_closed_form():
    t, d = 6, 8
    pe = L.relative_pos_emb(t, d)
    assert pe.shape == (11, 8)
    assert np.allclose(pe[t - 1], [0, 1] * 4)                   # position 0
    for r in range(2 * t - 1):
        p = t - 1 - r
        for i in range(d // 2):
            w = 10000.0 ** (-2 * i / d)
            assert abs(pe[r, 2 * i] - math.sin(p * w)) < 1e-14
            assert abs(pe[r, 2 * i + 1] - math.cos(p * w)) < 1e-14


def test_xl_attention_without_position_term_is_plain_attention():
    rng = np.random.default_rng(6)
    t, H, hd = 9, 2, 4
    q, k, v = (rng.standard_normal((t, H * hd)) for _ in range(3))
    u, bv = rng.standard_normal(H * hd), rng.standard_normal(H * hd)
    got = L.xl_attention(q, k, v, np.zeros((2 * t - 1, H * hd)), u, bv, H)
    hq = lambda a: t64(a).reshape(t, H, hd).transpose(0, 1)
    want = F.scaled_dot_product_attention(hq(q + u), hq(k), hq(v)).transpose(0, 1).reshape(t, -1)
    assert np.allclose(got, want.numpy(), rtol=1e-12, atol=1e-12)


def test_xl_attention_relative_term_brute_force():
    """Scores rebuilt from the position value i - j itself: the sinusoid
    evaluated at i - j, projected, dotted with q_i + v."""
    rng = np.random.default_rng(7)
    t, H, hd, dp = 7, 2, 4, 6
    q, k, v = (rng.standard_normal((t, H * hd)) for _ in range(3))
    u, bv = rng.standard_normal(H * hd), rng.standard_normal(H * hd)
    Wp = rng.standard_normal((H * hd, dp))
    p = L.relative_pos_emb(t, dp) @ Wp.T
    got = L.xl_attention(q, k, v, p, u, bv, H)

    def sinus(pos):
        return np.array([f(pos * 10000.0 ** (-2 * (c // 2) / dp))
                         for c, f in zip(range(dp), [math.sin, math.cos] * dp)])

    want = np.zeros((t, H * hd))
    for h in range(H):
        sl = slice(h * hd, (h + 1) * hd)
        for i in range(t):
            s = np.array([((q[i, sl] + u[sl]) @ k[j, sl]
                           + (q[i, sl] + bv[sl]) @ (Wp @ sinus(i - j))[sl]) / math.sqrt(hd)
                          for j in range(t)])
            e = np.exp(s - s.max())
            want[i, sl] = (e / e.sum()) @ v[:, sl]
    assert np.allclose(got, want, rtol=1e-11, atol=1e-12)


def test_xl_attention_position_one_means_previous_token():
    """A position term that is large only at relative position +1 makes
    every query copy the key just before it."""
    t, hd = 6, 4
    q = np.zeros((t, hd)); k = np.zeros((t, hd))
    v = np.arange(t, dtype=np.float64)[:, None] * np.ones((1, hd))
    bv = np.array([1.0, 0, 0, 0])
    p = np.zeros((2 * t - 1, hd))
    p[t - 1 - 1, 0] = 200.0                      # the row of position +1
    out = L.xl_attention(q, k, v, p, np.zeros(hd), bv, 1)
    assert np.allclose(out[1:, 0], np.arange(t - 1), atol=1e-9)
    assert abs(out[0, 0] - np.mean(np.arange(t))) < 1e-9     # no key before token 0


@pytest.mark.parametrize("k", [9, 4, 1])
def test_depthwise_conv1d_against_torch(k):
    rng = np.random.default_rng(k)
    t, d = 11, 5
    x, w, b = rng.standard_normal((t, d)), rng.standard_normal((d, k)), rng.standard_normal(d)
    lo = (k - 1) // 2
    xp = F.pad(t64(x).T[None], (lo, k - 1 - lo))
    want = F.conv1d(xp, t64(w)[:, None, :], t64(b), groups=d)[0].T.numpy()
    assert np.allclose(L.depthwise_conv1d(x, w, b), want, rtol=1e-12, atol=1e-12)


def _block(rng, d, ff, k, scale=0.2):
    B = {}
    for nm in ("ffn_norm", "ln1", "norm_conv", "ffn_norm_1", "ln2"):
        B[nm + "_w"] = 1 + 0.1 * rng.standard_normal(d)
        B[nm + "_b"] = 0.1 * rng.standard_normal(d)
    for nm, shape in (("ffn_up", (ff, d)), ("ffn_down", (d, ff)), ("ffn_up_1", (ff, d)),
                      ("ffn_down_1", (d, ff)), ("attn_q", (d, d)), ("attn_k", (d, d)),
                      ("attn_v", (d, d)), ("attn_o", (d, d)), ("conv_pw1", (2 * d, d)),
                      ("conv_pw2", (d, d))):
        B[nm + "_w"] = scale * rng.standard_normal(shape)
        B[nm + "_b"] = 0.1 * rng.standard_normal(shape[0])
    B["linear_pos_w"] = scale * rng.standard_normal((d, d))
    B["pos_bias_u"] = 0.1 * rng.standard_normal(d)
    B["pos_bias_v"] = 0.1 * rng.standard_normal(d)
    B["conv_dw_w"] = scale * rng.standard_normal((d, k))
    B["conv_dw_b"] = 0.1 * rng.standard_normal(d)
    B["conv_norm_w"] = 1 + 0.1 * rng.standard_normal(d)
    B["conv_norm_b"] = 0.1 * rng.standard_normal(d)
    return B


def test_block_with_silent_branches_is_its_final_norm():
    rng = np.random.default_rng(8)
    d, t = 8, 5
    B = _block(rng, d, 16, 3)
    for nm in ("ffn_down", "ffn_down_1", "attn_o", "conv_pw2"):
        B[nm + "_w"] = np.zeros_like(B[nm + "_w"])
        B[nm + "_b"] = np.zeros_like(B[nm + "_b"])
    x = rng.standard_normal((t, d))
    pe = L.relative_pos_emb(t, d)
    want = F.layer_norm(t64(x), (d,), t64(B["ln2_w"]), t64(B["ln2_b"]), eps=1e-5).numpy()
    assert np.allclose(L.conformer_block(x, B, pe, 2), want, rtol=1e-12, atol=1e-12)


def test_block_against_torch_composition():
    """The whole block as torch CPU ops: layer_norm, linear, silu,
    sigmoid, conv1d and the attention rebuilt from scores."""
    rng = np.random.default_rng(9)
    d, H, t, k = 8, 2, 6, 3
    B = _block(rng, d, 16, k)
    x = rng.standard_normal((t, d))
    pe = L.relative_pos_emb(t, d)
    T = {n: t64(a) for n, a in B.items()}
    ln = lambda a, nm: F.layer_norm(a, (d,), T[nm + "_w"], T[nm + "_b"], eps=1e-5)
    lin = lambda a, nm: F.linear(a, T[nm + "_w"], T[nm + "_b"])

    def ffn(a, s):
        return a + 0.5 * lin(F.silu(lin(ln(a, "ffn_norm" + s), "ffn_up" + s)), "ffn_down" + s)

    h = ffn(t64(x), "")
    n = ln(h, "ln1")
    q, kk, v = lin(n, "attn_q"), lin(n, "attn_k"), lin(n, "attn_v")
    p = F.linear(t64(pe), T["linear_pos_w"])
    hd = d // H
    att = torch.zeros(t, d, dtype=torch.float64)
    for hh in range(H):
        sl = slice(hh * hd, (hh + 1) * hd)
        ac = (q[:, sl] + T["pos_bias_u"][sl]) @ kk[:, sl].T
        bd = torch.stack([torch.stack([(q[i, sl] + T["pos_bias_v"][sl]) @ p[t - 1 - i + j, sl]
                                       for j in range(t)]) for i in range(t)])
        att[:, sl] = torch.softmax((ac + bd) / math.sqrt(hd), dim=1) @ v[:, sl]
    h = h + lin(att, "attn_o")
    g = lin(ln(h, "norm_conv"), "conv_pw1")
    g = F.glu(g, dim=1)
    c = F.conv1d(F.pad(g.T[None], ((k - 1) // 2, k - 1 - (k - 1) // 2)), T["conv_dw_w"][:, None],
                 T["conv_dw_b"], groups=d)[0].T
    c = F.silu(c * T["conv_norm_w"] + T["conv_norm_b"])
    h = h + lin(c, "conv_pw2")
    h = ffn(h, "_1")
    want = ln(h, "ln2").numpy()
    assert np.allclose(L.conformer_block(x, B, pe, H), want, rtol=1e-11, atol=1e-11)


def test_adapter_against_torch():
    rng = np.random.default_rng(10)
    W = {"adapter_norm_w": rng.standard_normal(8), "adapter_norm_b": rng.standard_normal(8),
         "adapter_up_w": rng.standard_normal((12, 8)), "adapter_up_b": rng.standard_normal(12),
         "adapter_down_w": rng.standard_normal((5, 12)), "adapter_down_b": rng.standard_normal(5)}
    x = rng.standard_normal((4, 8))
    T = {n: t64(a) for n, a in W.items()}
    h = F.layer_norm(t64(x), (8,), T["adapter_norm_w"], T["adapter_norm_b"], eps=1e-5)
    h = F.gelu(F.linear(h, T["adapter_up_w"], T["adapter_up_b"]))
    want = F.linear(h, T["adapter_down_w"], T["adapter_down_b"]).numpy()
    assert np.allclose(L.adapter(x, W), want, rtol=1e-12, atol=1e-12)


def test_encode_tiny_clip_shapes():
    rng = np.random.default_rng(11)
    d, H = 8, 2
    W = {"stem": _tiny_stem(rng, 128, 4), "pre_encode_out_w": 0.1 * rng.standard_normal((d, 64)),
         "pre_encode_out_b": np.zeros(d), "blocks": [_block(rng, d, 16, 9) for _ in range(2)],
         "adapter_norm_w": np.ones(d), "adapter_norm_b": np.zeros(d),
         "adapter_up_w": rng.standard_normal((12, d)), "adapter_up_b": np.zeros(12),
         "adapter_down_w": rng.standard_normal((6, 12)), "adapter_down_b": np.zeros(6)}
    for n in (320, 1000, 8000):
        y = L.encode(rng.uniform(-0.5, 0.5, n), W, H)
        assert y.shape == (L.num_tokens(n), 6) and np.all(np.isfinite(y))
    assert L.encode(np.zeros(0), W, H).shape == (0, 6)
