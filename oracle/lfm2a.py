"""Oracle for the second encoder: the LFM2A Conformer audio encoder.

TEST INFRASTRUCTURE (see the package docstring). float64 storage and
accumulation (numpy). Matrices follow y = x W^T with W stored [out][in].

Source: the docs.rs source page of cera 0.5.3,
``src/model/audio_encoder_gpu.rs`` ("audio_encoder_gpu.rs" below): the
module documentation, ``GpuMelFrontend``, ``dft_twiddles``,
``log_mel_spectrogram_gpu``, ``STEM_LAYER_MODES``, ``STEM_RELU_AFTER``,
``Conv2dSpec::padded``, ``conv_stem_gpu``, ``encode_audio_gpu``,
``macaron_ffn`` and the ``AudioEncoderGpuOps`` method documentation
(layernorm, gelu_erf, scaled_add, conv2d, glu_split, chan_affine_silu,
xl_attention, stft_frames, power_spec, mel_project, mel_norm).

The page fixes the order of every step and the structure of each op; it
does not print the constants and helpers it imports from its CPU modules.
Those are taken here as follows (each is a reading, listed in the design
notes):
  * N_FFT = 512: the page's [N_FFT, 2] float twiddle table is 4 KB.
  * window: periodic Hann (the page) of WIN = 400 samples (25 ms), centred
    in the 512-wide buffer with zero flanks (the page: zero-flanked).
  * HOP = 160 (10 ms); center padding of N_FFT / 2 zeros on each side
    (the page: N_FFT / 2 per side), so a clip of n > 0 samples has
    1 + n // HOP frames, and the statistics use the first n // HOP of them.
  * pre-emphasis y[0] = x[0], y[n] = x[n] - 0.97 x[n-1], on the clip before
    the padding.
  * Slaney mel scale with Slaney area normalisation, 128 bands, 0..8 kHz.
  * log: ln(band + 2^-24).
  * per-bin normalisation: (x - mean) / (std + 1e-5), std with the n - 1
    divisor, over the first n // HOP frames; later frames are set to 0.
    A clip with fewer than two such frames has no defined std and is
    refused.
  * stem kernels 3x3 (the page's comments), 256 channels, so 128 mel bins
    leave 16 and the projection input is 256 * 16 = 4096 wide.
  * relative positions: row r of the (2t - 1)-row table is position
    t - 1 - r, entries sin(p w_i), cos(p w_i) interleaved with
    w_i = 10000^(-2i / 512); the score of query i and key j uses the row of
    position i - j (row t - 1 - i + j).
  * LayerNorm eps 1e-5; depthwise kernel 9; widths n_embd 512, 8 heads,
    n_ff 2048, 17 blocks, adapter 512 -> 2048 -> 2048.
Every function is pinned by a CPU test to a library routine, a closed form,
a brute-force sum or an invariant. What nothing here can pin is the set of
readings above against the page's own CPU modules, which the pages do not
hold: parity unpinned for those constants.
"""
from __future__ import annotations

import math

import numpy as np

SAMPLE_RATE = 16000
N_FFT = 512
N_BINS = N_FFT // 2 + 1
WIN = 400
HOP = 160
PREEMPH = 0.97
N_MEL = 128
LOG_MEL_EPS = 2.0 ** -24
NORM_EPS = 1e-5
LN_EPS = 1e-5
STEM_CH = 256
POS_EMB_DIM = 512

# (depthwise, stride, pad) of the five stem convolutions, and whether a
# ReLU follows each (audio_encoder_gpu.rs, STEM_LAYER_MODES and
# STEM_RELU_AFTER).
STEM_LAYER_MODES = [(False, 2, 1), (True, 2, 1), (False, 1, 0), (True, 2, 1), (False, 1, 0)]
STEM_RELU_AFTER = [True, False, True, False, True]

CONFIG = dict(n_embd=512, n_head=8, n_ff=2048, n_layer=17, conv_kernel=9,
              n_mel=N_MEL, adapter=2048, llm_hidden=2048)


class RefusedClip(ValueError):
    """A clip the per-bin statistics cannot be taken over."""


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------------ sizes

def num_frames(n: int) -> int:
    """STFT frames of an n-sample clip with N_FFT / 2 zeros of padding on
    each side: 0 for an empty clip, else 1 + n // HOP."""
    n = int(n)
    return 0 if n <= 0 else 1 + n // HOP


def effective_frames(n: int) -> int:
    """Frames the per-bin statistics are taken over: n // HOP."""
    return max(int(n), 0) // HOP


def conv_out(h: int, k: int, stride: int, pad: int) -> int:
    """Output length of one convolution axis (audio_encoder_gpu.rs,
    ``Conv2dSpec::padded``): (h + 2 pad - k) // stride + 1, or 0 when the
    kernel exceeds the padded input."""
    p = h + 2 * pad
    return 0 if p < k else (p - k) // stride + 1


def num_tokens(n: int) -> int:
    """Tokens after the stem: the frame count through the three stride-2
    3x3 convolutions (the 1x1 ones keep it)."""
    h = num_frames(n)
    for dw, s, p in STEM_LAYER_MODES:
        k = 1 if (not dw and s == 1) else 3
        h = conv_out(h, k, s, p) if h > 0 else 0
    return h


# -------------------------------------------------------------- front end

def hann_periodic(n: int) -> np.ndarray:
    """Periodic Hann window of n points: 0.5 - 0.5 cos(2 pi k / n)."""
    k = np.arange(n, dtype=np.float64)
    return 0.5 - 0.5 * np.cos(2.0 * np.pi * k / n)


def padded_window() -> np.ndarray:
    """The WIN-point periodic Hann centred in an N_FFT-wide buffer, zeros
    either side (audio_encoder_gpu.rs, ``GpuMelFrontend``: the window
    buffer)."""
    w = np.zeros(N_FFT)
    left = (N_FFT - WIN) // 2
    w[left:left + WIN] = hann_periodic(WIN)
    return w


def preemphasis(x) -> np.ndarray:
    """y[0] = x[0], y[n] = x[n] - PREEMPH x[n - 1]."""
    x = _f64(x)
    y = x.copy()
    y[1:] = x[1:] - PREEMPH * x[:-1]
    return y


def stft_frames(x) -> np.ndarray:
    """[F, N_FFT] windowed frames (audio_encoder_gpu.rs, ``stft_frames``):
    pre-emphasis, N_FFT / 2 zeros of padding each side, frame j = padded
    samples [j HOP, j HOP + N_FFT) times the padded window."""
    y = preemphasis(x)
    F = num_frames(len(y))
    pad = np.concatenate([np.zeros(N_FFT // 2), y, np.zeros(N_FFT // 2)])
    win = padded_window()
    out = np.zeros((F, N_FFT))
    for j in range(F):
        out[j] = pad[j * HOP:j * HOP + N_FFT] * win
    return out


def power_spectrum(frames) -> np.ndarray:
    """|X[k]|^2 on the N_BINS bins of each frame's DFT (audio_encoder_gpu.rs,
    ``power_spec``), X[k] = sum_n x[n] e^{-2 pi i k n / N_FFT}; numpy's real
    FFT evaluates the sum."""
    X = np.fft.rfft(_f64(frames), n=N_FFT, axis=-1)
    return X.real ** 2 + X.imag ** 2


def hz_to_mel(f):
    """Slaney mel scale: linear, 3 mel per 200 Hz, below 1 kHz; above it,
    15 mel plus 27 mel per factor 6.4 of frequency."""
    f = _f64(f)
    lin = f * 3.0 / 200.0
    log = 15.0 + np.log(np.maximum(f, 1e-300) / 1000.0) * 27.0 / math.log(6.4)
    return np.where(f >= 1000.0, log, lin)


def mel_to_hz(m):
    """Inverse of ``hz_to_mel``."""
    m = _f64(m)
    lin = m * 200.0 / 3.0
    log = 1000.0 * np.exp((m - 15.0) * math.log(6.4) / 27.0)
    return np.where(m >= 15.0, log, lin)


def mel_filterbank(n_mel: int = N_MEL) -> np.ndarray:
    """[n_mel, N_BINS] Slaney filter bank: n_mel + 2 edge frequencies evenly
    spaced in mel over 0..SAMPLE_RATE/2, triangle m rising from edge m to
    m + 1 and falling to m + 2 over the bin frequencies k SAMPLE_RATE /
    N_FFT, scaled by 2 / (edge m+2 - edge m) so each has unit area in Hz."""
    edges = mel_to_hz(np.linspace(hz_to_mel(0.0), hz_to_mel(SAMPLE_RATE / 2.0), n_mel + 2))
    f = np.arange(N_BINS) * SAMPLE_RATE / N_FFT
    fb = np.zeros((n_mel, N_BINS))
    for m in range(n_mel):
        lo, c, hi = edges[m], edges[m + 1], edges[m + 2]
        rise = (f - lo) / (c - lo)
        fall = (hi - f) / (hi - c)
        fb[m] = np.maximum(0.0, np.minimum(rise, fall)) * (2.0 / (hi - lo))
    return fb


def log_mel_raw(x) -> np.ndarray:
    """[F, N_MEL] ln(mel band power + LOG_MEL_EPS) before the normalisation
    (audio_encoder_gpu.rs, ``mel_project``, laid out time-major here)."""
    P = power_spectrum(stft_frames(x))
    return np.log(P @ mel_filterbank().T + LOG_MEL_EPS)


def normalize_per_bin(mel, n_eff: int) -> np.ndarray:
    """Per-mel-bin normalisation (audio_encoder_gpu.rs, ``mel_norm``): each
    bin's mean and std over the first n_eff frames, (x - mean) /
    (std + NORM_EPS); frames from n_eff on are 0."""
    mel = _f64(mel)
    if n_eff < 2:
        raise RefusedClip(f"{n_eff} frame(s) leave the per-bin std undefined")
    head = mel[:n_eff]
    mu = head.mean(axis=0)
    sd = np.sqrt(((head - mu) ** 2).sum(axis=0) / (n_eff - 1))
    out = np.zeros_like(mel)
    out[:n_eff] = (head - mu) / (sd + NORM_EPS)
    return out


def log_mel(x) -> np.ndarray:
    """The front end (audio_encoder_gpu.rs, ``log_mel_spectrogram_gpu``):
    [F, N_MEL] normalised log-mel features of one clip."""
    return normalize_per_bin(log_mel_raw(x), effective_frames(len(x)))


# ------------------------------------------------------------------- stem

def conv2d(x, w, b, stride: int, pad: int, groups: int) -> np.ndarray:
    """Direct 2D convolution (audio_encoder_gpu.rs, ``conv2d``):
    x [Cin, H, W], w [Cout, Cin/groups, kh, kw], b [Cout];
    out[o, y, z] = b[o] + sum over the group's input channels i and taps
    (dy, dz) of w[o, i, dy, dz] x[i, y s + dy - pad, z s + dz - pad],
    x zero outside its extent. Returns [Cout, Ho, Wo]."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    cin, H, W = x.shape
    cout, cpg, kh, kw = w.shape
    Ho, Wo = conv_out(H, kh, stride, pad), conv_out(W, kw, stride, pad)
    xp = np.zeros((cin, H + 2 * pad, W + 2 * pad))
    xp[:, pad:pad + H, pad:pad + W] = x
    out = np.repeat(b[:, None, None], Ho, axis=1).repeat(Wo, axis=2)
    opg = cout // groups
    for g in range(groups):
        xs = xp[g * cpg:(g + 1) * cpg]
        ws = w[g * opg:(g + 1) * opg]
        for dy in range(kh):
            for dz in range(kw):
                patch = xs[:, dy:dy + stride * (Ho - 1) + 1:stride,
                           dz:dz + stride * (Wo - 1) + 1:stride]      # [cpg, Ho, Wo]
                out[g * opg:(g + 1) * opg] += np.tensordot(ws[:, :, dy, dz], patch, axes=1)
    return out


def depthwise_conv2d(x, w, b, stride: int, pad: int) -> np.ndarray:
    """``conv2d`` with groups = channels, written per channel as a product
    of each shifted plane with its own tap."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    c, H, W = x.shape
    _, _, kh, kw = w.shape
    Ho, Wo = conv_out(H, kh, stride, pad), conv_out(W, kw, stride, pad)
    xp = np.zeros((c, H + 2 * pad, W + 2 * pad))
    xp[:, pad:pad + H, pad:pad + W] = x
    out = np.repeat(b[:, None, None], Ho, axis=1).repeat(Wo, axis=2)
    for dy in range(kh):
        for dz in range(kw):
            patch = xp[:, dy:dy + stride * (Ho - 1) + 1:stride, dz:dz + stride * (Wo - 1) + 1:stride]
            out += w[:, 0, dy, dz][:, None, None] * patch
    return out


def conv_stem(feat, W) -> np.ndarray:
    """Conv stem and input projection (audio_encoder_gpu.rs,
    ``conv_stem_gpu``): the [F, n_mel] features as one [1, F, n_mel] plane,
    the five convolutions of STEM_LAYER_MODES with ReLU after layers 0, 2
    and 4, the [C, t, f] result flattened to [t, C f] (channel-major inside
    a row), then pre_encode_out (with bias). Returns [t, n_embd]."""
    x = _f64(feat)[None]
    for (dw, s, p), relu, (w, b) in zip(STEM_LAYER_MODES, STEM_RELU_AFTER, W["stem"]):
        x = depthwise_conv2d(x, w, b, s, p) if dw else conv2d(x, w, b, s, p, 1)
        if relu:
            x = np.maximum(x, 0.0)
    C, t, f = x.shape
    flat = x.transpose(1, 0, 2).reshape(t, C * f)
    return flat @ _f64(W["pre_encode_out_w"]).T + _f64(W["pre_encode_out_b"])


# ----------------------------------------------------------------- blocks

def layer_norm(x, w, b, eps: float = LN_EPS) -> np.ndarray:
    """Affine LayerNorm over the last axis (audio_encoder_gpu.rs,
    ``layernorm``): (x - mean) / sqrt(biased variance + eps) * w + b."""
    x = _f64(x)
    mu = x.mean(axis=-1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=-1, keepdims=True)
    return (x - mu) / np.sqrt(var + eps) * _f64(w) + _f64(b)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-_f64(x)))


def silu(x):
    x = _f64(x)
    return x * sigmoid(x)


def gelu_erf(x):
    """GELU in its erf form (audio_encoder_gpu.rs, ``gelu_erf``):
    x/2 (1 + erf(x / sqrt 2))."""
    x = _f64(x)
    erf = np.vectorize(math.erf, otypes=[np.float64])
    return 0.5 * x * (1.0 + erf(x / math.sqrt(2.0)))


def linear(x, w, b=None):
    y = _f64(x) @ _f64(w).T
    return y if b is None else y + _f64(b)


def relative_pos_emb(t: int, d: int = POS_EMB_DIM) -> np.ndarray:
    """[2t - 1, d] sinusoidal table of the relative positions t - 1, ...,
    -(t - 1) (the page builds it on the host per chunk: its
    ``relative_pos_emb``); entry (r, 2i) = sin(p w_i), (r, 2i + 1) =
    cos(p w_i), p = t - 1 - r, w_i = 10000^(-2i/d)."""
    p = (t - 1 - np.arange(2 * t - 1, dtype=np.float64))[:, None]
    w = 10000.0 ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    out = np.zeros((2 * t - 1, d))
    out[:, 0::2] = np.sin(p * w)
    out[:, 1::2] = np.cos(p * w)
    return out


def xl_attention(q, k, v, p, bias_u, bias_v, n_head: int) -> np.ndarray:
    """Self-attention with the Transformer-XL relative-position term
    (audio_encoder_gpu.rs, ``xl_attention``): per head, q, k, v [t, hd]
    slices, p [2t - 1, hd] slice, u and v biases [hd]:
      score(i, j) = ((q_i + u) . k_j + (q_i + v) . p_{t-1-i+j}) / sqrt(hd),
    softmax over the t keys j, out_i = sum_j softmax_ij v_j.
    Returns [t, n_head hd]."""
    q, k, v, p = _f64(q), _f64(k), _f64(v), _f64(p)
    t, d = q.shape
    hd = d // n_head
    bu = _f64(bias_u).reshape(n_head, hd)
    bv = _f64(bias_v).reshape(n_head, hd)
    out = np.zeros((t, d))
    i = np.arange(t)[:, None]
    j = np.arange(t)[None, :]
    rows = t - 1 - i + j
    for h in range(n_head):
        sl = slice(h * hd, (h + 1) * hd)
        ac = (q[:, sl] + bu[h]) @ k[:, sl].T
        bd_all = (q[:, sl] + bv[h]) @ p[:, sl].T          # [t, 2t - 1]
        bd = np.take_along_axis(bd_all, rows, axis=1)
        s = (ac + bd) / math.sqrt(hd)
        s = s - s.max(axis=1, keepdims=True)
        e = np.exp(s)
        out[:, sl] = (e / e.sum(axis=1, keepdims=True)) @ v[:, sl]
    return out


def depthwise_conv1d(x, w, b) -> np.ndarray:
    """Depthwise convolution along time (audio_encoder_gpu.rs,
    ``encode_audio_gpu``, convolution module): x [t, d], w [d, k], b [d];
    pad k - 1 split as (k - 1) // 2 before and the rest after;
    out[i, c] = b[c] + sum_j w[c, j] x[i + j - (k - 1) // 2, c]."""
    x, w, b = _f64(x), _f64(w), _f64(b)
    t, d = x.shape
    k = w.shape[1]
    lo = (k - 1) // 2
    xp = np.zeros((t + k - 1, d))
    xp[lo:lo + t] = x
    out = np.repeat(b[None], t, axis=0)
    for j in range(k):
        out += xp[j:j + t] * w[:, j]
    return out


def macaron_ffn(x, L, sfx: str) -> np.ndarray:
    """Half-step feed-forward (audio_encoder_gpu.rs, ``macaron_ffn``):
    x + 0.5 (SiLU(LN(x) W_up^T + b_up) W_down^T + b_down)."""
    h = layer_norm(x, L["ffn_norm" + sfx + "_w"], L["ffn_norm" + sfx + "_b"])
    h = silu(linear(h, L["ffn_up" + sfx + "_w"], L["ffn_up" + sfx + "_b"]))
    return _f64(x) + 0.5 * linear(h, L["ffn_down" + sfx + "_w"], L["ffn_down" + sfx + "_b"])


def conformer_block(x, L, pos_emb, n_head: int) -> np.ndarray:
    """One block (audio_encoder_gpu.rs, ``encode_audio_gpu``, stage 3):
    FFN-1/2, relative-position self-attention, convolution module, FFN-1/2,
    final LayerNorm (no residual around it)."""
    x = macaron_ffn(x, L, "")
    h = layer_norm(x, L["ln1_w"], L["ln1_b"])
    q = linear(h, L["attn_q_w"], L["attn_q_b"])
    k = linear(h, L["attn_k_w"], L["attn_k_b"])
    v = linear(h, L["attn_v_w"], L["attn_v_b"])
    p = linear(pos_emb, L["linear_pos_w"])                 # no bias on the page
    a = xl_attention(q, k, v, p, L["pos_bias_u"], L["pos_bias_v"], n_head)
    x = x + linear(a, L["attn_o_w"], L["attn_o_b"])
    h = layer_norm(x, L["norm_conv_w"], L["norm_conv_b"])
    g = linear(h, L["conv_pw1_w"], L["conv_pw1_b"])
    d = g.shape[1] // 2
    g = g[:, :d] * sigmoid(g[:, d:])                       # glu_split
    c = depthwise_conv1d(g, L["conv_dw_w"], L["conv_dw_b"])
    c = silu(c * _f64(L["conv_norm_w"]) + _f64(L["conv_norm_b"]))   # chan_affine_silu
    x = x + linear(c, L["conv_pw2_w"], L["conv_pw2_b"])
    x = macaron_ffn(x, L, "_1")
    return layer_norm(x, L["ln2_w"], L["ln2_b"])


def adapter(x, W) -> np.ndarray:
    """MLP adapter to the language model's width (audio_encoder_gpu.rs,
    ``encode_audio_gpu``, stage 4): LN, up (+ bias), erf GELU, down
    (+ bias)."""
    h = layer_norm(x, W["adapter_norm_w"], W["adapter_norm_b"])
    h = gelu_erf(linear(h, W["adapter_up_w"], W["adapter_up_b"]))
    return linear(h, W["adapter_down_w"], W["adapter_down_b"])


def encode_features(feat, W, n_head: int = CONFIG["n_head"], layers=None) -> np.ndarray:
    """Stem, blocks and adapter from [F, n_mel] features: [t, llm_hidden]
    (audio_encoder_gpu.rs, ``encode_audio_gpu``)."""
    x = conv_stem(feat, W)
    t = x.shape[0]
    pe = relative_pos_emb(t, _f64(W["blocks"][0]["linear_pos_w"]).shape[1]) if W["blocks"] else None
    blocks = W["blocks"] if layers is None else W["blocks"][:layers]
    for L in blocks:
        x = conformer_block(x, L, pe, n_head)
    return adapter(x, W)


def encode(pcm, W, n_head: int = CONFIG["n_head"]) -> np.ndarray:
    """Raw 16 kHz PCM to [t, llm_hidden] embeddings (audio_encoder_gpu.rs,
    ``encode_audio_pcm_gpu``). An empty clip gives [0, llm_hidden]."""
    if len(pcm) == 0:
        return np.zeros((0, _f64(W["adapter_down_w"]).shape[0]))
    return encode_features(log_mel(pcm), W, n_head)
