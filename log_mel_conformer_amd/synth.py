"""Seeded synthetic inputs: waveforms and random-init weights.

This module is shared by the HIP path's tests and benchmark and by the
oracle's tests. It holds no step of the encoder's arithmetic: it only draws
random numbers (numpy ``default_rng``, PCG64) and shapes them into the
workloads below. Every value is drawn in float64 and cast to float32; the
bf16 variants round every matrix to the nearest bfloat16 (ties to even)
before either side sees it, so both sides start from identical numbers.

Workloads (16 kHz mono, t = n / 16000):

* ``tone_clip``      one 1.0 s clip, 0.5*sin(2*pi*440 t) + N(0, 0.01^2), seed 0
* ``multisine_clip`` 30 s: 8 sinusoids, f ~ U(50, 7900) Hz, a ~ U(0, 0.1),
                     zero phase, + N(0, 0.02^2); one seed per clip
* ``white_clip``     30 s of U(-1, 1), one seed per clip
* ``ragged_batch``   64 clips, lengths ~ U{16000..480000} (seed 12345); clip i
                     is N(0, 0.05^2) noise through the unity-DC-gain one-pole
                     lowpass y[n] = 0.95 y[n-1] + 0.05 u[n]
* ``make_lfm2a_weights`` the LFM2A encoder (17 blocks of width 512):
                     matrices and conv kernels N(0, 1/fan_in), linear
                     biases 0.05 N(0, 1), LayerNorm and per-channel affine
                     gains 1 + 0.1 N(0, 1) with biases 0.1 N(0, 1),
                     pos_bias_u / pos_bias_v 0.1 N(0, 1); every matrix the
                     GEMMs read (the pointwise stem kernels included) is
                     rounded to bf16.
* ``make_weights``   matrices and conv kernels N(0, 1/fan_in); per_dim_scale
                     N(0, 0.1) (0.1 read as the variance); norm gains
                     1 + 0.1 N(0, 1); out_proj bias 0.1 N(0, 1); every
                     clippable projection clamps at +-8.
"""
from __future__ import annotations

import numpy as np

SR = 16000
MAX_SAMPLES = 480000

HIDDEN = 1024
HEADS = 8
HEAD_DIM = 128
FF = 4096
KERNEL = 5
C0 = 128
C1 = 32
OUT_HIDDEN = 1536
OUT_DIM = 512


# ----------------------------------------------------------------- waveforms

def tone_clip(seed: int = 0, n: int = 16000) -> np.ndarray:
    rng = np.random.default_rng(seed)
    t = np.arange(n, dtype=np.float64) / SR
    x = 0.5 * np.sin(2 * np.pi * 440.0 * t) + rng.normal(0.0, 0.01, n)
    return x.astype(np.float32)


def multisine_clip(seed: int = 0, n: int = MAX_SAMPLES) -> np.ndarray:
    rng = np.random.default_rng(seed)
    f = rng.uniform(50.0, 7900.0, 8)
    a = rng.uniform(0.0, 0.1, 8)
    t = np.arange(n, dtype=np.float64) / SR
    x = np.zeros(n, dtype=np.float64)
    for fk, ak in zip(f, a):
        x += ak * np.sin(2 * np.pi * fk * t)
    x += rng.normal(0.0, 0.02, n)
    return x.astype(np.float32)


def recorded_clip(seed: int, rate: int, seconds: float, channels: int = 2) -> np.ndarray:
    """A clip as a recorder delivers it, ahead of mixdown and resampling:
    interleaved frames [n, channels] float32 at `rate`, n = rate * seconds.
    Every channel holds the same 8 sines (frequencies U(50, 0.45 rate) Hz,
    amplitudes U(0, 0.1), drawn in that order, zero phase) plus its own
    N(0, 0.02^2) noise, so content sits above the 8 kHz a 16 kHz signal can
    keep as well as below it."""
    rng = np.random.default_rng(seed)
    n = int(round(rate * seconds))
    f = rng.uniform(50.0, 0.45 * rate, 8)
    a = rng.uniform(0.0, 0.1, 8)
    t = np.arange(n, dtype=np.float64) / rate
    base = np.zeros(n, dtype=np.float64)
    for fk, ak in zip(f, a):
        base += ak * np.sin(2 * np.pi * fk * t)
    out = np.empty((n, channels), dtype=np.float32)
    for c in range(channels):
        out[:, c] = (base + rng.normal(0.0, 0.02, n)).astype(np.float32)
    return out


def recorded_batch(clips: int, rate: int, seconds: float, channels: int = 2):
    return [recorded_clip(i, rate, seconds, channels) for i in range(clips)]


def pack_frames(clips):
    """Interleaved multichannel clips back to back: ([sum n, channels]
    float32, frame offsets int64 [B+1])."""
    off = np.zeros(len(clips) + 1, dtype=np.int64)
    off[1:] = np.cumsum([len(c) for c in clips])
    ch = clips[0].shape[1] if clips else 1
    data = (np.concatenate(clips, axis=0) if clips else np.zeros((0, ch), np.float32))
    return np.ascontiguousarray(data, dtype=np.float32), off


def white_clip(seed: int = 0, n: int = MAX_SAMPLES) -> np.ndarray:
    return np.random.default_rng(seed).uniform(-1.0, 1.0, n).astype(np.float32)


def ragged_lengths(count: int = 64, seed: int = 12345) -> np.ndarray:
    return np.random.default_rng(seed).integers(16000, MAX_SAMPLES + 1, count)


def pink_clip(seed: int, n: int) -> np.ndarray:
    from scipy.signal import lfilter
    u = np.random.default_rng(seed).normal(0.0, 0.05, n)
    y = lfilter([0.05], [1.0, -0.95], u)
    return y.astype(np.float32)


def tone_batch():
    """One 1 s tone clip (the smallest parity workload)."""
    return [tone_clip(0)]


def multisine_batch(clips: int, n: int = MAX_SAMPLES, first_seed: int = 0):
    return [multisine_clip(first_seed + i, n) for i in range(clips)]


def white_batch(clips: int, n: int = MAX_SAMPLES):
    return [white_clip(i, n) for i in range(clips)]


def ragged_batch(count: int = 64):
    lens = ragged_lengths(count)
    return [pink_clip(i, int(n)) for i, n in enumerate(lens)]


def pack(clips):
    """Concatenate clips back to back; returns (samples f32, offsets int64[B+1])."""
    off = np.zeros(len(clips) + 1, dtype=np.int64)
    for i, c in enumerate(clips):
        off[i + 1] = off[i] + len(c)
    wave = np.concatenate(clips).astype(np.float32) if clips else np.zeros(0, np.float32)
    return wave, off


# ------------------------------------------------------------------- weights

def round_bf16(x: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value (ties to even), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).reshape(np.shape(x))


def _mat(rng, out_f, in_f):
    return (rng.standard_normal((out_f, in_f)) / np.sqrt(in_f)).astype(np.float32)


def _gain(rng, n):
    return (1.0 + 0.1 * rng.standard_normal(n)).astype(np.float32)


CLIP8 = (-8.0, 8.0, -8.0, 8.0)

# Names of every matrix a layer holds (rounded to bf16 in the bf16 workloads).
LAYER_MATRICES = ("ff1_w1", "ff1_w2", "q", "k", "v", "post", "rel_k",
                  "lc_start", "lc_end", "ff2_w1", "ff2_w2")
TOP_MATRICES = ("conv1", "in_proj", "out_proj", "embed")


def make_layer(seed: int, hidden: int = HIDDEN, heads: int = HEADS, ff: int = FF,
               kernel: int = KERNEL, clip=CLIP8) -> dict:
    rng = np.random.default_rng(seed)
    hd = hidden // heads
    L = {}
    for f in ("ff1", "ff2"):
        L[f + "_pre"] = _gain(rng, hidden)
        L[f + "_w1"] = _mat(rng, ff, hidden)
        L[f + "_w2"] = _mat(rng, hidden, ff)
        L[f + "_post"] = _gain(rng, hidden)
        L[f + "_w1_clip"] = clip
        L[f + "_w2_clip"] = clip
    L["attn_pre"] = _gain(rng, hidden)
    for m in ("q", "k", "v", "post"):
        L[m] = _mat(rng, hidden, hidden)
        L[m + "_clip"] = clip
    L["attn_post"] = _gain(rng, hidden)
    L["per_dim_scale"] = rng.normal(0.0, np.sqrt(0.1), hd).astype(np.float32)
    L["rel_k"] = _mat(rng, hidden, hidden)
    L["lc_pre"] = _gain(rng, hidden)
    L["lc_start"] = _mat(rng, 2 * hidden, hidden)
    L["lc_start_clip"] = clip
    L["lc_dw"] = (rng.standard_normal((hidden, kernel)) / np.sqrt(kernel)).astype(np.float32)
    L["lc_norm"] = _gain(rng, hidden)
    L["lc_end"] = _mat(rng, hidden, hidden)
    L["lc_end_clip"] = clip
    L["norm_out"] = _gain(rng, hidden)
    return L


def make_weights(layers: int = 12, bf16: bool = False, clip=CLIP8) -> dict:
    """The whole encoder's parameters. Seeds: 999 for the subsampler and the
    head, 1000 + i for layer i."""
    rng = np.random.default_rng(999)
    W = {}
    W["conv0"] = (rng.standard_normal((C0, 1, 3, 3)) / np.sqrt(9.0)).astype(np.float32)
    W["ln0"] = _gain(rng, C0)
    W["conv1"] = (rng.standard_normal((C1, C0, 3, 3)) / np.sqrt(C0 * 9.0)).astype(np.float32)
    W["ln1"] = _gain(rng, C1)
    W["in_proj"] = _mat(rng, HIDDEN, C1 * 32)
    W["out_proj"] = _mat(rng, OUT_HIDDEN, HIDDEN)
    W["out_bias"] = (0.1 * rng.standard_normal(OUT_HIDDEN)).astype(np.float32)
    W["embed"] = _mat(rng, OUT_DIM, OUT_HIDDEN)
    W["layers"] = [make_layer(1000 + i, clip=clip) for i in range(layers)]
    if bf16:
        for k in TOP_MATRICES:
            W[k] = round_bf16(W[k])
        for L in W["layers"]:
            for k in LAYER_MATRICES:
                L[k] = round_bf16(L[k])
    return W


Q8_MATRICES = ("ff1_w1", "ff1_w2", "q", "k", "v", "post", "lc_start", "lc_end", "ff2_w1",
               "ff2_w2")


def quantize_rows(w: np.ndarray):
    """An int8 checkpoint of a matrix, as a quantised pack would hold it:
    symmetric per output row, scale = max |w_row| / 127 (float32),
    q = round(w / scale) clamped to +-127. (Producing the checkpoint is
    outside the encoder; the encoder consumes q and the scales.)"""
    w = np.asarray(w, dtype=np.float32)
    s = (np.abs(w).max(axis=1) / 127.0).astype(np.float32)
    s[s == 0] = 1.0
    q = np.clip(np.rint(w / s[:, None]), -127, 127).astype(np.int8)
    return q, s


def make_weights_q8(layers: int = 12, clip=CLIP8):
    """The encoder with int8 projections: the same draws as make_weights;
    the ten clippable projections of every layer as int8 + per-row scales,
    every other matrix bf16-rounded. Returns (weights, scales), scales a
    list (per layer) of dicts name -> float32 [out]."""
    W = make_weights(layers=layers, bf16=True, clip=clip)
    Wf = make_weights(layers=layers, bf16=False, clip=clip)
    scales = []
    for L, Lf in zip(W["layers"], Wf["layers"]):
        sc = {}
        for k in Q8_MATRICES:
            L[k], sc[k] = quantize_rows(Lf[k])
        scales.append(sc)
    return W, scales


CONFIG = dict(hidden=HIDDEN, heads=HEADS, left=12, n_dist=13, kernel=KERNEL,
              softcap=50.0, residual_weight=0.5, eps=1e-6)


# ------------------------------------------------------------ LFM2A encoder

LFM2A_MATRICES = ("ffn_up_w", "ffn_down_w", "attn_q_w", "attn_k_w", "attn_v_w", "attn_o_w",
                  "linear_pos_w", "conv_pw1_w", "conv_pw2_w", "ffn_up_1_w", "ffn_down_1_w")


def _bias(rng, n):
    return (0.05 * rng.standard_normal(n)).astype(np.float32)


def _shift(rng, n):
    return (0.1 * rng.standard_normal(n)).astype(np.float32)


def make_lfm2a_block(seed: int, d: int = 512, ff: int = 2048, kernel: int = 9) -> dict:
    rng = np.random.default_rng(seed)
    L = {}
    for nm in ("ffn_norm", "ln1", "norm_conv", "ffn_norm_1", "ln2"):
        L[nm + "_w"] = _gain(rng, d)
        L[nm + "_b"] = _shift(rng, d)
    for nm, (o, i) in (("ffn_up", (ff, d)), ("ffn_down", (d, ff)), ("attn_q", (d, d)),
                       ("attn_k", (d, d)), ("attn_v", (d, d)), ("attn_o", (d, d)),
                       ("conv_pw1", (2 * d, d)), ("conv_pw2", (d, d)), ("ffn_up_1", (ff, d)),
                       ("ffn_down_1", (d, ff))):
        L[nm + "_w"] = round_bf16(_mat(rng, o, i))
        L[nm + "_b"] = _bias(rng, o)
    L["linear_pos_w"] = round_bf16(_mat(rng, d, d))
    L["pos_bias_u"] = _shift(rng, d)
    L["pos_bias_v"] = _shift(rng, d)
    L["conv_dw_w"] = (rng.standard_normal((d, kernel)) / np.sqrt(kernel)).astype(np.float32)
    L["conv_dw_b"] = _bias(rng, d)
    L["conv_norm_w"] = _gain(rng, d)
    L["conv_norm_b"] = _shift(rng, d)
    return L


def make_lfm2a_weights(layers: int = 17) -> dict:
    """The LFM2A encoder's parameters in the oracle's layout (oracle.lfm2a):
    seed 777 for the stem and the adapter, 2000 + i for block i."""
    rng = np.random.default_rng(777)
    stem = []
    for shape in ((256, 1, 3, 3), (256, 1, 3, 3), (256, 256, 1, 1), (256, 1, 3, 3),
                  (256, 256, 1, 1)):
        fan_in = shape[1] * shape[2] * shape[3]
        w = (rng.standard_normal(shape) / np.sqrt(fan_in)).astype(np.float32)
        if shape[1] == 256:
            w = round_bf16(w)      # the pointwise layers run on the bf16 GEMM
        stem.append((w, _bias(rng, shape[0])))
    W = {"stem": stem}
    W["pre_encode_out_w"] = round_bf16(_mat(rng, 512, 4096))
    W["pre_encode_out_b"] = _bias(rng, 512)
    W["adapter_norm_w"] = _gain(rng, 512)
    W["adapter_norm_b"] = _shift(rng, 512)
    W["adapter_up_w"] = round_bf16(_mat(rng, 2048, 512))
    W["adapter_up_b"] = _bias(rng, 2048)
    W["adapter_down_w"] = round_bf16(_mat(rng, 2048, 2048))
    W["adapter_down_b"] = _bias(rng, 2048)
    W["blocks"] = [make_lfm2a_block(2000 + i) for i in range(layers)]
    return W
