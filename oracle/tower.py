"""Oracle tower: subsampler, Conformer layers and the output head.

TEST INFRASTRUCTURE (see the package docstring). float64 storage and
accumulation. Matrices follow y = x W^T with W stored [out][in].
Source: egemma2_audio.rs (cortiq-engine 0.8.49), module documentation
steps 3-5 and the items named in each docstring; the RMS norm follows
``rms_plain`` / ``rms_w`` of ltxdit.rs (cortiq-engine 0.5.94).

Weights are a dict (see ``encode_clips``); per-layer dicts use these keys:
ff{1,2}_pre, ff{1,2}_w1 [ff, d], ff{1,2}_w2 [d, ff], ff{1,2}_post,
ff{1,2}_w{1,2}_clip (in_lo, in_hi, out_lo, out_hi), attn_pre, q, k, v, post
[d, d] with q_clip..post_clip, attn_post, per_dim_scale [head_dim],
rel_k [d, d], lc_pre, lc_start [2d, d] (+ _clip), lc_dw [d, kernel],
lc_norm, lc_end [d, d] (+ _clip), norm_out.
"""
from __future__ import annotations

import math

import numpy as np

EPS = 1e-6


def _f64(x):
    return np.asarray(x, dtype=np.float64)


# ------------------------------------------------------------ subsampling

def layer_norm_relu(x: np.ndarray, g: np.ndarray) -> np.ndarray:
    """LayerNorm over the last (channel) axis, mean and biased variance,
    eps 1e-6, gain only (no bias), then ReLU (egemma2_audio.rs,
    ``layer_norm_relu``)."""
    x = _f64(x)
    mean = x.mean(axis=-1, keepdims=True)
    var = ((x - mean) ** 2).mean(axis=-1, keepdims=True)
    return np.maximum((x - mean) / np.sqrt(var + EPS) * _f64(g), 0.0)


def conv3x3_s2(x: np.ndarray, w: np.ndarray) -> np.ndarray:
    """3x3 convolution, stride 2, zero padding 1, no bias, channels last.

    x [T, F, Cin], w [Cout, Cin, 3, 3] (dt along time, df along frequency);
    out[t, f, co] = sum_{ci,dt,df} w[co,ci,dt,df] x[2t+dt-1, 2f+df-1, ci],
    with x zero outside [0,T) x [0,F) (egemma2_audio.rs, ``subsample``).
    """
    x = _f64(x)
    w = _f64(w)
    T, F, _ = x.shape
    To, Fo = -(-T // 2), -(-F // 2)
    xp = np.zeros((2 * To + 1, 2 * Fo + 1, x.shape[2]))
    xp[1:T + 1, 1:F + 1] = x
    out = np.zeros((To, Fo, w.shape[0]))
    for dt in range(3):
        for df in range(3):
            patch = xp[dt:dt + 2 * To:2, df:df + 2 * Fo:2]        # [To, Fo, Cin]
            out += patch @ w[:, :, dt, df].T
    return out


def subsample(mel: np.ndarray, W: dict) -> np.ndarray:
    """[F, 128] log-mel -> [ceil(F/4), hidden] rows after ``input_proj``.

    conv0 (1->128) + LN + ReLU, conv1 (128->32) + LN + ReLU, flatten
    frequency-major (feature = f*32 + c), then x W_in^T
    (egemma2_audio.rs, module documentation step 3 and ``subsample``;
    ``input_proj_linear`` belongs to the subsampler's parameters).
    """
    mel = _f64(mel)
    if mel.shape[0] == 0:
        return np.zeros((0, W["in_proj"].shape[0]))
    y0 = layer_norm_relu(conv3x3_s2(mel[:, :, None], W["conv0"]), W["ln0"])
    y1 = layer_norm_relu(conv3x3_s2(y0, W["conv1"]), W["ln1"])
    x = y1.reshape(y1.shape[0], -1)
    return x @ _f64(W["in_proj"]).T


# ------------------------------------------------------------- primitives

def rms_norm(x: np.ndarray, w=None) -> np.ndarray:
    """x / sqrt(mean(x^2) + 1e-6), times the weight plainly when given
    (ltxdit.rs ``rms_w`` / ``rms_plain``; egemma2_audio.rs module
    documentation: the weight multiplies plainly, not as 1 + w)."""
    x = _f64(x)
    y = x / np.sqrt((x * x).mean(axis=-1, keepdims=True) + EPS)
    return y if w is None else y * _f64(w)


def clip_linear(x: np.ndarray, w: np.ndarray, clip) -> np.ndarray:
    """Clippable linear: clamp the input, x W^T, clamp the output
    (egemma2_audio.rs, ``ClipLin::apply``). ``clip`` is
    (in_lo, in_hi, out_lo, out_hi); +-inf disables a bound."""
    lo_i, hi_i, lo_o, hi_o = clip
    y = np.clip(_f64(x), lo_i, hi_i) @ _f64(w).T
    return np.clip(y, lo_o, hi_o)


def sigmoid(x):
    return 1.0 / (1.0 + np.exp(-_f64(x)))


def silu(x):
    """x * sigmoid(x) (egemma2_audio.rs, ``silu_slice``)."""
    x = _f64(x)
    return x * sigmoid(x)


def softplus(x):
    """ln(1 + e^x), passing x through above 20 as torch does
    (egemma2_audio.rs, ``AudioTower::load``)."""
    x = _f64(x)
    return np.where(x > 20.0, x, np.log1p(np.exp(np.minimum(x, 20.0))))


def tower_constants(hidden=1024, heads=8, chunk=12, ctx_left=13, ctx_right=0):
    """Derived attention constants (egemma2_audio.rs, ``AudioTower::load``):
    window ``left`` = ctx_left - 1 keys, ``n_dist`` relative rows,
    q_scale = head_dim^-1/2 / ln 2 and k_scale = ln(1 + e) / ln 2."""
    if ctx_right != 0:
        raise ValueError("attention_context_right must be 0")
    head_dim = hidden // heads
    return dict(
        head_dim=head_dim,
        left=max(ctx_left - 1, 1),
        n_dist=(chunk + ctx_left - 1 + ctx_right) // 2 + 1,
        q_scale=head_dim ** -0.5 / math.log(2.0),
        k_scale=math.log(1.0 + math.e) / math.log(2.0),
    )


def rel_pos_table(n_dist: int, hidden: int) -> np.ndarray:
    """Sinusoids of the relative distances, [n_dist, hidden]: row d holds
    sin(d inv_i) for i < hidden/2, then cos(d inv_i), with
    inv_i = exp(-i ln(10000) / (hidden/2 - 1)) (egemma2_audio.rs,
    ``AudioTower::load``)."""
    n_ts = hidden // 2
    incr = math.log(10000.0) / (max(n_ts, 2) - 1)
    inv = np.exp(-np.arange(n_ts, dtype=np.float64) * incr)
    t = np.arange(n_dist, dtype=np.float64)[:, None] * inv[None, :]
    return np.concatenate([np.sin(t), np.cos(t)], axis=1)


def relative_keys(rel_k: np.ndarray, n_dist: int) -> np.ndarray:
    """R = PE rel_k^T, [n_dist, hidden]; ``relative_k_proj`` has no clamp."""
    rel_k = _f64(rel_k)
    return rel_pos_table(n_dist, rel_k.shape[1]) @ rel_k.T


# ------------------------------------------------------------ the layer

def ffn(h, L, f, residual_weight=0.5):
    """h + residual_weight * RMS_post(W2 silu(W1 RMS_pre(h))) through clippable
    linears (egemma2_audio.rs, ``ffn`` and ``add_normed``)."""
    a = rms_norm(h, L[f + "_pre"])
    u = silu(clip_linear(a, L[f + "_w1"], L[f + "_w1_clip"]))
    y = clip_linear(u, L[f + "_w2"], L[f + "_w2_clip"])
    return _f64(h) + residual_weight * rms_norm(y, L[f + "_post"])


def local_attention(q, k, v, R, pos, heads, left=12, softcap=50.0):
    """The attention core on already scaled q and k, [n, d] each.

    For token t and head hh, distances d < span = min(pos[t] + 1, left):
    logit = q_t . k_{t-d} + q_t . R[d]; s = softcap tanh(logit / softcap);
    p = softmax over d (natural exp); o_t = sum_d p_d v_{t-d}. Rows t-d for
    d > pos[t] belong to another clip (or precede the packed buffer) and are
    never read (egemma2_audio.rs, ``attention``). Explicit loops: the mask is
    the loop bound.
    """
    q, k, v, R = _f64(q), _f64(k), _f64(v), _f64(R)
    n, d = q.shape
    hd = d // heads
    o = np.zeros((n, d))
    for t in range(n):
        span = min(int(pos[t]) + 1, left)
        for hh in range(heads):
            sl = slice(hh * hd, (hh + 1) * hd)
            s = np.empty(span)
            for dist in range(span):
                logit = q[t, sl] @ k[t - dist, sl] + q[t, sl] @ R[dist, sl]
                s[dist] = softcap * math.tanh(logit / softcap)
            p = np.exp(s - s.max())
            p /= p.sum()
            for dist in range(span):
                o[t, sl] += p[dist] * v[t - dist, sl]
    return o


def attention_block(h, L, pos, heads=8, R=None, left=12, softcap=50.0, n_dist=13):
    """h + RMS_post_attn(post(attention(RMS_pre_attn(h)))), residual weight 1
    (egemma2_audio.rs, ``encode_locked`` and ``attention``)."""
    d = _f64(h).shape[1]
    c = tower_constants(hidden=d, heads=heads)
    a = rms_norm(h, L["attn_pre"])
    q = clip_linear(a, L["q"], L["q_clip"])
    k = clip_linear(a, L["k"], L["k_clip"])
    v = clip_linear(a, L["v"], L["v_clip"])
    hd = d // heads
    q_dim = softplus(L["per_dim_scale"])
    q = q * c["q_scale"] * np.tile(q_dim, d // hd)[None, :]
    k = k * c["k_scale"]
    if R is None:
        R = relative_keys(L["rel_k"], n_dist)
    o = local_attention(q, k, v, R, pos, heads, left, softcap)
    y = clip_linear(o, L["post"], L["post_clip"])
    return _f64(h) + rms_norm(y, L["attn_post"])


def glu(g):
    """[n, 2d] -> [n, d]: first half times sigmoid(second half)
    (egemma2_audio.rs, ``glu``)."""
    g = _f64(g)
    d = g.shape[1] // 2
    return g[:, :d] * sigmoid(g[:, d:])


def causal_dwconv(x, w, pos):
    """Depthwise causal convolution: out[t, c] = sum_k w[c, k] x[t - (K-1-k), c]
    over taps that stay inside the clip (K-1-k <= pos[t])
    (egemma2_audio.rs, ``dwconv``)."""
    x, w = _f64(x), _f64(w)
    n, d = x.shape
    K = w.shape[1]
    out = np.zeros((n, d))
    for t in range(n):
        for kk in range(K):
            back = K - 1 - kk
            if back <= pos[t]:
                out[t] += w[:, kk] * x[t - back]
    return out


def light_conv(h, L, pos):
    """h + lc_end(silu(RMS_conv(dwconv(glu(lc_start(RMS_pre(h))))))), residual
    weight 1, no norm on the residual branch (egemma2_audio.rs,
    ``encode_locked``, ``glu``, ``dwconv``, ``norm_silu``)."""
    a = rms_norm(h, L["lc_pre"])
    g = clip_linear(a, L["lc_start"], L["lc_start_clip"])
    c = causal_dwconv(glu(g), L["lc_dw"], pos)
    c = silu(rms_norm(c, L["lc_norm"]))
    return _f64(h) + clip_linear(c, L["lc_end"], L["lc_end_clip"])


def conformer_layer(h, L, pos, heads=8, R=None, residual_weight=0.5):
    """FFN1, attention, light conv, FFN2, then RMS_out
    (egemma2_audio.rs, module documentation step 4 and ``encode_locked``)."""
    h = ffn(h, L, "ff1", residual_weight)
    h = attention_block(h, L, pos, heads, R)
    h = light_conv(h, L, pos)
    h = ffn(h, L, "ff2", residual_weight)
    return rms_norm(h, L["norm_out"])


def head(h, W):
    """(h W_out^T + b), weightless RMS norm, then W_emb: [n, 512]
    (egemma2_audio.rs, module documentation step 5 and ``encode_locked``)."""
    o = _f64(h) @ _f64(W["out_proj"]).T + _f64(W["out_bias"])
    return rms_norm(o) @ _f64(W["embed"]).T


def encode_clips(clips, W, heads=8, layers=None, with_head=True, trace=None):
    """The encoder over a list of mono 16 kHz clips, packed back to back.

    Each clip: log-mel, then subsample; rows are concatenated with pos = the
    row's index inside its clip; then the layers and the head; the result
    is split per clip (egemma2_audio.rs, ``soft_tokens`` and
    ``encode_locked``). ``trace`` (a list) receives the packed subsampler
    output, every layer's output and the head's input projection.
    """
    from .frontend import log_mel
    xs, lens = [], []
    for c in clips:
        m = log_mel(c)
        x = subsample(m, W)
        xs.append(x)
        lens.append(x.shape[0])
    out_dim = W["embed"].shape[0] if with_head else W["in_proj"].shape[0]
    n = sum(lens)
    if n == 0:
        return [np.zeros((0, out_dim)) for _ in clips]
    h = np.concatenate(xs, axis=0)
    pos = np.concatenate([np.arange(l) for l in lens])
    if trace is not None:
        trace.append(h.copy())
    Ls = W["layers"] if layers is None else W["layers"][:layers]
    for L in Ls:
        h = conformer_layer(h, L, pos, heads)
        if trace is not None:
            trace.append(h.copy())
    e = head(h, W) if with_head else h
    res, off = [], 0
    for l in lens:
        res.append(e[off:off + l])
        off += l
    return res
