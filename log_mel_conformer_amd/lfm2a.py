"""Thin Python binding of the LFM2A encoder in libae.so (include/lfm2a.h):
argument marshalling only. Every step runs in the library's HIP kernels;
there is no fallback (a missing library raises, as in ``ae``).

Names follow include/lfm2a.h: ``num_frames``, ``num_tokens``, ``plan``,
``logmel``, ``Model``, ``stem``, ``block``, ``adapter``, ``encode``,
``xl_attention``.
"""
from __future__ import annotations

import ctypes as C

import numpy as np

from . import ae
from .ae import AE_ERR_INVALID, AE_ERR_SHAPE, AeError, _check, _dev, _i64, _ptr, _stream

_P = C.c_void_p


class Config(C.Structure):
    _fields_ = [("n_mel", C.c_int32), ("stem_ch", C.c_int32), ("n_embd", C.c_int32),
                ("n_head", C.c_int32), ("n_ff", C.c_int32), ("n_layer", C.c_int32),
                ("conv_kernel", C.c_int32), ("pos_dim", C.c_int32), ("adapter", C.c_int32),
                ("llm_hidden", C.c_int32), ("eps", C.c_float)]


BLOCK_FIELDS = [
    "ffn_norm_w", "ffn_norm_b", "ffn_up_w", "ffn_up_b", "ffn_down_w", "ffn_down_b",
    "ln1_w", "ln1_b", "attn_q_w", "attn_q_b", "attn_k_w", "attn_k_b", "attn_v_w", "attn_v_b",
    "attn_o_w", "attn_o_b", "pos_bias_u", "pos_bias_v", "linear_pos_w",
    "norm_conv_w", "norm_conv_b", "conv_pw1_w", "conv_pw1_b", "conv_dw_w", "conv_dw_b",
    "conv_norm_w", "conv_norm_b", "conv_pw2_w", "conv_pw2_b",
    "ffn_norm_1_w", "ffn_norm_1_b", "ffn_up_1_w", "ffn_up_1_b", "ffn_down_1_w", "ffn_down_1_b",
    "ln2_w", "ln2_b"]
# matrices handed to the GEMMs (bf16); every other block tensor is float32
BLOCK_MATRICES = ("ffn_up_w", "ffn_down_w", "attn_q_w", "attn_k_w", "attn_v_w", "attn_o_w",
                  "linear_pos_w", "conv_pw1_w", "conv_pw2_w", "ffn_up_1_w", "ffn_down_1_w")


class BlockWeights(C.Structure):
    _fields_ = [(n, _P) for n in BLOCK_FIELDS]


class Weights(C.Structure):
    _fields_ = [("stem_w", _P * 5), ("stem_b", _P * 5), ("pre_encode_out_w", _P),
                ("pre_encode_out_b", _P), ("blocks", C.POINTER(BlockWeights)),
                ("adapter_norm_w", _P), ("adapter_norm_b", _P), ("adapter_up_w", _P),
                ("adapter_up_b", _P), ("adapter_down_w", _P), ("adapter_down_b", _P)]


_sigs_done = False


def lib():
    global _sigs_done
    L = ae.lib()
    if not _sigs_done:
        i64p = C.POINTER(C.c_int64)
        sigs = {
            "lfm2a_config_default": (None, [C.POINTER(Config)]),
            "lfm2a_num_frames": (C.c_int64, [C.c_int64]),
            "lfm2a_num_tokens": (C.c_int64, [C.c_int64]),
            "lfm2a_plan": (C.c_int, [i64p, C.c_int32, i64p, i64p, i64p]),
            "lfm2a_plan_frames": (C.c_int, [i64p, C.c_int32, i64p]),
            "lfm2a_logmel_workspace_bytes": (C.c_size_t, [C.c_int32]),
            "lfm2a_logmel": (C.c_int, [_P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "lfm2a_model_create": (C.c_int, [C.POINTER(Config), C.POINTER(Weights), C.c_int, _P,
                                             C.POINTER(_P)]),
            "lfm2a_model_destroy": (None, [_P]),
            "lfm2a_workspace_bytes": (C.c_size_t, [_P, C.c_int32, C.c_int64, C.c_int64,
                                                   C.c_int64]),
            "lfm2a_stem": (C.c_int, [_P, _P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "lfm2a_block": (C.c_int, [_P, C.c_int32, _P, i64p, C.c_int32, _P, C.c_size_t, _P]),
            "lfm2a_adapter": (C.c_int, [_P, _P, C.c_int64, _P, _P, C.c_size_t, _P]),
            "lfm2a_encode": (C.c_int, [_P, _P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "lfm2a_attention_workspace_bytes": (C.c_size_t, [C.c_int32]),
            "lfm2a_xl_attention": (C.c_int, [_P, _P, C.c_int64, _P, _P, i64p, C.c_int32, _P, _P,
                                             C.c_size_t, _P]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _sigs_done = True
    return L


def default_config(**over) -> Config:
    c = Config()
    lib().lfm2a_config_default(C.byref(c))
    for k, v in over.items():
        setattr(c, k, v)
    return c


def num_frames(n: int) -> int:
    return int(lib().lfm2a_num_frames(int(n)))


def num_tokens(n: int) -> int:
    return int(lib().lfm2a_num_tokens(int(n)))


def plan(lengths):
    """Prefix sums of samples, frames and tokens (host int64 [B+1] each)."""
    n, p = _i64(lengths)
    B = len(n)
    outs = [np.zeros(B + 1, np.int64) for _ in range(3)]
    _check(lib().lfm2a_plan(p, B, *[o.ctypes.data_as(C.POINTER(C.c_int64)) for o in outs]))
    return dict(sample_off=outs[0], frame_off=outs[1], token_off=outs[2])


def plan_frames(frame_off):
    """Token prefix sums of a packed feature layout (host int64 [B+1])."""
    fo, fp = _i64(frame_off)
    B = len(fo) - 1
    to = np.zeros(B + 1, np.int64)
    _check(lib().lfm2a_plan_frames(fp, B, to.ctypes.data_as(C.POINTER(C.c_int64))))
    return to


def _sample_plan(sample_off):
    so, sp = _i64(sample_off)
    if len(so) < 1 or so[0] != 0:
        raise AeError(AE_ERR_INVALID, "sample_off must start at 0")
    lens = np.diff(so)
    if np.any(lens < 0):
        raise AeError(AE_ERR_INVALID, "sample_off must be non-decreasing")
    return so, sp, plan(lens)


def _ws(nbytes, device="cuda"):
    import torch
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def logmel(wave, sample_off, out=None):
    """wave: cuda float32 [sum N]; sample_off: host int64 [B+1] ->
    normalised features [sum F, 128]."""
    import torch
    so, sp, pl = _sample_plan(sample_off)
    B = len(so) - 1
    F = int(pl["frame_off"][-1])
    _dev(wave, "wave", torch.float32, numel=int(so[-1]))
    if out is None:
        out = torch.empty((F, 128), dtype=torch.float32, device=wave.device)
    _dev(out, "out", torch.float32, shape=(F, 128))
    ws = _ws(lib().lfm2a_logmel_workspace_bytes(B), wave.device)
    _check(lib().lfm2a_logmel(_ptr(wave), sp, B, _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


_STEM_SHAPES = [(256, 1, 3, 3), (256, 1, 3, 3), (256, 256, 1, 1), (256, 1, 3, 3),
                (256, 256, 1, 1)]


def _block_shapes(cfg: Config):
    d, ff, k = cfg.n_embd, cfg.n_ff, cfg.conv_kernel
    s = {}
    for n in BLOCK_FIELDS:
        s[n] = (d,)
    s.update(ffn_up_w=(ff, d), ffn_up_b=(ff,), ffn_down_w=(d, ff), ffn_up_1_w=(ff, d),
             ffn_up_1_b=(ff,), ffn_down_1_w=(d, ff), attn_q_w=(d, d), attn_k_w=(d, d),
             attn_v_w=(d, d), attn_o_w=(d, d), linear_pos_w=(d, cfg.pos_dim),
             conv_pw1_w=(2 * d, d), conv_pw1_b=(2 * d,), conv_dw_w=(d, k), conv_pw2_w=(d, d))
    return s


class Model:
    """Device copies of an LFM2A weight dict (as made by
    ``synth.make_lfm2a_weights``: the oracle's key names) plus the library's
    model handle. Matrices go to the device in bf16, everything else in
    float32; shapes are checked, naming the tensor on a mismatch."""

    def __init__(self, weights: dict, dtype: str = "bf16", device="cuda", **cfg_over):
        import torch
        if dtype != "bf16":
            raise AeError(ae.AE_ERR_UNSUPPORTED, "the LFM2A encoder is implemented in bf16 only")
        cfg_over.setdefault("n_layer", len(weights["blocks"]))
        self.cfg = default_config(**cfg_over)
        cfg = self.cfg
        self._keep = []

        def dev(x, is_mat, name, shape):
            t = x if torch.is_tensor(x) else torch.as_tensor(np.asarray(x, dtype=np.float32))
            if tuple(t.shape) != tuple(shape):
                raise AeError(ae.AE_ERR_SHAPE,
                              f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
            t = t.to(device=device, dtype=torch.bfloat16 if is_mat else torch.float32).contiguous()
            self._keep.append(t)
            return C.c_void_p(t.data_ptr())

        shapes = _block_shapes(cfg)
        self._blocks = (BlockWeights * cfg.n_layer)()
        for i in range(cfg.n_layer):
            Lw = weights["blocks"][i]
            for n in BLOCK_FIELDS:
                setattr(self._blocks[i], n, dev(Lw[n], n in BLOCK_MATRICES, f"blocks.{i}.{n}",
                                                shapes[n]))
        W = Weights()
        for i, (w, b) in enumerate(weights["stem"]):
            W.stem_w[i] = dev(w, False, f"stem.{i}.w", _STEM_SHAPES[i])
            W.stem_b[i] = dev(b, False, f"stem.{i}.b", (256,))
        d = cfg.n_embd
        W.pre_encode_out_w = dev(weights["pre_encode_out_w"], True, "pre_encode_out_w", (d, 4096))
        W.pre_encode_out_b = dev(weights["pre_encode_out_b"], False, "pre_encode_out_b", (d,))
        W.blocks = self._blocks
        W.adapter_norm_w = dev(weights["adapter_norm_w"], False, "adapter_norm_w", (d,))
        W.adapter_norm_b = dev(weights["adapter_norm_b"], False, "adapter_norm_b", (d,))
        W.adapter_up_w = dev(weights["adapter_up_w"], True, "adapter_up_w", (cfg.adapter, d))
        W.adapter_up_b = dev(weights["adapter_up_b"], False, "adapter_up_b", (cfg.adapter,))
        W.adapter_down_w = dev(weights["adapter_down_w"], True, "adapter_down_w",
                               (cfg.llm_hidden, cfg.adapter))
        W.adapter_down_b = dev(weights["adapter_down_b"], False, "adapter_down_b",
                               (cfg.llm_hidden,))
        self._w = W
        h = C.c_void_p()
        _check(lib().lfm2a_model_create(C.byref(cfg), C.byref(W), ae.AE_BF16, _stream(),
                                        C.byref(h)))
        self.handle = h
        self._ws = None

    def workspace(self, B: int, frames: int, tokens: int, max_tokens: int):
        import torch
        need = int(lib().lfm2a_workspace_bytes(self.handle, B, frames, tokens, max_tokens))
        if self._ws is None or self._ws.numel() < need:
            self._ws = None
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().lfm2a_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stem(model: Model, feat, frame_off, out=None):
    """feat: cuda float32 [sum F, 128]; frame_off: host int64 [B+1] ->
    x [sum T, n_embd] float32."""
    import torch
    fo, fp = _i64(frame_off)
    B = len(fo) - 1
    to = plan_frames(fo)
    T = int(to[-1])
    _dev(feat, "feat", torch.float32, numel=int(fo[-1]) * 128)
    if out is None:
        out = torch.empty((T, model.cfg.n_embd), dtype=torch.float32, device=feat.device)
    _dev(out, "out", torch.float32, shape=(T, model.cfg.n_embd))
    ws = model.workspace(B, int(fo[-1]), T, int(np.diff(to).max(initial=0)))
    _check(lib().lfm2a_stem(model.handle, _ptr(feat), fp, B, _ptr(out), _ptr(ws), ws.numel(),
                            _stream()))
    return out


def block(model: Model, layer: int, x, token_off):
    """One Conformer block in place on x (cuda float32 [n, n_embd])."""
    import torch
    to, tp = _i64(token_off)
    B = len(to) - 1
    _dev(x, "x", torch.float32, shape=(int(to[-1]), model.cfg.n_embd))
    ws = model.workspace(B, 0, int(to[-1]), int(np.diff(to).max(initial=0)))
    _check(lib().lfm2a_block(model.handle, int(layer), _ptr(x), tp, B, _ptr(ws), ws.numel(),
                             _stream()))
    return x


def adapter(model: Model, x, out=None):
    import torch
    if not torch.is_tensor(x) or x.dim() != 2:
        raise AeError(AE_ERR_SHAPE, "x: a 2-D tensor [n, n_embd] is required")
    n = x.shape[0]
    _dev(x, "x", torch.float32, shape=(n, model.cfg.n_embd))
    if out is None:
        out = torch.empty((n, model.cfg.llm_hidden), dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, shape=(n, model.cfg.llm_hidden))
    ws = model.workspace(1, 0, n, 0)
    _check(lib().lfm2a_adapter(model.handle, _ptr(x), n, _ptr(out), _ptr(ws), ws.numel(),
                               _stream()))
    return out


def encode(model: Model, wave, sample_off, out=None):
    """wave: cuda float32 [sum N]; sample_off: host int64 [B+1] ->
    embeddings [sum T, llm_hidden] float32."""
    import torch
    so, sp, pl = _sample_plan(sample_off)
    B = len(so) - 1
    F, T = int(pl["frame_off"][-1]), int(pl["token_off"][-1])
    _dev(wave, "wave", torch.float32, numel=int(so[-1]))
    if out is None:
        out = torch.empty((T, model.cfg.llm_hidden), dtype=torch.float32, device=wave.device)
    _dev(out, "out", torch.float32, shape=(T, model.cfg.llm_hidden))
    ws = model.workspace(B, F, T, int(np.diff(pl["token_off"]).max(initial=0)))
    _check(lib().lfm2a_encode(model.handle, _ptr(wave), sp, B, _ptr(out), _ptr(ws), ws.numel(),
                              _stream()))
    return out


def xl_attention(qkv, p, t_max, u, v, token_off, out=None):
    """The attention kernel alone: qkv cuda bf16 [n, 1536], p cuda bf16
    [2 t_max - 1, 512], u, v cuda float32 [512]; token_off host int64."""
    import torch
    to, tp = _i64(token_off)
    B = len(to) - 1
    n = int(to[-1])
    _dev(qkv, "qkv", torch.bfloat16, shape=(n, 1536))
    _dev(p, "p", torch.bfloat16, shape=(2 * int(t_max) - 1, 512))
    _dev(u, "u", torch.float32, shape=(512,))
    _dev(v, "v", torch.float32, shape=(512,))
    if out is None:
        out = torch.empty((n, 512), dtype=torch.bfloat16, device=qkv.device)
    _dev(out, "out", torch.bfloat16, shape=(n, 512))
    ws = _ws(lib().lfm2a_attention_workspace_bytes(B), qkv.device)
    _check(lib().lfm2a_xl_attention(_ptr(qkv), _ptr(p), int(t_max), _ptr(u), _ptr(v), tp, B,
                                    _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out
