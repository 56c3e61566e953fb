"""Thin Python binding of libae.so (ctypes): argument marshalling only.

Every step of the encoder runs in the library's HIP kernels; this module
turns torch tensors into device pointers, host offset arrays into int64
buffers and the current torch stream into the library's stream argument.
There is no fallback: if libae.so is missing, importing the library
raises.

Names follow include/ae.h: ``logmel``, ``subsample``, ``conformer_layer``,
``encode``, ``num_frames``, ``num_tokens``, ``plan``, ``Model``, and for the
step ahead of the log-mel ``resampled_length``, ``Resampler``, ``mixdown``,
``resample``, ``to_mono_16k``; around it ``expand_ids`` and
``merge_soft_tokens``.
"""
from __future__ import annotations

import ctypes as C
import os

import numpy as np

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libae.so")

AE_OK, AE_ERR_INVALID, AE_ERR_SHAPE, AE_ERR_CAPACITY, AE_ERR_UNSUPPORTED, AE_ERR_HIP = range(6)
AE_F32, AE_BF16 = 0, 1
KERNEL_CLASSES = ("logmel", "conv0", "conv1", "gemm_ffn1", "gemm_ffn2", "gemm_qkv", "gemm_post",
                  "gemm_lcstart", "gemm_lcend", "gemm_head", "rownorm", "attn", "lconv",
                  "resample", "mixdown", "merge", "dequant",
                  "lfm_front", "lfm_stem", "lfm_gemm_stem", "lfm_gemm_ffn1", "lfm_gemm_ffn2",
                  "lfm_gemm_attn", "lfm_gemm_conv", "lfm_gemm_adapter", "lfm_ln", "lfm_attn",
                  "lfm_dwconv")


class AeError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"libae status {status}: {msg}")
        self.status = status


class Config(C.Structure):
    _fields_ = [("hidden", C.c_int32), ("heads", C.c_int32), ("layers", C.c_int32),
                ("ff", C.c_int32), ("conv_kernel", C.c_int32), ("chunk", C.c_int32),
                ("ctx_left", C.c_int32), ("ctx_right", C.c_int32), ("softcap", C.c_float),
                ("residual_weight", C.c_float), ("out_hidden", C.c_int32), ("out_dim", C.c_int32)]


class TokenIds(C.Structure):
    _fields_ = [("audio", C.c_int32), ("boa", C.c_int32), ("eoa", C.c_int32), ("bos", C.c_int32),
                ("eos", C.c_int32)]


class Clip(C.Structure):
    _fields_ = [("in_lo", C.c_float), ("in_hi", C.c_float), ("out_lo", C.c_float),
                ("out_hi", C.c_float)]


_P = C.c_void_p
LAYER_FIELDS = [
    ("ff1_pre", _P), ("ff1_w1", _P), ("ff1_w1_clip", Clip), ("ff1_w2", _P), ("ff1_w2_clip", Clip),
    ("ff1_post", _P), ("attn_pre", _P), ("q", _P), ("q_clip", Clip), ("k", _P), ("k_clip", Clip),
    ("v", _P), ("v_clip", Clip), ("post", _P), ("post_clip", Clip), ("attn_post", _P),
    ("per_dim_scale", _P), ("rel_k", _P), ("lc_pre", _P), ("lc_start", _P), ("lc_start_clip", Clip),
    ("lc_dw", _P), ("lc_norm", _P), ("lc_end", _P), ("lc_end_clip", Clip), ("ff2_pre", _P),
    ("ff2_w1", _P), ("ff2_w1_clip", Clip), ("ff2_w2", _P), ("ff2_w2_clip", Clip), ("ff2_post", _P),
    ("norm_out", _P)]


class LayerWeights(C.Structure):
    _fields_ = LAYER_FIELDS


Q8_FIELDS = ("ff1_w1", "ff1_w2", "q", "k", "v", "post", "lc_start", "lc_end", "ff2_w1", "ff2_w2")


class LayerScales(C.Structure):
    _fields_ = [(n, _P) for n in Q8_FIELDS]


class Weights(C.Structure):
    _fields_ = [("conv0", _P), ("ln0", _P), ("conv1", _P), ("ln1", _P), ("in_proj", _P),
                ("layers", C.POINTER(LayerWeights)), ("out_proj", _P), ("out_bias", _P),
                ("embed", _P)]


_lib = None


def lib():
    """The loaded libae.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with python -m log_mel_conformer_amd.build")
        L = C.CDLL(LIB_PATH)
        i64p = C.POINTER(C.c_int64)
        sigs = {
            "ae_config_default": (None, [C.POINTER(Config)]),
            "ae_last_error": (C.c_char_p, []),
            "ae_num_frames": (C.c_int64, [C.c_int64]),
            "ae_num_tokens": (C.c_int64, [C.c_int64]),
            "ae_plan": (C.c_int, [i64p, C.c_int32, i64p, i64p, i64p, i64p]),
            "ae_plan_frames": (C.c_int, [i64p, C.c_int32, i64p, i64p]),
            "ae_model_create": (C.c_int, [C.POINTER(Config), C.POINTER(Weights), C.c_int, _P,
                                          C.POINTER(_P)]),
            "ae_model_create_q8": (C.c_int, [C.POINTER(Config), C.POINTER(Weights),
                                             C.POINTER(LayerScales), _P, C.POINTER(_P)]),
            "ae_model_destroy": (None, [_P]),
            "ae_workspace_bytes": (C.c_size_t, [_P, C.c_int32, C.c_int64, C.c_int64]),
            "ae_logmel_workspace_bytes": (C.c_size_t, [C.c_int32]),
            "ae_logmel": (C.c_int, [_P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "ae_subsample": (C.c_int, [_P, _P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "ae_conformer_layer": (C.c_int, [_P, C.c_int32, _P, _P, C.c_int64, _P, C.c_size_t, _P]),
            "ae_encode": (C.c_int, [_P, _P, i64p, C.c_int32, _P, C.POINTER(_P), _P, C.c_size_t, _P]),
            "ae_encode_static": (C.c_int, [_P, _P, i64p, C.c_int32, _P, _P]),
            "ae_resampled_length": (C.c_int64, [C.c_int64, C.c_int32, C.c_int32]),
            "ae_resampler_create": (C.c_int, [C.c_int32, C.c_int32, _P, C.POINTER(_P)]),
            "ae_resampler_destroy": (None, [_P]),
            "ae_resampler_info": (C.c_int, [_P, C.POINTER(C.c_int32), i64p,
                                            C.POINTER(C.c_int32), C.POINTER(C.c_int32)]),
            "ae_resample_workspace_bytes": (C.c_size_t, [C.c_int32, C.c_int64, C.c_int32]),
            "ae_mixdown": (C.c_int, [_P, C.c_int64, C.c_int32, _P, _P]),
            "ae_resample": (C.c_int, [_P, _P, i64p, C.c_int32, _P, _P, C.c_size_t, _P]),
            "ae_to_mono_16k": (C.c_int, [_P, _P, i64p, C.c_int32, C.c_int32, _P, _P, C.c_size_t,
                                         _P]),
            "ae_expand_ids": (C.c_int, [C.POINTER(C.c_int32), C.c_int64, i64p, C.c_int32,
                                        C.POINTER(TokenIds), C.c_int64, C.POINTER(C.c_int32),
                                        C.c_int64, i64p]),
            "ae_merge_workspace_bytes": (C.c_size_t, [C.c_int64]),
            "ae_merge_soft_tokens": (C.c_int, [_P, C.c_int64, C.c_int32, _P, C.c_int64, C.c_int32,
                                               _P, _P, _P, C.c_size_t, _P]),
            "ae_timing_enable": (C.c_int, [C.c_int32]),
            "ae_timing_read": (C.c_int, [i64p, C.POINTER(C.c_double)]),
            "ae_probe_mfma": (C.c_int, [C.c_int32, _P, i64p, _P]),
        }
        for name, (res, args) in sigs.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _check(status):
    if status != AE_OK:
        raise AeError(status, lib().ae_last_error().decode())


def _i64(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int64))
    return a, a.ctypes.data_as(C.POINTER(C.c_int64))


def _stream():
    import torch
    return C.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    return C.c_void_p(t.data_ptr()) if t is not None else None


def _dev(t, name, dtype, numel=None, shape=None):
    """Refuse, before any launch, a tensor the kernels would read or write
    out of bounds: not a tensor on the current GPU, the wrong dtype, not
    contiguous, or smaller than the call's sizes."""
    import torch
    if not torch.is_tensor(t):
        raise AeError(AE_ERR_INVALID, f"{name}: a torch tensor is required, got {type(t).__name__}")
    if t.device.type != "cuda":
        raise AeError(AE_ERR_INVALID, f"{name}: must be a GPU tensor, not on {t.device}")
    if t.device.index != torch.cuda.current_device():
        raise AeError(AE_ERR_INVALID, f"{name}: on {t.device}, not the current GPU "
                                      f"cuda:{torch.cuda.current_device()}")
    if t.dtype != dtype:
        raise AeError(AE_ERR_INVALID, f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise AeError(AE_ERR_INVALID, f"{name}: must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise AeError(AE_ERR_SHAPE, f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if numel is not None and t.numel() < numel:
        raise AeError(AE_ERR_SHAPE, f"{name}: {t.numel()} elements, the call needs {numel}")
    return t


# ------------------------------------------------------------------ sizes

def default_config(**over) -> Config:
    c = Config()
    lib().ae_config_default(C.byref(c))
    for k, v in over.items():
        setattr(c, k, v)
    return c


def num_frames(n: int) -> int:
    return int(lib().ae_num_frames(int(n)))


def num_tokens(n: int) -> int:
    return int(lib().ae_num_tokens(int(n)))


def plan(lengths):
    """Prefix sums (samples capped at 30 s, frames, conv0 rows, tokens)."""
    n, p = _i64(lengths)
    B = len(n)
    outs = [np.zeros(B + 1, np.int64) for _ in range(4)]
    _check(lib().ae_plan(p, B, *[o.ctypes.data_as(C.POINTER(C.c_int64)) for o in outs]))
    return dict(sample_off=outs[0], frame_off=outs[1], row_off=outs[2], token_off=outs[3])


def plan_frames(frame_off):
    """conv0-row and token prefix sums of a packed log-mel layout."""
    fo, fp = _i64(frame_off)
    B = len(fo) - 1
    outs = [np.zeros(B + 1, np.int64) for _ in range(2)]
    _check(lib().ae_plan_frames(fp, B, *[o.ctypes.data_as(C.POINTER(C.c_int64)) for o in outs]))
    return dict(frame_off=fo, row_off=outs[0], token_off=outs[1])


def _sample_plan(sample_off):
    """Lengths from packed sample offsets, then ae_plan."""
    so, sp = _i64(sample_off)
    if len(so) < 1 or so[0] != 0:
        raise AeError(AE_ERR_INVALID, "sample_off must start at 0")
    lens = np.diff(so)
    if np.any(lens < 0):
        raise AeError(AE_ERR_INVALID, "sample_off must be non-decreasing")
    return so, sp, plan(lens)


# ------------------------------------------------------------------ model

_MATRICES = ("ff1_w1", "ff1_w2", "q", "k", "v", "post", "rel_k", "lc_start", "lc_end",
             "ff2_w1", "ff2_w2")


def _expected_layer_shapes(cfg: Config):
    d, ff, hd, K = cfg.hidden, cfg.ff, cfg.hidden // cfg.heads, cfg.conv_kernel
    s = {}
    for f in ("ff1", "ff2"):
        s[f + "_pre"] = (d,); s[f + "_post"] = (d,)
        s[f + "_w1"] = (ff, d); s[f + "_w2"] = (d, ff)
    for m in ("q", "k", "v", "post", "rel_k", "lc_end"):
        s[m] = (d, d)
    s.update(attn_pre=(d,), attn_post=(d,), per_dim_scale=(hd,), lc_pre=(d,),
             lc_start=(2 * d, d), lc_dw=(d, K), lc_norm=(d,), norm_out=(d,))
    return s


class Model:
    """Device copies of the weights plus the library's model handle.

    ``weights`` is a dict as made by ``synth.make_weights`` (numpy or torch
    arrays); matrices are stored in ``dtype`` ('f32' or 'bf16'), vectors in
    float32. Shapes are checked against the configuration, naming the
    tensor on a mismatch. With ``scales`` (per layer, name -> float32 [out],
    as made by ``synth.make_weights_q8``) the ten clippable projections of
    each layer are int8 and the model is ae_model_create_q8's.
    """

    def __init__(self, weights: dict, dtype: str = "bf16", device="cuda", scales=None,
                 **cfg_over):
        import torch
        if scales is not None and dtype != "bf16":
            raise AeError(AE_ERR_UNSUPPORTED, "int8 projections need dtype bf16")
        self.dtype = dtype
        self.dt = AE_BF16 if dtype == "bf16" else AE_F32
        mat_t = torch.bfloat16 if dtype == "bf16" else torch.float32
        cfg_over.setdefault("layers", len(weights["layers"]))
        self.cfg = default_config(**cfg_over)
        cfg = self.cfg
        self._keep = []

        def dev(x, is_mat, name, shape, int8=False):
            if int8:
                a = np.asarray(x)
                if a.dtype != np.int8:
                    raise AeError(AE_ERR_INVALID, f"{name}: int8 expected, got {a.dtype}")
                t = torch.from_numpy(np.ascontiguousarray(a))
            else:
                t = torch.as_tensor(np.asarray(x, dtype=np.float32)) if not torch.is_tensor(x) else x
            if tuple(t.shape) != tuple(shape):
                raise AeError(AE_ERR_SHAPE, f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
            dt_ = torch.int8 if int8 else (mat_t if is_mat else torch.float32)
            t = t.to(device=device, dtype=dt_).contiguous()
            self._keep.append(t)
            return C.c_void_p(t.data_ptr())

        d = cfg.hidden
        shapes = _expected_layer_shapes(cfg)
        self._layers = (LayerWeights * cfg.layers)()
        for i in range(cfg.layers):
            L = weights["layers"][i]
            lw = self._layers[i]
            for name, typ in LAYER_FIELDS:
                if typ is Clip:
                    lo_i, hi_i, lo_o, hi_o = L[name]
                    setattr(lw, name, Clip(lo_i, hi_i, lo_o, hi_o))
                else:
                    q8 = scales is not None and name in Q8_FIELDS
                    setattr(lw, name, dev(L[name], name in _MATRICES, f"layers.{i}.{name}",
                                          shapes[name], int8=q8))
        W = Weights()
        W.conv0 = dev(weights["conv0"], False, "conv0", (128, 1, 3, 3))
        W.ln0 = dev(weights["ln0"], False, "ln0", (128,))
        W.conv1 = dev(weights["conv1"], True, "conv1", (32, 128, 3, 3))
        W.ln1 = dev(weights["ln1"], False, "ln1", (32,))
        W.in_proj = dev(weights["in_proj"], True, "in_proj", (d, 1024))
        W.layers = self._layers
        W.out_proj = dev(weights["out_proj"], True, "out_proj", (cfg.out_hidden, d))
        W.out_bias = dev(weights["out_bias"], False, "out_bias", (cfg.out_hidden,))
        W.embed = dev(weights["embed"], True, "embed", (cfg.out_dim, cfg.out_hidden))
        self._w = W
        h = C.c_void_p()
        if scales is None:
            _check(lib().ae_model_create(C.byref(cfg), C.byref(W), self.dt, _stream(), C.byref(h)))
        else:
            self._scales = (LayerScales * cfg.layers)()
            for i in range(cfg.layers):
                for name in Q8_FIELDS:
                    setattr(self._scales[i], name,
                            dev(scales[i][name], False, f"layers.{i}.{name}.scale",
                                (shapes[name][0],)))
            _check(lib().ae_model_create_q8(C.byref(cfg), C.byref(W), self._scales, _stream(),
                                            C.byref(h)))
        self.handle = h
        self._ws = None

    def workspace(self, B: int, frames: int, tokens: int):
        import torch
        need = int(lib().ae_workspace_bytes(self.handle, B, frames, tokens))
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        return self._ws

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            lib().ae_model_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


# ---------------------------------------------------------------- compute

def logmel(wave, sample_off, out=None):
    """wave: cuda float32 [sum N]; sample_off: host int64 [B+1] -> [sum F, 128]."""
    import torch
    so, sp, pl = _sample_plan(sample_off)
    B = len(so) - 1
    F = int(pl["frame_off"][-1])
    _dev(wave, "wave", torch.float32, numel=int(so[-1]))
    if out is None:
        out = torch.empty((F, 128), dtype=torch.float32, device=wave.device)
    _dev(out, "out", torch.float32, shape=(F, 128))
    ws = torch.empty(max(int(lib().ae_logmel_workspace_bytes(B)), 256), dtype=torch.uint8,
                     device=wave.device)
    _check(lib().ae_logmel(_ptr(wave), sp, B, _ptr(out), _ptr(ws), ws.numel(), _stream()))
    return out


def subsample(model: Model, mel, frame_off, out=None):
    """mel: cuda float32 [sum F, 128]; frame_off host int64 [B+1] -> [sum T, hidden]."""
    import torch
    pf = plan_frames(frame_off)
    fo, fp = _i64(pf["frame_off"])
    B = len(fo) - 1
    F = int(fo[-1])
    T = int(pf["token_off"][-1])
    _dev(mel, "mel", torch.float32, numel=F * 128)
    if out is None:
        out = torch.empty((T, model.cfg.hidden), dtype=torch.float32, device=mel.device)
    _dev(out, "out", torch.float32, shape=(T, model.cfg.hidden))
    ws = model.workspace(B, F, T)
    _check(lib().ae_subsample(model.handle, _ptr(mel), fp, B, _ptr(out), _ptr(ws), ws.numel(),
                              _stream()))
    return out


def conformer_layer(model: Model, layer: int, h, pos):
    """In place on h: cuda float32 [n, hidden]; pos: cuda int32 [n]."""
    import torch
    if not torch.is_tensor(h) or h.dim() != 2:
        raise AeError(AE_ERR_SHAPE, "h: a 2-D tensor [n, hidden] is required")
    n = h.shape[0]
    _dev(h, "h", torch.float32, shape=(n, model.cfg.hidden))
    _dev(pos, "pos", torch.int32, shape=(n,))
    ws = model.workspace(1, 0, n)
    _check(lib().ae_conformer_layer(model.handle, layer, _ptr(h), _ptr(pos), n, _ptr(ws),
                                    ws.numel(), _stream()))
    return h


def encode(model: Model, wave, sample_off, out=None, trace: bool = False):
    """Soft tokens [sum T, out_dim] of the packed clips. With trace=True also
    returns [subsampler output, each layer's output, output_proj + bias]."""
    import torch
    so, sp, pl = _sample_plan(sample_off)
    B = len(so) - 1
    F, T = int(pl["frame_off"][-1]), int(pl["token_off"][-1])
    _dev(wave, "wave", torch.float32, numel=int(so[-1]))
    if out is None:
        out = torch.empty((T, model.cfg.out_dim), dtype=torch.float32, device=wave.device)
    _dev(out, "out", torch.float32, shape=(T, model.cfg.out_dim))
    ws = model.workspace(B, F, T)
    tr = None
    tr_arr = None
    if trace:
        L = model.cfg.layers
        tr = [torch.empty((T, model.cfg.hidden), dtype=torch.float32, device=wave.device)
              for _ in range(L + 1)]
        tr.append(torch.empty((T, model.cfg.out_hidden), dtype=torch.float32, device=wave.device))
        tr_arr = (C.c_void_p * len(tr))(*[t.data_ptr() for t in tr])
    _check(lib().ae_encode(model.handle, _ptr(wave), sp, B, _ptr(out),
                           C.cast(tr_arr, C.POINTER(C.c_void_p)) if tr_arr is not None else None,
                           _ptr(ws), ws.numel(), _stream()))
    return (out, tr) if trace else out


STATIC_SCRATCH_BYTES = 128 << 20   # AE_STATIC_SCRATCH_BYTES


def encode_static(model: Model, wave, sample_off, out=None):
    """ae_encode_static: the encoder on the library's static scratch (no
    workspace; nothing allocated by the call itself). Same results as
    ``encode``; batches beyond AE_STATIC_SCRATCH_BYTES raise
    AE_ERR_CAPACITY."""
    import torch
    so, sp, pl = _sample_plan(sample_off)
    B = len(so) - 1
    T = int(pl["token_off"][-1])
    _dev(wave, "wave", torch.float32, numel=int(so[-1]))
    if out is None:
        out = torch.empty((T, model.cfg.out_dim), dtype=torch.float32, device=wave.device)
    _dev(out, "out", torch.float32, shape=(T, model.cfg.out_dim))
    _check(lib().ae_encode_static(model.handle, _ptr(wave), sp, B, _ptr(out), _stream()))
    return out


def resampled_length(n: int, from_rate: int, to_rate: int = 16000) -> int:
    v = int(lib().ae_resampled_length(int(n), int(from_rate), int(to_rate)))
    if v < 0:
        raise AeError(AE_ERR_INVALID, f"no resampled length for n={n}, {from_rate} -> {to_rate}")
    return v


class Resampler:
    """A planned rate conversion (ae_resampler_create): the per-phase tap
    table lives on the current device until close()."""

    def __init__(self, from_rate: int, to_rate: int = 16000):
        self.from_rate, self.to_rate = int(from_rate), int(to_rate)
        h = C.c_void_p()
        _check(lib().ae_resampler_create(self.from_rate, self.to_rate, _stream(), C.byref(h)))
        self.handle = h
        self._ws = None

    def info(self) -> dict:
        q, ph, o = C.c_int32(), C.c_int32(), C.c_int32()
        nz = C.c_int64()
        _check(lib().ae_resampler_info(self.handle, C.byref(q), C.byref(nz), C.byref(ph),
                                       C.byref(o)))
        return {"taps_per_phase_max": q.value, "nonzero_taps_per_cycle": nz.value,
                "phases": ph.value, "in_per_cycle": o.value}

    def out_offsets(self, in_off) -> np.ndarray:
        lens = np.diff(np.asarray(in_off, dtype=np.int64))
        out = np.zeros(len(lens) + 1, dtype=np.int64)
        out[1:] = np.cumsum([resampled_length(n, self.from_rate, self.to_rate) for n in lens])
        return out

    def workspace(self, B: int, frames: int, channels: int, device):
        import torch
        need = max(int(lib().ae_resample_workspace_bytes(B, frames, channels)), 256)
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def close(self):
        if getattr(self, "handle", None) is not None and _lib is not None:
            import torch
            torch.cuda.synchronize()
            lib().ae_resampler_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def mixdown(x, channels: int, out=None):
    """x: cuda float32 [frames, channels] (or flat, interleaved) -> [frames]."""
    import torch
    _dev(x, "x", torch.float32)
    if channels < 1 or x.numel() % channels:
        raise AeError(AE_ERR_SHAPE, f"x: {x.numel()} values is not whole frames of {channels} channels")
    frames = x.numel() // channels
    if out is None:
        out = torch.empty(frames, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, shape=(frames,))
    _check(lib().ae_mixdown(_ptr(x), frames, channels, _ptr(out), _stream()))
    return out


def resample(r: Resampler, x, in_off, out=None):
    """x: cuda float32 [sum N], clip i at [in_off[i], in_off[i+1]) -> the
    clips resampled, packed."""
    import torch
    io, ip = _i64(in_off)
    B = len(io) - 1
    total = int(r.out_offsets(io)[-1])
    _dev(x, "x", torch.float32, numel=int(io[-1]))
    if out is None:
        out = torch.empty(total, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, shape=(total,))
    ws = r.workspace(B, int(io[-1]), 1, x.device)
    _check(lib().ae_resample(r.handle, _ptr(x), ip, B, _ptr(out), _ptr(ws), ws.numel(),
                             _stream()))
    return out


def to_mono_16k(r: Resampler, x, in_off, channels: int, out=None):
    """x: cuda float32 [sum N, channels] interleaved frames, clip i at frames
    [in_off[i], in_off[i+1]) -> mono 16 kHz clips, packed."""
    import torch
    io, ip = _i64(in_off)
    B = len(io) - 1
    total = int(r.out_offsets(io)[-1])
    _dev(x, "x", torch.float32, numel=int(io[-1]) * int(channels))
    if out is None:
        out = torch.empty(total, dtype=torch.float32, device=x.device)
    _dev(out, "out", torch.float32, shape=(total,))
    ws = r.workspace(B, int(io[-1]), channels, x.device)
    _check(lib().ae_to_mono_16k(r.handle, _ptr(x), ip, B, channels, _ptr(out), _ptr(ws),
                                ws.numel(), _stream()))
    return out


RELEASE_AUDIO, RELEASE_BOA, RELEASE_EOA = 258881, 256000, 258883


def expand_ids(body, n_soft, bos, eos, max_tokens, audio=RELEASE_AUDIO, boa=RELEASE_BOA,
               eoa=RELEASE_EOA) -> np.ndarray:
    """Host: the placeholder expansion of one input (ae_expand_ids)."""
    b = np.ascontiguousarray(np.asarray(body, dtype=np.int32))
    n, npp = _i64(n_soft)
    tok = TokenIds(audio, boa, eoa, bos, eos)
    cap = int(len(b) + 2 + int(np.sum(n)) + len(n))
    out = np.zeros(max(cap, 1), dtype=np.int32)
    out_len = C.c_int64()
    _check(lib().ae_expand_ids(b.ctypes.data_as(C.POINTER(C.c_int32)), len(b), npp, len(n),
                               C.byref(tok), int(max_tokens),
                               out.ctypes.data_as(C.POINTER(C.c_int32)), len(out),
                               C.byref(out_len)))
    return out[:out_len.value]


def merge_soft_tokens(ids, x, soft, audio=RELEASE_AUDIO):
    """Device, in place on x (cuda float32 [L, d]): the audio rows of ids
    (cuda int32 [L]) take the rows of soft (cuda float32 [S, d]) in order.
    Returns the number of audio rows (a device int64 tensor)."""
    import torch
    if not torch.is_tensor(x) or x.dim() != 2 or not torch.is_tensor(soft) or soft.dim() != 2:
        raise AeError(AE_ERR_SHAPE, "x [L, d] and soft [S, d] must be 2-D tensors")
    L, d = x.shape
    _dev(x, "x", torch.float32)
    _dev(ids, "ids", torch.int32, shape=(L,))
    _dev(soft, "soft", torch.float32, shape=(soft.shape[0], d))
    ws = torch.empty(max(int(lib().ae_merge_workspace_bytes(L)), 256), dtype=torch.uint8,
                     device=x.device)
    count = torch.zeros(1, dtype=torch.int64, device=x.device)
    _check(lib().ae_merge_soft_tokens(_ptr(ids), L, int(audio), _ptr(soft), soft.shape[0], d,
                                      _ptr(x), _ptr(count), _ptr(ws), ws.numel(), _stream()))
    return count


def timing_enable(cls):
    idx = -1 if cls is None else (KERNEL_CLASSES.index(cls) if isinstance(cls, str) else int(cls))
    _check(lib().ae_timing_enable(idx))


def timing_read():
    n = C.c_int64()
    ms = C.c_double()
    _check(lib().ae_timing_read(C.byref(n), C.byref(ms)))
    return int(n.value), float(ms.value)


def probe_mfma(iters, sink):
    """Launch the matrix-core rate probe on the current stream; returns the
    flops it performs (the caller times it). sink: a CUDA float32 tensor."""
    import torch
    _dev(sink, "sink", torch.float32, numel=1)
    flops = C.c_int64()
    _check(lib().ae_probe_mfma(int(iters), _ptr(sink), C.byref(flops), _stream()))
    return int(flops.value)
