"""Oracle for int8 weights with per-row scales.

TEST INFRASTRUCTURE (see the package docstring). The quantised linear layer
in the engine.py listing (hugingapi.com multimodalart/scenema-audio,
``_Int8Linear``) keeps an int8 matrix and one float scale per output row and
widens it on every forward: w = float32(q) * scale[row], cast to the
activation dtype, then an ordinary linear layer (egemma2_audio.rs,
``AudioTower::load``, likewise widens a quantised pack at load, to its f32
GEMM type). Widened to the bf16 GEMM operands of this encoder, a quantised
tower is the bf16 tower whose matrices are bf16(float32(q) * s): that is
what this module computes; the tower itself is ``oracle.encode_clips`` on
those matrices.
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """float32 -> nearest bf16 (ties to even), returned as float32."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def dequantize_rows(q, scale) -> np.ndarray:
    """bf16(float32(q[r][c]) * scale[r]) as float64: int8 q [out][in], one
    float32 scale per output row."""
    q = np.asarray(q)
    if q.dtype != np.int8:
        raise TypeError("q must be int8")
    s = np.asarray(scale, dtype=np.float32)
    w = q.astype(np.float32) * s[:, None]
    return round_bf16(w).astype(np.float64)
