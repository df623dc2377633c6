"""Rotary position embedding gathered by position value (oracle).

Source: NeMo Automodel PR 2376, commit message of the RoPE fix: cos/sin must be
gathered by the actual position values, with the cache sized to the highest
requested position (which exceeds the sequence length for the per-depth
offsets), instead of being sliced by sequence length. EAGLE's per-depth offset is
arange(seq_len) + step index; packed sequences restart their positions.

Readings:

- position of draft row (d, p): p - a_s + d, with a_s the start of the packed
  sequence holding p. A depth-d query sits at position anchor + d (speculators
  guide, "Architecture": depth d predicts for position anchor + d).
- Llama rotate-half convention (the draft layers are Llama-style, speculators
  guide): frequencies theta^(-2j/D) for j < D/2, pairs (j, j + D/2) rotated by
  angle pos * theta^(-2j/D). No rope scaling, no partial rotary. Applied to q
  and k, never to v.
- everything in float64.
"""
from __future__ import annotations

import numpy as np

from .cod import row_depths


def inv_freq(D: int, theta: float) -> np.ndarray:
    j = np.arange(D // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * j / D)


def angles(pos, D: int, theta: float) -> np.ndarray:
    """[len(pos), D/2] rotation angles pos * theta^(-2j/D)."""
    return np.asarray(pos, dtype=np.float64)[:, None] * inv_freq(D, theta)[None, :]


def table(D: int, theta: float, max_pos: int):
    """cos and sin [max_pos+1, D/2], indexed by position value."""
    a = angles(np.arange(max_pos + 1), D, theta)
    return np.cos(a), np.sin(a)


def rotate(x: np.ndarray, pos, theta: float) -> np.ndarray:
    """Rotate-half RoPE of x [R, heads, D] (float64) at positions pos [R]."""
    D = x.shape[-1]
    a = angles(pos, D, theta)[:, None, :]           # [R, 1, D/2]
    c, s = np.cos(a), np.sin(a)
    x1, x2 = x[..., : D // 2], x[..., D // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rotate_transpose(y: np.ndarray, pos, theta: float) -> np.ndarray:
    """The transpose (inverse) of ``rotate`` at the same positions: maps the gradient with
    respect to the rotated vectors to the gradient with respect to the unrotated ones."""
    D = y.shape[-1]
    a = angles(pos, D, theta)[:, None, :]
    c, s = np.cos(a), np.sin(a)
    y1, y2 = y[..., : D // 2], y[..., D // 2:]
    return np.concatenate([y1 * c + y2 * s, y2 * c - y1 * s], axis=-1)


def row_positions(idx, depth_off, cu_seqlens) -> np.ndarray:
    """Position value p - a_s + d of every draft row."""
    idx = np.asarray(idx, dtype=np.int64)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    seq = np.searchsorted(cu, idx, side="right") - 1
    return idx - cu[seq] + row_depths(depth_off)
