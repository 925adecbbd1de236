"""Rotary re-rotation of reused keys, in fp64.

Position-independent reuse: keys computed offline at one position are turned by
a rotary transform from that original position to the position where the
document actually sits, so that the reused cache carries no position error
([SS] 技术原理 2 位置无关缓存复用, first item; [AB] 主な機能, second item).
RoPE rotates each pair of channels by an angle proportional to the position, so
moving a key by delta positions is a rotation by delta * theta_m of pair m.

The pages give no RoPE form.  Reading: rotate-half pairs (m, m + D/2) with
theta_m = base^(-2m/D), no frequency scaling (the convention of the Mistral,
Qwen3 and Llama models the pages measure on); the interleaved pairing
(2m, 2m + 1) is kept as an option.

TEST INFRASTRUCTURE ONLY (see the package docstring).
"""
from __future__ import annotations

import numpy as np

ROTATE_HALF = 0
INTERLEAVED = 1


def inv_freq(head_dim: int, base: float) -> np.ndarray:
    """theta_m = base^(-2m/D) for m in [0, D/2), fp64."""
    m = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(np.float64(base), -2.0 * m / head_dim)


def pair_index(head_dim: int, style: int):
    """(first, second) channel index of each rotated pair."""
    half = head_dim // 2
    m = np.arange(half)
    if style == ROTATE_HALF:
        return m, m + half
    if style == INTERLEAVED:
        return 2 * m, 2 * m + 1
    raise ValueError("unknown rope style")


def rotate(x: np.ndarray, delta, base: float, style: int = ROTATE_HALF) -> np.ndarray:
    """R(delta) x for x [..., D]; delta is a scalar or broadcasts against x[..., 0].

    For pair (a, b) with angle t = delta * theta_m:
      x'[a] = x[a] cos t - x[b] sin t,   x'[b] = x[b] cos t + x[a] sin t.
    """
    x = np.asarray(x, np.float64)
    D = x.shape[-1]
    a, b = pair_index(D, style)
    t = np.asarray(delta, np.float64)[..., None] * inv_freq(D, base)
    c, s = np.cos(t), np.sin(t)
    out = np.empty_like(x)
    out[..., a] = x[..., a] * c - x[..., b] * s
    out[..., b] = x[..., b] * c + x[..., a] * s
    return out
