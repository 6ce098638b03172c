"""Rotary position re-rotation (oracle side).

AKV (news.farwalk.ai page, section "AKV 如何工作"): Repos rewrites kept keys to
positions 0..r-1 by a RoPE rotation and leaves values unchanged.  The pages do not
print the rotary formula; the reading taken here is the NeoX / Qwen half-split
form with frequency theta^(-2i/d) for pair (i, i + d/2), i < d/2:

    x'[i]       = x[i] cos(p w_i) - x[i + d/2] sin(p w_i)
    x'[i + d/2] = x[i + d/2] cos(p w_i) + x[i] sin(p w_i),   w_i = theta^(-2i/d)

Rotating a key stored at position a by delta = b - a gives the key at position b,
because R(b) = R(delta) R(a).  All arithmetic is fp64.
"""
import numpy as np


def frequencies(d: int, theta: float) -> np.ndarray:
    return theta ** (-(2.0 * np.arange(d // 2, dtype=np.float64)) / d)


def rotate(x: np.ndarray, delta, theta: float) -> np.ndarray:
    """Rotate x[..., n, (H,) d] by per-token offsets delta[n] (fp64)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    h = d // 2
    delta = np.asarray(delta, dtype=np.float64)
    ang = delta.reshape(delta.shape + (1,)) * frequencies(d, theta)  # [n, d/2]
    if x.ndim == delta.ndim + 2:  # per-token head axis
        ang = ang[..., None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[..., :h], x[..., h:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
