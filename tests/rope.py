"""Rotary position embedding for test inputs: a caller-side transform that produces the
position-embedded Q/K of the local attention.  Standard form: feature pairs (2i, 2i+1) of
the token at position p are rotated by the angle p * base^(-2i/d)."""

import numpy as np


def rope(x, base=10000.0, pos0=0):
    """x: [..., L, d] (d even) -> same shape, float64; positions pos0 .. pos0 + L - 1."""
    x = np.asarray(x, dtype=np.float64)
    L, d = x.shape[-2], x.shape[-1]
    inv = base ** (-np.arange(0, d, 2, dtype=np.float64) / d)            # [d/2]
    ang = (pos0 + np.arange(L, dtype=np.float64))[:, None] * inv[None]   # [L, d/2]
    c, s = np.cos(ang), np.sin(ang)
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out
