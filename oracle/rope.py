"""Rotary position embedding in float64 (test infrastructure only).

[SINK] section "como funciona": with RoPE the cache keeps keys before rotation and
the positional rotation is applied again at every decode step, at positions
counted inside the cache.  The pages name RoPE without restating it, so this is
the textbook rotary embedding: dimension pairs are rotated in their plane by the
angle ``pos * base**(-2i/D)`` for pair i < D/2.

Pairing (a reading; the pages do not fix it): "half" pairs element i with element
i + D/2 (the Llama layout the decode shapes follow); "interleaved" pairs 2i with
2i+1.  The rotation of a pair (a, b) by angle phi is the counter-clockwise plane
rotation (a cos phi - b sin phi, a sin phi + b cos phi).
"""
import numpy as np


def rope_inv_freq(head_dim: int, base: float) -> np.ndarray:
    """Angular frequency of each of the D/2 pairs: base ** (-2 i / D)."""
    if head_dim % 2:
        raise ValueError("head_dim must be even")
    i = np.arange(head_dim // 2, dtype=np.float64)
    return float(base) ** (-2.0 * i / head_dim)


def apply_rope(x: np.ndarray, pos, base: float, pairs: str = "half") -> np.ndarray:
    """Rotate the last axis of ``x`` (shape [..., D]) at positions ``pos``.

    ``pos`` broadcasts against ``x.shape[:-1]``.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    phi = np.asarray(pos, dtype=np.float64)[..., None] * rope_inv_freq(D, base)
    c, s = np.cos(phi), np.sin(phi)
    if pairs == "half":
        a, b = x[..., : D // 2], x[..., D // 2:]
    elif pairs == "interleaved":
        a, b = x[..., 0::2], x[..., 1::2]
    else:
        raise ValueError(pairs)
    ra = a * c - b * s
    rb = a * s + b * c
    out = np.empty(np.broadcast_shapes(x.shape, phi.shape[:-1] + (D,)), dtype=np.float64)
    if pairs == "half":
        out[..., : D // 2], out[..., D // 2:] = ra, rb
    else:
        out[..., 0::2], out[..., 1::2] = ra, rb
    return out
