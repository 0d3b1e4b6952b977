"""Rotary position embedding in float64 (test infrastructure only).

KVMEM (section "Engineering and cost ...") keeps position-free raw K and
re-applies RoPE at the block's new compact position; the Mean-K index is built
from K with RoPE removed.  IntentKV works on post-RoPE K and Q.

Reading (the pages name RoPE but not its layout): rotate-half pairing, i.e.
coordinate i is paired with i + D/2, frequency omega_i = theta^(-2i/D) for
i < D/2, and position p rotates each pair by the angle p * omega_i:
    y_i       = x_i * cos(p w_i) - x_{i+D/2} * sin(p w_i)
    y_{i+D/2} = x_{i+D/2} * cos(p w_i) + x_i * sin(p w_i)
Removing RoPE is the rotation by -p.  Angles are formed in float64.
Parity unpinned: the pairing the pages' models use (no page value fixes it).
"""

import numpy as np


def rope_omega(D, theta):
    """omega_i = theta^(-2i/D), i = 0 .. D/2 - 1, float64."""
    if D % 2:
        raise ValueError("D must be even")
    i = np.arange(D // 2, dtype=np.float64)
    return np.power(float(theta), -2.0 * i / D)


def rope_rotate(x, pos, theta, inverse=False):
    """Rotate x[..., t, :] by position pos[t] (or undo it when inverse=True).

    x: [..., T, D] float64-convertible; pos: [T] integer positions.
    """
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    ang = np.asarray(pos, dtype=np.float64)[:, None] * rope_omega(D, theta)[None, :]
    if inverse:
        ang = -ang
    c, s = np.cos(ang), np.sin(ang)                # [T, D/2]
    x1, x2 = x[..., :half], x[..., half:]
    y = np.empty_like(x)
    y[..., :half] = x1 * c - x2 * s
    y[..., half:] = x2 * c + x1 * s
    return y
