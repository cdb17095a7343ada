"""Rotary position embedding (RoPE), rotate-half form, in float64 (oracle).

Test infrastructure only (see ``oracle/__init__.py``).  The pages fix only the
base: [G3] "How it works" keeps theta = 1e4 on the local (sliding-window)
layers, and [KB] §2 "Interleaved local/global schemes" gives 1e4 on local and
1e6 on global layers.  The rest is a reading, the standard rotary form: the
d/2 pairs (x_i, x_{i + d/2}) are rotated by the angle p * base^(-2i/d) for a
token at position p:

    x_i'       = x_i cos(a) - x_{i+d/2} sin(a)
    x_{i+d/2}' = x_{i+d/2} cos(a) + x_i sin(a).

Nothing here is shared with the kernels or the input generator.
"""

import numpy as np


def rope_rotate_half(x, positions, base):
    """x: [..., T, H, d] (the position axis is -3); positions: [T] ints.

    Returns the rotated array in float64.
    """
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even head dimension")
    half = d // 2
    i = np.arange(half, dtype=np.float64)
    freq = float(base) ** (-2.0 * i / d)                        # theta_i
    ang = np.asarray(positions, dtype=np.float64)[:, None] * freq[None, :]   # [T, d/2]
    c = np.cos(ang)[:, None, :]                                  # broadcast over heads
    s = np.sin(ang)[:, None, :]
    a, b = x[..., :half], x[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)
