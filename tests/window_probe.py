"""Inputs that make a kernel's window boundary visible in its outputs (test
helper; it builds inputs only and holds no attention arithmetic).

Key row s carries the binary code of an integer c(s) (normally its position)
in its first NB channels: +1 for a set bit, -1 for a clear bit, 0 in the other
channels.  A query aimed at the integer p carries A times the code of p.  Then
q . k_s = A (NB - 2 ham(c(s), p)), which is largest exactly at the key whose
code is p, and every other key scores at least 2A lower before scaling
(2A scale = 22.6 nats at A = 128, d_h = 128; 32 nats at d_h = 64): its weight
is below e^-22.
  * target in the row's attended set: o_t is that key's value row;
  * target outside it: o_t is the mean of the value rows of the attended keys
    whose codes are nearest to p.
An off-by-one window therefore swings o_t by O(1) (two different value rows)
instead of ~1/W, so the 2e-2 gate sees it.  Every product and partial sum of
the scores is an integer multiple of A in fp32, so the score ranking is exact
in the kernels as well.

Query heads take different aims (``aims``): the same launch checks the
window's two ends, just inside and just outside, on every row.
"""

import numpy as np
import torch

A = 128.0


def nbits(n):
    """Bits needed for the codes 0 .. n-1."""
    return max(1, int(n - 1).bit_length())


def code(values, NB, D):
    """float32 [..., D]: the +-1 code of each integer in ``values`` (taken mod
    2^NB) in channels 0..NB-1, zeros after."""
    v = np.asarray(values, dtype=np.int64) % (1 << NB)
    bits = (v[..., None] >> np.arange(NB)) & 1
    out = np.zeros(v.shape + (D,), dtype=np.float32)
    out[..., :NB] = 2.0 * bits - 1.0
    return out


def bf16(x):
    """CPU bf16 tensor of a float32 array whose values bf16 holds exactly."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    assert np.array_equal(t.float().numpy(), np.asarray(x, dtype=np.float32)), "not exact in bf16"
    return t


# Aims of the causal probes, by query head h (aim h % 8): offsets from the
# row's own position t, or (None, p) for the absolute position p.
CAUSAL_AIMS = [
    ("t-W", lambda t, W: t - W),          # just outside the start (exclusion)
    ("t-W+1", lambda t, W: t - W + 1),    # the oldest key of the window
    ("t", lambda t, W: t),                # the row itself (newest key)
    ("t+1", lambda t, W: t + 1),          # just outside the end (future)
    ("t-W+2", lambda t, W: t - W + 2),
    ("t-1", lambda t, W: t - 1),
    ("t-W-1", lambda t, W: t - W - 1),
    ("0", lambda t, W: 0 * t),            # the first position (ramp rows)
]


def causal_queries(B, T, Hq, D, W, NB, aims=CAUSAL_AIMS, shift=0):
    """q [B, T, Hq, D] float32: head h aims at aims[(h + shift) % len(aims)]."""
    t = np.arange(T, dtype=np.int64)
    q = np.zeros((B, T, Hq, D), dtype=np.float32)
    for h in range(Hq):
        q[:, :, h] = A * code(aims[(h + shift) % len(aims)][1](t, W), NB, D)[None]
    return q
