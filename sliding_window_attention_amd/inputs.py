"""Seeded synthetic inputs shared by the tests, the bench and the oracle checks.

This module holds no attention arithmetic: it only draws random numbers, rounds
them to the I/O dtype, rotates q/k by RoPE for the local-layer workload (input
preparation, applied identically before either side sees the data) and lays out
ring-cache state.  Both the HIP path and the CPU oracle consume what it returns.

Recipe: NumPy ``default_rng(seed)`` (PCG64) ``standard_normal`` in float32,
rounded once to bfloat16 (round-to-nearest-even, torch's CPU cast) for the bf16
workloads; float32 workloads keep the float32 draws.
"""

from dataclasses import dataclass, field
import math

import numpy as np
import torch


def normal(shape, seed):
    """i.i.d. N(0, 1) float32 draws from PCG64(seed)."""
    return np.random.default_rng(seed).standard_normal(shape, dtype=np.float32)


def as_io(x, dtype):
    """Round a float array to the I/O dtype; returns a CPU torch tensor."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16) if dtype == "bf16" else t.clone()


def widen(t):
    """Exact float32 NumPy copy of a CPU tensor's values (bf16 widens exactly)."""
    return t.detach().to("cpu", torch.float32).numpy()


def rope_rotate_half(x, base=1.0e4):
    """Rotate-half RoPE over the last axis, positions = index along axis 1.

    x: float [B, T, H, d] (d even).  Pairs (x_i, x_{i+d/2}) are rotated by angle
    pos * base^(-2i/d), computed in float64 and returned as float64.  The local
    layers of the Gemma 3 study note use base 1e4; the pages fix only the base,
    so the pairing convention is a reading (it is applied before both sides and
    cannot affect parity).
    """
    x = np.asarray(x, dtype=np.float64)
    B, T, H, D = x.shape
    half = D // 2
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / D)
    ang = np.arange(T, dtype=np.float64)[:, None] * inv[None, :]
    cos = np.cos(ang)[None, :, None, :]
    sin = np.sin(ang)[None, :, None, :]
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * cos - x2 * sin, x1 * sin + x2 * cos], axis=-1)


@dataclass
class PrefillCase:
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    W: int
    dtype: str = "bf16"
    rope: bool = False
    seed: int = 0


@dataclass
class DecodeCase:
    B: int
    W: int
    Hq: int
    Hkv: int
    D: int
    cur_lo: int
    cur_hi: int
    dtype: str = "bf16"
    seed: int = 0


@dataclass
class LongformerCase:
    B: int
    T: int
    H: int
    D: int
    r: int
    dilation: list = field(default_factory=list)
    globals_: list = field(default_factory=list)
    dtype: str = "bf16"
    seed: int = 0


@dataclass
class ChunkCase:
    B: int
    L: int         # query tokens per request (the chunk)
    S: int         # ring slots
    W: int
    Hq: int
    Hkv: int
    D: int
    p_lo: int      # first chunk position ~ U[p_lo, p_hi)
    p_hi: int
    dtype: str = "bf16"
    seed: int = 0


# The workloads: seeded N(0, 1) tensors with the shapes of the pages' examples
# (n = 16 symmetric table, Mistral-shaped prefill and ring decode, Gemma 3 local
# layers, Longformer-base).
C1 = LongformerCase(B=1, T=16, H=1, D=64, r=2, dilation=[1], globals_=[], dtype="f32", seed=1000)
C2 = PrefillCase(B=1, T=16384, Hq=32, Hkv=8, D=128, W=4096, seed=1001)
C3 = PrefillCase(B=2, T=32768, Hq=32, Hkv=16, D=128, W=1024, rope=True, seed=1002)
C4 = DecodeCase(B=64, W=4096, Hq=32, Hkv=8, D=128, cur_lo=4096, cur_hi=32768, seed=1003)
C5 = LongformerCase(B=8, T=4096, H=12, D=64, r=256, dilation=[1] * 8 + [2] * 4,
                    globals_=[0, 8], seed=1004)
# chunked prefill into a Mistral-shaped ring: 512-token chunks, W = 4096, a ring
# of W + L - 1 slots, chunk starts anywhere in a 32K context
C6 = ChunkCase(B=4, L=512, S=4096 + 511, W=4096, Hq=32, Hkv=8, D=128, p_lo=4096,
               p_hi=32768 - 512, seed=1006)


def prefill_inputs(c: PrefillCase):
    """q [B,T,Hq,D], k, v [B,T,Hkv,D] as CPU tensors in the I/O dtype."""
    rng = np.random.default_rng(c.seed)
    q = rng.standard_normal((c.B, c.T, c.Hq, c.D), dtype=np.float32)
    k = rng.standard_normal((c.B, c.T, c.Hkv, c.D), dtype=np.float32)
    v = rng.standard_normal((c.B, c.T, c.Hkv, c.D), dtype=np.float32)
    if c.rope:
        q = rope_rotate_half(q)
        k = rope_rotate_half(k)
    return as_io(q, c.dtype), as_io(k, c.dtype), as_io(v, c.dtype)


def full_ring_positions(cur, W):
    """Absolute position held by each slot after tokens 0..cur were written with
    slot = position mod W: slot j holds the newest p <= cur with p = j (mod W),
    or -1 if no such p >= 0 exists."""
    cur = np.asarray(cur, dtype=np.int64).reshape(-1, 1)
    j = np.arange(W, dtype=np.int64).reshape(1, -1)
    p = cur - np.mod(cur - j, W)
    return np.where(p >= 0, p, -1).astype(np.int32)


def decode_inputs(c: DecodeCase):
    """q [B,Hq,D], k_cache, v_cache [B,Hkv,W,D], slot_pos [B,W] int32, cur_pos [B] int32.

    cur_pos ~ U[cur_lo, cur_hi) (integers); the ring holds tokens 0..cur_pos
    (write-before-read state: the current token is already in its slot).
    """
    rng = np.random.default_rng(c.seed)
    q = rng.standard_normal((c.B, c.Hq, c.D), dtype=np.float32)
    k = rng.standard_normal((c.B, c.Hkv, c.W, c.D), dtype=np.float32)
    v = rng.standard_normal((c.B, c.Hkv, c.W, c.D), dtype=np.float32)
    cur = rng.integers(c.cur_lo, c.cur_hi, size=c.B).astype(np.int32)
    slot_pos = full_ring_positions(cur, c.W)
    return (as_io(q, c.dtype), as_io(k, c.dtype), as_io(v, c.dtype),
            torch.from_numpy(slot_pos), torch.from_numpy(cur))


def chunk_inputs(c: ChunkCase):
    """q [B,L,Hq,D], k_cache, v_cache [B,Hkv,S,D], slot_pos [B,S] int32,
    q_pos [B,L] int32.

    The chunk of request b holds positions p0_b .. p0_b+L-1 with p0_b ~
    U[p_lo, p_hi); the ring holds tokens 0 .. p0_b+L-1 (the chunk already
    appended), i.e. slot j holds the newest such position congruent to j mod S.
    """
    rng = np.random.default_rng(c.seed)
    q = rng.standard_normal((c.B, c.L, c.Hq, c.D), dtype=np.float32)
    k = rng.standard_normal((c.B, c.Hkv, c.S, c.D), dtype=np.float32)
    v = rng.standard_normal((c.B, c.Hkv, c.S, c.D), dtype=np.float32)
    p0 = rng.integers(c.p_lo, c.p_hi, size=c.B).astype(np.int64)
    q_pos = (p0[:, None] + np.arange(c.L)[None, :]).astype(np.int32)
    slot_pos = full_ring_positions(p0 + c.L - 1, c.S)
    return (as_io(q, c.dtype), as_io(k, c.dtype), as_io(v, c.dtype),
            torch.from_numpy(slot_pos), torch.from_numpy(q_pos))


def longformer_inputs(c: LongformerCase):
    """q, k, v [B,T,H,D]; dilation [H] int32; global_idx [B,G] int32 (host)."""
    rng = np.random.default_rng(c.seed)
    q = rng.standard_normal((c.B, c.T, c.H, c.D), dtype=np.float32)
    k = rng.standard_normal((c.B, c.T, c.H, c.D), dtype=np.float32)
    v = rng.standard_normal((c.B, c.T, c.H, c.D), dtype=np.float32)
    dil = np.asarray(c.dilation if c.dilation else [1] * c.H, dtype=np.int32)
    g = np.asarray([list(c.globals_)] * c.B, dtype=np.int32).reshape(c.B, len(c.globals_))
    return as_io(q, c.dtype), as_io(k, c.dtype), as_io(v, c.dtype), dil, g


def default_scale(D):
    return 1.0 / math.sqrt(D)
