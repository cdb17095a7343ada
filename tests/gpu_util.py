"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import torch

# Tolerances: bf16 I/O with fp32 accumulation vs the fp64 oracle, and the
# float32 path (max abs error on the outputs).
TOL_BF16 = 2e-2
TOL_F32 = 1e-5
TOL_LSE_BF16 = 2e-3   # lse sees exact bf16 products summed in fp32
TOL_LSE_F32 = 1e-5


def banner(msg):
    """Name the case before a GPU step (so a failing run says what it was doing)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def dev(t):
    return t.to("cuda")


def host(t):
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)


def max_err(got, want):
    got = np.asarray(got, dtype=np.float64)
    want = np.asarray(want, dtype=np.float64)
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - want))) if got.size else 0.0
