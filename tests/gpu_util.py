"""Helpers shared by the GPU parity tests (no attention arithmetic here)."""

import sys

import numpy as np
import torch

# Tolerances: bf16 I/O with fp32 accumulation vs the fp64 oracle, and the
# float32 path (max abs error on the outputs).
TOL_BF16 = 2e-2
TOL_F32 = 1e-5
# lse, bf16 path: the scores are exact bf16 products summed in fp32, but the
# row sum l adds the weights p rounded to bf16 (the ones the P.V product uses),
# each off by at most 2^-8 relative, so ln l may be off by ln(1 + 2^-8) =
# 3.9e-3 when a row's few weights all round the same way (many-key rows average
# out far below that); exp2 / log2 and fp32 sums add ~1e-6.
TOL_LSE_BF16 = 4e-3
TOL_LSE_F32 = 1e-5
# lse when q = 0: every score is 0, every weight is exactly 1 (2^0, also in
# bf16), so the row sum l is the integer |S_t| held exactly in fp32 (< 2^24)
# and lse = log2(l) ln 2 carries only the rounding of the hardware log2 (about
# one ulp) and of the product: |error| <= 2^-22 |lse| < 3e-6 for |S_t| <= 2^15.
# A one-key change of |S_t| moves lse by ln((n+1)/n) >= 1/(n+1), i.e. by at
# least 3e-5 for n <= 32768, so this bound separates |S_t| from |S_t| +- 1.
TOL_LSE_EXACT = 1e-5


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
