"""GPU parity at the full workload sizes, in the launch configuration the bench
times, on sampled outputs the oracle computes one by one (all heads), plus
whole-output sanity (finite, every row written)."""

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_LSE_BF16, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _sample_rows(T, W, seed, n_rand=8):
    rng = np.random.default_rng(seed)
    rows = set(range(0, 12)) | set(range(max(0, W - 6), min(T, W + 6))) | set(range(T - 6, T))
    rows |= set(rng.integers(0, T, size=n_rand).tolist())
    return np.array(sorted(rows))


@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_prefill_fullsize_sampled(cfg):
    c = getattr(inp, cfg)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill full size {cfg} B={c.B} T={c.T} W={c.W} Hq={c.Hq} Hkv={c.Hkv}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = bd.prefill(qd, kd, vd, c.W, return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    rows = _sample_rows(c.T, c.W, 5)
    o_s = host(o[:, rows])
    l_s = host(lse[:, :, rows])
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), c.W, rows=rows)
    assert max_err(o_s, ro) <= TOL_BF16
    assert max_err(l_s, rl) <= TOL_LSE_BF16


def test_decode_fullsize_all_outputs():
    c = inp.C4
    q, kc, vc, sp, cur = inp.decode_inputs(c)
    banner(f"decode full size B={c.B} W={c.W} Hq={c.Hq} Hkv={c.Hkv}")
    o, lse = bd.decode(dev(q), dev(kc), dev(vc), dev(sp), dev(cur), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_decode(inp.widen(q), inp.widen(kc), inp.widen(vc), sp.numpy(),
                               cur.numpy(), c.W)
    assert max_err(host(o), ro) <= TOL_BF16
    assert max_err(host(lse), rl) <= TOL_LSE_BF16


def test_longformer_fullsize_sampled():
    c = inp.C5
    q, k, v, dl, g = inp.longformer_inputs(c)
    banner(f"longformer full size B={c.B} T={c.T} H={c.H} r={c.r}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), c.r, dl, g, return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all())
    rows = np.array(sorted(set(_sample_rows(c.T, 2 * c.r, 6).tolist()) | set(c.globals_) |
                           {9, 511, 512, 513, 1023, 1024, 1025}))
    ro, rl = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), c.r, dl, g, rows=rows)
    assert max_err(host(o[:, rows]), ro) <= TOL_BF16
    assert max_err(host(lse[:, :, rows]), rl) <= TOL_LSE_BF16
