"""GPU parity: swa_prefill_dilated (causal windows {t - i*d : 0 <= i < W}, one
dilation per query head) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu

# B, T, Hq, Hkv, D, W, dilation per query head.  Groups whose heads share a
# dilation are packed four (or two) heads per workgroup; mixed groups run one
# head per workgroup.
SMALL = [
    (1, 300, 4, 2, 128, 70, [1, 2, 3, 1]),          # mixed within a group
    (2, 333, 8, 2, 128, 40, [2] * 4 + [3] * 4),    # uniform groups, 4 heads packed
    (1, 257, 8, 8, 64, 64, [1, 2, 3, 4, 5, 6, 7, 8]),
    (1, 200, 2, 1, 128, 500, [4, 7]),              # window longer than every class
    (1, 129, 4, 1, 64, 1, [2, 2, 2, 2]),           # W = 1: own value
    (1, 90, 2, 2, 128, 9, [100, 3]),               # dilation beyond T
    (2, 1000, 8, 2, 128, 100, [1] * 4 + [2] * 4),  # an undilated group next to a dilated one
    (1, 515, 6, 3, 64, 33, [2, 2, 5, 5, 3, 3]),    # two heads per group packed
]


def _run(case, dtype):
    B, T, Hq, Hkv, D, W, dil = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype=dtype, seed=T + 3 * Hq + W)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill_dilated {dtype} {case}")
    o, lse = bd.prefill_dilated(dev(q), dev(k), dev(v), W, dil, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W, dilation=dil)
    return host(o), host(lse), ro, rl


@pytest.mark.parametrize("case", SMALL, ids=[str(c[:6]) for c in SMALL])
def test_prefill_dilated_bf16(case):
    o, lse, ro, rl = _run(case, "bf16")
    assert max_err(o, ro) <= TOL_BF16
    assert max_err(lse, rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("case", SMALL[:6], ids=[str(c[:6]) for c in SMALL[:6]])
def test_prefill_dilated_f32(case):
    o, lse, ro, rl = _run(case, "f32")
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_LSE_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("W,d", [(1, 2), (3, 2), (3, 3), (5, 4), (16, 3)])
def test_dilated_index_readout(dtype, W, d):
    # q = 0 and one-hot v read the kernels' connectivity sets out exactly
    n, D = 16, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.zeros(1, n, 4, D)
    k = torch.from_numpy(inp.normal((1, n, 1, D), 23))
    v = torch.zeros(1, n, 1, D)
    for s in range(n):
        v[0, s, 0, s] = 1.0
    banner(f"prefill_dilated readout {dtype} W={W} d={d}")
    o = host(bd.prefill_dilated(dev(q.to(tdt)), dev(k.to(tdt)), dev(v.to(tdt)), W, [d, d, 1, d]))
    for h, dh in enumerate((d, d, 1, d)):
        for t in range(n):
            sup = np.nonzero(o[0, t, h])[0].tolist()
            assert sup == oracle.causal_dilated_index_set(t, W, dh).tolist()
            np.testing.assert_allclose(o[0, t, h][sup], 1.0 / len(sup), rtol=2 ** -8)


def test_all_ones_is_prefill():
    c = inp.PrefillCase(B=1, T=300, Hq=8, Hkv=2, D=128, W=70, seed=5)
    q, k, v = (dev(x) for x in inp.prefill_inputs(c))
    banner("prefill_dilated all ones == prefill")
    a = bd.prefill(q, k, v, c.W)
    b = bd.prefill_dilated(q, k, v, c.W, [1] * 8)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_prefill_dilated_fullsize_row_set():
    # the timed dilated workload (headline shape, dilations 1, 2 and 4 on groups
    # of heads) in bench.py's launch configuration: rows [0, W+256), [T-256, T)
    # and 1024 seeded random rows, all heads
    c = inp.C2
    dil = [1] * 16 + [2] * 8 + [4] * 8
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill_dilated full size T={c.T} W={c.W} row set")
    o, lse = bd.prefill_dilated(dev(q), dev(k), dev(v), c.W, dil, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), host(lse)
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([np.arange(0, c.W + 256), np.arange(c.T - 256, c.T),
                                     rng.integers(0, c.T, 1024)]))
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(oracle.swa_prefill, (inp.widen(q), inp.widen(k), inp.widen(v)),
                                      rows, dict(W=c.W, dilation=dil)):
        e = max_err(host(o[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"rows {rc[0]}..{rc[-1]} max err {e}"
        assert max_err(lse[:, :, rc], rl) <= TOL_LSE_BF16, f"lse rows {rc[0]}..{rc[-1]}"
    banner(f"prefill_dilated: {len(rows)} rows x all heads, max err {worst:.3e}")
