"""GPU parity: swa_prefill (causal sliding window) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu

# B, T, Hq, Hkv, D, W  -- ragged T, W around the 64-key tile, W >= T, W = 1,
# head packing 4 / 2 / 1 (group 4, 2, 3, 1)
SMALL = [
    (1, 16, 1, 1, 64, 4),
    (1, 16, 1, 1, 128, 16),
    (2, 300, 4, 2, 128, 70),
    (1, 257, 8, 2, 64, 256),
    (1, 200, 4, 4, 128, 1000),
    (1, 130, 2, 1, 128, 1),
    (2, 333, 8, 8, 64, 63),
    (1, 333, 8, 2, 128, 65),
    (1, 129, 32, 8, 128, 64),
    (1, 161, 12, 4, 128, 97),
    (1, 700, 4, 1, 128, 128),
    (3, 95, 6, 3, 64, 33),
]


def _run(case, dtype):
    B, T, Hq, Hkv, D, W = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype=dtype, seed=hash(case) % 1000)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill {dtype} {case}")
    o, lse = bd.prefill(dev(q), dev(k), dev(v), W, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W)
    return host(o), host(lse), ro, rl


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_prefill_bf16(case):
    o, lse, ro, rl = _run(case, "bf16")
    assert max_err(o, ro) <= TOL_BF16
    assert max_err(lse, rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("case", SMALL[:6], ids=[str(c) for c in SMALL[:6]])
def test_prefill_f32(case):
    o, lse, ro, rl = _run(case, "f32")
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_LSE_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [(1, 300, 4, 2, 128), (1, 257, 8, 2, 64)], ids=str)
def test_prefill_window_past_int_range(case, dtype):
    # W = 2^31 - 1 is full causal attention: the oracle runs at W = T
    B, T, Hq, Hkv, D = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=T, dtype=dtype, seed=3 + T)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill {dtype} W=2^31-1 {case}")
    o, lse = bd.prefill(dev(q), dev(k), dev(v), 2**31 - 1, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), T)
    tol, tol_lse = (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)
    assert max_err(host(o), ro) <= tol
    assert max_err(host(lse), rl) <= tol_lse


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,D,Hq,Hkv,W", [(16, 64, 1, 1, 1), (16, 64, 1, 1, 4), (16, 64, 1, 1, 16),
                                          (16, 64, 1, 1, 20), (128, 128, 4, 1, 1),
                                          (128, 128, 4, 1, 63), (128, 128, 4, 1, 64),
                                          (128, 128, 4, 1, 65), (128, 128, 2, 1, 100),
                                          (128, 128, 1, 1, 127), (128, 128, 1, 1, 300)])
def test_prefill_index_readout(dtype, T, D, Hq, Hkv, W):
    # q = 0 makes every attended key weigh 1/|S_t|; v_s = e_s (one-hot) makes
    # o_t's support exactly S_t, so the kernels' window is read out exactly.
    q = torch.zeros(1, T, Hq, D)
    k = torch.from_numpy(inp.normal((1, T, Hkv, D), 5))
    v = torch.zeros(1, T, Hkv, D)
    for s in range(T):
        v[0, s, :, s] = 1.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    banner(f"prefill index readout {dtype} T={T} W={W} Hq={Hq}")
    o = host(bd.prefill(dev(q.to(tdt)), dev(k.to(tdt)), dev(v.to(tdt)), W))
    for t in range(T):
        S = oracle.causal_index_set(t, W)
        for h in range(Hq):
            row = o[0, t, h]
            assert np.nonzero(row)[0].tolist() == S.tolist(), (t, h)
            np.testing.assert_allclose(row[S], 1.0 / len(S), rtol=2 ** -8)


@pytest.mark.parametrize("W", [64, 100, 128, 1000])
@pytest.mark.parametrize("inside", [False, True])
def test_prefill_boundary_adversarial(W, inside):
    # Plant a key that dominates row t's softmax just outside (k_{t-W}) or just
    # inside (k_{t-W+1}) its window: an off-by-one window moves o_t by O(1).
    B, T, Hq, Hkv, D = 1, 1100, 4, 2, 128
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, seed=77)
    q, k, v = inp.prefill_inputs(c)
    qn, kn = inp.widen(q), inp.widen(k)
    for t in range(W + 3, T, 97):
        s = t - W + (1 if inside else 0)
        for kvh in range(Hkv):
            u = qn[0, t, kvh * (Hq // Hkv)]
            kn[0, s, kvh] = 8.0 * np.sqrt(D) * u / np.linalg.norm(u)
    k = inp.as_io(kn, "bf16")
    banner(f"prefill adversarial W={W} inside={inside}")
    o = host(bd.prefill(dev(q), dev(k), dev(v), W))
    ro, _ = oracle.swa_prefill(qn, inp.widen(k), inp.widen(v), W)
    assert max_err(o, ro) <= TOL_BF16


def test_prefill_writes_only_output_and_is_deterministic():
    c = inp.PrefillCase(B=1, T=300, Hq=8, Hkv=2, D=128, W=90, seed=3)
    q, k, v = (dev(x) for x in inp.prefill_inputs(c))
    banner("prefill determinism")
    o1 = bd.prefill(q, k, v, 90)
    o2 = bd.prefill(q, k, v, 90)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    out = torch.full((2, 1, 300, 8, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    bd.prefill(q, k, v, 90, out=out[0])
    torch.cuda.synchronize()
    assert torch.equal(out[0], o1) and bool((out[1] == 7.0).all())
