"""GPU parity: attention sinks (pinned first tokens and per-head sink scores) in
causal prefill (swa_prefill_sinks), chunked prefill over a ring with pinned sink
slots (swa_prefill_cached) and the sink-aware ring append."""

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _logits(Hq, seed, scale=2.0):
    return (np.random.default_rng(seed).standard_normal(Hq) * scale).astype(np.float32)


def _tols(dtype):
    return (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,W,Hq,Hkv,D,n_sink,logits", [
    (2, 300, 64, 8, 2, 128, 4, True),     # sinks before the window of most rows
    (1, 150, 100, 4, 4, 64, 32, False),   # sinks partly inside the window (counted once)
    (1, 20, 8, 4, 2, 128, 32, True),      # more sink tokens than positions
    (1, 40, 64, 2, 1, 64, 32, True),      # W > T: every sink already in the window
    (2, 200, 1, 4, 1, 128, 3, True),      # W = 1: self plus the sinks
    (2, 260, 40, 8, 4, 128, 5, True),     # two heads per K/V head: two row blocks per workgroup
    (1, 96, 50, 4, 2, 128, 0, True),      # sink scores only
    (1, 333, 70, 4, 2, 64, 16, True),
])
def test_prefill_sinks_matches_oracle(dtype, B, T, W, Hq, Hkv, D, n_sink, logits):
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype=dtype, seed=T + W + n_sink)
    q, k, v = inp.prefill_inputs(c)
    z = _logits(Hq, T) if logits else None
    banner(f"prefill_sinks {dtype} B={B} T={T} W={W} Hq={Hq} Hkv={Hkv} D={D} n_sink={n_sink} "
           f"logits={logits}")
    o, lse = bd.prefill_sinks(dev(q), dev(k), dev(v), W, n_sink=n_sink,
                              sink_logit=None if z is None else dev(torch.from_numpy(z)),
                              return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W, n_sink=n_sink,
                                sink_logit=None if z is None else z.astype(np.float64))
    tol, ltol = _tols(dtype)
    assert max_err(host(o), ro) <= tol
    assert max_err(host(lse), rl) <= ltol


@pytest.mark.parametrize("z", [25.0, -40.0])
def test_prefill_sink_score_extremes(z):
    # a dominant sink drives o towards 0; a negligible one leaves plain SWA
    c = inp.PrefillCase(B=1, T=128, Hq=4, Hkv=2, D=128, W=32, seed=91)
    q, k, v = inp.prefill_inputs(c)
    zz = np.full(4, z, dtype=np.float32)
    banner(f"prefill sink score {z}")
    o = host(bd.prefill_sinks(dev(q), dev(k), dev(v), 32, sink_logit=dev(torch.from_numpy(zz))))
    ro, _ = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), 32,
                               sink_logit=zz.astype(np.float64))
    assert max_err(o, ro) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_append_with_sinks_bit_exact(dtype):
    B, L, S, Hkv, D, n_sink = 2, 6, 20, 2, 64, 4
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros(B, Hkv, S, D, dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    ok = np.zeros((B, Hkv, S, D)); ov = np.zeros_like(ok); osp = np.full((B, S), -1)
    banner(f"cache_append sinks {dtype}")
    for step in range(9):
        kn = torch.from_numpy(inp.normal((B, L, Hkv, D), 92 + step)).to(tdt)
        vn = torch.from_numpy(inp.normal((B, L, Hkv, D), 110 + step)).to(tdt)
        pos = torch.from_numpy(np.tile(np.arange(step * L, step * L + L, dtype=np.int32), (B, 1)))
        bd.cache_append(dev(kn), dev(vn), dev(pos), kc, vc, sp, n_sink=n_sink)
        oracle.ring_append(ok, ov, osp, inp.widen(kn), inp.widen(vn), pos.numpy(), n_sink=n_sink)
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), ok) and np.array_equal(host(vc), ov)
    assert np.array_equal(sp.cpu().numpy(), osp)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_sink_ring_chunks_equal_prefill(dtype):
    # sequence fed chunk by chunk into pinned sink slots + a rolling region of
    # W + L - 1 slots; every chunk's output equals the prefill-with-sinks rows
    B, T, Hq, Hkv, D, W, L, n_sink = 2, 260, 8, 2, 128, 48, 40, 4
    S = n_sink + W + L - 1
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype=dtype, seed=93)
    q, k, v = inp.prefill_inputs(c)
    z = _logits(Hq, 94)
    zt = dev(torch.from_numpy(z))
    banner(f"sink ring chunks vs prefill_sinks {dtype}")
    op = host(bd.prefill_sinks(dev(q), dev(k), dev(v), W, n_sink=n_sink, sink_logit=zt))
    kc = torch.zeros(B, Hkv, S, D, dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    tol = _tols(dtype)[0]
    for t0 in range(0, T, L):
        t1 = min(T, t0 + L)
        pos = torch.arange(t0, t1, dtype=torch.int32).repeat(B, 1)
        bd.cache_append(dev(k[:, t0:t1].contiguous()), dev(v[:, t0:t1].contiguous()), dev(pos),
                        kc, vc, sp, n_sink=n_sink)
        oc = host(bd.prefill_cached(dev(q[:, t0:t1].contiguous()), kc, vc, sp, dev(pos), W,
                                    n_sink=n_sink, sink_logit=zt))
        assert max_err(oc, op[:, t0:t1]) <= tol
    ro, _ = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W,
                               rows=list(range(t0, T)), n_sink=n_sink, sink_logit=z.astype(np.float64))
    assert max_err(oc, ro) <= tol


def test_prefill_sinks_full_size_row_set():
    # the timed sinks workload (headline shape, 4 sink tokens, per-head sink
    # scores) in bench.py's launch configuration: rows [0, W+256) (the ramp,
    # where the sinks lie inside the window, and the first rows whose window
    # has left them), [T-256, T) and 1024 seeded random rows, all heads
    c = inp.C2
    q, k, v = inp.prefill_inputs(c)
    z = _logits(c.Hq, 95)
    banner("prefill_sinks full size row set")
    o, lse = bd.prefill_sinks(dev(q), dev(k), dev(v), c.W, n_sink=4,
                              sink_logit=dev(torch.from_numpy(z)), return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), host(lse)
    rng = np.random.default_rng(96)
    rows = np.unique(np.concatenate([np.arange(0, c.W + 256), np.arange(c.T - 256, c.T),
                                     rng.integers(0, c.T, 1024)]))
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(oracle.swa_prefill, (inp.widen(q), inp.widen(k), inp.widen(v)),
                                      rows, dict(W=c.W, n_sink=4, sink_logit=z.astype(np.float64))):
        e = max_err(host(o[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"rows {rc[0]}..{rc[-1]} max err {e}"
        assert max_err(lse[:, :, rc], rl) <= TOL_LSE_BF16, f"lse rows {rc[0]}..{rc[-1]}"
    banner(f"prefill_sinks: {len(rows)} rows x all heads, max err {worst:.3e}")
