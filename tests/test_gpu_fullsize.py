"""GPU parity at the full workload sizes, in the launch configuration the bench
times: prefill on the rows [0, W+256) and [T-256, T) plus 4096 seeded random
rows (all heads and batch rows), decode and Longformer on every output, all
against the oracle (run over the host cores by ``oracle.pool``); and every row
with q = 0 against closed forms (exact window sizes through lse)."""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_LSE_BF16, TOL_LSE_EXACT, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _row_set(T, W, seed, n_rand=4096):
    """[0, W+256) and [T-256, T) (the ramp, the first full windows, the end)
    plus n_rand seeded random rows."""
    rng = np.random.default_rng(seed)
    rows = np.concatenate([np.arange(0, min(T, W + 256)), np.arange(max(0, T - 256), T),
                           rng.integers(0, T, size=n_rand)])
    return np.unique(rows)


def _compare_rows(o, lse, fn, arrays, rows, kwargs, what, lse_tol=TOL_LSE_BF16):
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(fn, arrays, rows, kwargs):
        e = max_err(host(o[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"{what}: rows {rc[0]}..{rc[-1]} max err {e}"
        assert max_err(host(lse[:, :, rc]), rl) <= lse_tol, f"{what}: lse rows {rc[0]}..{rc[-1]}"
    banner(f"{what}: {len(rows)} rows x all heads, max err {worst:.3e}")


@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_prefill_fullsize_row_set(cfg):
    c = getattr(inp, cfg)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill full size {cfg} B={c.B} T={c.T} W={c.W} Hq={c.Hq} Hkv={c.Hkv}")
    o, lse = bd.prefill(dev(q), dev(k), dev(v), c.W, return_lse=True)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all())
    o, lse = o.cpu(), lse.cpu()
    _compare_rows(o, lse, oracle.swa_prefill, (inp.widen(q), inp.widen(k), inp.widen(v)),
                  _row_set(c.T, c.W, 5), dict(W=c.W), f"prefill {cfg}")


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


def test_longformer_fullsize_all_outputs():
    # every output (all batch rows, rows and heads, global rows included) of
    # the full-size launch, against the oracle one batch row at a time
    c = inp.C5
    q, k, v, dl, g = inp.longformer_inputs(c)
    banner(f"longformer full size, all outputs: B={c.B} T={c.T} H={c.H} r={c.r}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), c.r, dl, g, return_lse=True)
    torch.cuda.synchronize()
    _compare_rows(o.cpu(), lse.cpu(), oracle.swa_longformer,
                  (inp.widen(q), inp.widen(k), inp.widen(v)), np.arange(c.T),
                  dict(r=c.r, dilation=dl, global_idx=g), "longformer all outputs")


# ---- every row at full size, q = 0 ----------------------------------------------
# With q = 0 every score is 0, so each row's softmax weights are uniform over its
# attended set S_t and o_t is the plain mean of v over S_t, lse_t = ln |S_t|
# (a closed form of the masked softmax: [KB] §2 window N_t, [MB] four-step
# computation).  The means come from prefix sums over the sequence, so every row
# of the full-size launch is checked, not a sample.  The expected values are
# computed here from the window definitions alone; they do not touch the oracle
# or the GPU output.

def _zero_q_bf16(shape_q, shape_kv, seed):
    q = torch.zeros(shape_q, dtype=torch.bfloat16)
    k = inp.as_io(inp.normal(shape_kv, seed + 11), "bf16")
    v = inp.as_io(inp.normal(shape_kv, seed + 12), "bf16")
    return q, k, v


def _prefix(x, axis):
    """Prefix sums along `axis` with a leading zero (float64)."""
    z = np.zeros_like(np.take(x, [0], axis=axis), dtype=np.float64)
    return np.concatenate([z, np.cumsum(x, axis=axis, dtype=np.float64)], axis=axis)


@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_prefill_fullsize_zero_query_every_row(cfg):
    c = getattr(inp, cfg)
    q, k, v = _zero_q_bf16((c.B, c.T, c.Hq, c.D), (c.B, c.T, c.Hkv, c.D), c.seed)
    banner(f"prefill full size, q = 0, every row: {cfg} B={c.B} T={c.T} W={c.W}")
    o, lse = bd.prefill(dev(q), dev(k), dev(v), c.W, return_lse=True)
    torch.cuda.synchronize()
    cs = _prefix(inp.widen(v), axis=1)                       # [B, T+1, Hkv, D]
    t = np.arange(c.T)
    lo = np.maximum(0, t - c.W + 1)                          # S_t = [lo, t]
    n = (t - lo + 1).astype(np.float64)
    mean = (cs[:, t + 1] - cs[:, lo]) / n[None, :, None, None]
    group = c.Hq // c.Hkv
    for h in range(c.Hq):
        assert max_err(host(o[:, :, h]), mean[:, :, h // group]) <= TOL_BF16, f"head {h}"
    want_lse = np.broadcast_to(np.log(n)[None, None, :], (c.B, c.Hq, c.T))
    assert max_err(host(lse), want_lse) <= TOL_LSE_EXACT


def test_longformer_fullsize_zero_query_every_row():
    c = inp.C5
    q, k, v = _zero_q_bf16((c.B, c.T, c.H, c.D), (c.B, c.T, c.H, c.D), c.seed)
    dl = np.asarray(c.dilation, dtype=np.int32)
    g = np.asarray([c.globals_] * c.B, dtype=np.int32)
    banner(f"longformer full size, q = 0, every row: B={c.B} T={c.T} H={c.H} r={c.r}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), c.r, dl, g, return_lse=True)
    torch.cuda.synchronize()
    vn = inp.widen(v).astype(np.float64)                    # [B, T, H, D]
    G = np.asarray(c.globals_)
    i = np.arange(c.T)
    for h in range(c.H):
        d = int(dl[h])
        want = np.empty((c.B, c.T, c.D))
        cnt = np.empty(c.T)
        # window {i + k d : |k| <= r} inside [0, T), as a range of each residue class
        for rho in range(d):
            pos = np.arange(rho, c.T, d)
            cs = _prefix(vn[:, pos, h], axis=1)              # [B, len+1, D]
            ci = np.arange(len(pos))
            lo, hi = np.maximum(0, ci - c.r), np.minimum(len(pos) - 1, ci + c.r)
            want[:, pos] = cs[:, hi + 1] - cs[:, lo]
            cnt[pos] = hi - lo + 1
        # union with the global positions outside the row's window
        for gp in G:
            outside = ~((np.abs(i - gp) % d == 0) & (np.abs(i - gp) // d <= c.r))
            want[:, outside] += vn[:, gp, h][:, None, :]
            cnt[outside] += 1
        # global rows attend every position
        want[:, G] = vn[:, :, h].sum(axis=1)[:, None, :]
        cnt[G] = c.T
        assert max_err(host(o[:, :, h]), want / cnt[None, :, None]) <= TOL_BF16, f"head {h}"
        want_lse = np.broadcast_to(np.log(cnt)[None, :], (c.B, c.T))
        assert max_err(host(lse[:, h]), want_lse) <= TOL_LSE_EXACT, f"lse head {h}"
