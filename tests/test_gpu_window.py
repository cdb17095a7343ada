"""GPU: the kernels' windows read out exactly at the full workload sizes.

Two kinds of checks, both through the real kernels in the launch
configuration the bench times:

* Window probes (``window_probe``): keys carry the binary code of their
  position, and each query head aims at one position relative to its row (just
  inside or just outside either end of the window, the row itself, the next
  row, a global or sink position).  The aimed key dominates the softmax by
  e^22, so an off-by-one window swings an output by O(1).  Every row of every
  head is compared with the oracle (run over the host cores by
  ``oracle.pool``).
* q = 0: every weight is exactly 1, the row sum l is the integer |S_t| and lse
  = ln |S_t| to within TOL_LSE_EXACT, which separates |S_t| from |S_t| +- 1 on
  every row (the means of v are checked too).

Windows: causal t-W < s <= t ([KB] §2 "Derivation", N_t = [max(0, t-W+1), t];
[G3] "How it works"), symmetric |i-j| <= r with dilation and global tokens
([PP] §1.1, §3.1, §4.3), dilated causal {t - i d} ([KB] §2 "Dilation"), ring
slots by stored position ([KB] §2 "KV cache"; [G3] "How it works").
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_LSE_EXACT, banner, dev, host, max_err
import window_probe as wp

pytestmark = pytest.mark.gpu


def _check_rows(o_gpu, fn, arrays, rows, kwargs, what, lse_gpu=None, lse_tol=None, chunk=64):
    """Compare the GPU output rows (o_gpu: CPU tensor [B, T, H, D]) with the
    oracle's, chunk by chunk as the pool returns them."""
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(fn, arrays, rows, kwargs, chunk=chunk):
        e = max_err(host(o_gpu[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"{what}: rows {rc[0]}..{rc[-1]} max err {e}"
        if lse_gpu is not None:
            el = max_err(host(lse_gpu[:, :, rc]), rl)
            assert el <= lse_tol, f"{what}: lse rows {rc[0]}..{rc[-1]} err {el}"
    banner(f"{what}: {len(rows)} rows x all heads, max err {worst:.3e}")


# ---------------------------------------------------------------- causal probes

@pytest.mark.parametrize("cfg", ["C2", "C3"])
def test_causal_window_probe_every_row(cfg):
    c = getattr(inp, cfg)
    NB = wp.nbits(c.T)
    k = np.broadcast_to(wp.code(np.arange(c.T), NB, c.D)[None, :, None, :],
                        (c.B, c.T, c.Hkv, c.D)).copy()
    q = wp.causal_queries(c.B, c.T, c.Hq, c.D, c.W, NB)
    v = inp.normal((c.B, c.T, c.Hkv, c.D), c.seed + 21)
    qb, kb, vb = wp.bf16(q), wp.bf16(k), inp.as_io(v, "bf16")
    banner(f"causal window probe {cfg} B={c.B} T={c.T} W={c.W} Hq={c.Hq} Hkv={c.Hkv}")
    o = bd.prefill(dev(qb), dev(kb), dev(vb), c.W).cpu()
    torch.cuda.synchronize()
    _check_rows(o, oracle.swa_prefill, (inp.widen(qb), inp.widen(kb), inp.widen(vb)),
                np.arange(c.T), dict(W=c.W), f"causal probe {cfg}")


def test_dilated_window_probe_every_row():
    # the headline shape with dilation 1 / 2 / 4 on head groups (the bench's mix)
    c = inp.C2
    dil = [1] * 16 + [2] * 8 + [4] * 8
    NB = wp.nbits(c.T)
    t = np.arange(c.T)
    k = np.broadcast_to(wp.code(t, NB, c.D)[None, :, None, :], (c.B, c.T, c.Hkv, c.D)).copy()
    aims = [lambda t, d: t - (c.W - 1) * d,   # oldest key of the dilated window
            lambda t, d: t - c.W * d,         # one step past it
            lambda t, d: t,                   # the row
            lambda t, d: t + d,               # next key of the row's class (future)
            lambda t, d: t - d,
            lambda t, d: t - 1,               # another class unless d = 1
            lambda t, d: t - (c.W - 1) * d + 1,
            lambda t, d: t - (c.W + 1) * d]
    q = np.zeros((c.B, c.T, c.Hq, c.D), dtype=np.float32)
    for h in range(c.Hq):
        q[:, :, h] = wp.A * wp.code(aims[h % 8](t, dil[h]), NB, c.D)[None]
    v = inp.normal((c.B, c.T, c.Hkv, c.D), c.seed + 22)
    qb, kb, vb = wp.bf16(q), wp.bf16(k), inp.as_io(v, "bf16")
    banner(f"dilated window probe T={c.T} W={c.W} dil 1/2/4")
    o = bd.prefill_dilated(dev(qb), dev(kb), dev(vb), c.W, dil).cpu()
    torch.cuda.synchronize()
    _check_rows(o, oracle.swa_prefill, (inp.widen(qb), inp.widen(kb), inp.widen(vb)),
                np.arange(c.T), dict(W=c.W, dilation=dil), "dilated probe")


def test_sink_window_probe():
    # the headline shape with 4 sink tokens: sinks stay visible, position 4
    # (just past them) only inside the window
    c = inp.C2
    n_sink = 4
    NB = wp.nbits(c.T)
    t = np.arange(c.T)
    k = np.broadcast_to(wp.code(t, NB, c.D)[None, :, None, :], (c.B, c.T, c.Hkv, c.D)).copy()
    aims = [lambda t: 0 * t, lambda t: 0 * t + n_sink - 1, lambda t: 0 * t + n_sink,
            lambda t: t - c.W, lambda t: t - c.W + 1, lambda t: t, lambda t: t + 1,
            lambda t: 0 * t + n_sink + 1]
    q = np.zeros((c.B, c.T, c.Hq, c.D), dtype=np.float32)
    for h in range(c.Hq):
        q[:, :, h] = wp.A * wp.code(aims[h % 8](t), NB, c.D)[None]
    v = inp.normal((c.B, c.T, c.Hkv, c.D), c.seed + 23)
    qb, kb, vb = wp.bf16(q), wp.bf16(k), inp.as_io(v, "bf16")
    banner(f"sink window probe T={c.T} W={c.W} n_sink={n_sink}")
    o = bd.prefill_sinks(dev(qb), dev(kb), dev(vb), c.W, n_sink=n_sink).cpu()
    torch.cuda.synchronize()
    rng = np.random.default_rng(31)
    rows = np.unique(np.concatenate([np.arange(0, c.W + 256), np.arange(c.T - 256, c.T),
                                     rng.integers(0, c.T, 2048)]))
    _check_rows(o, oracle.swa_prefill, (inp.widen(qb), inp.widen(kb), inp.widen(vb)), rows,
                dict(W=c.W, n_sink=n_sink), "sink probe")


# ---------------------------------------------------------------- Longformer probe

@pytest.mark.parametrize("shift", [0, 4])
def test_longformer_window_probe_every_row(shift):
    c = inp.C5
    r = c.r
    dil = np.asarray(c.dilation, dtype=np.int32)
    g = np.asarray([c.globals_] * c.B, dtype=np.int32)
    NB = wp.nbits(c.T)
    i = np.arange(c.T)
    k = np.broadcast_to(wp.code(i, NB, c.D)[None, :, None, :], (c.B, c.T, c.H, c.D)).copy()
    aims = [lambda i, d: i + r * d,           # right end of the window
            lambda i, d: i + (r + 1) * d,     # one step past it
            lambda i, d: i - r * d,           # left end
            lambda i, d: i - (r + 1) * d,     # one step past it
            lambda i, d: i + r * d + 1,       # another class (d = 2) / past the end (d = 1)
            lambda i, d: 0 * i + c.globals_[-1],  # a global key (always attended)
            lambda i, d: i,
            lambda i, d: i - 1]               # another class for d = 2
    q = np.zeros((c.B, c.T, c.H, c.D), dtype=np.float32)
    for h in range(c.H):
        q[:, :, h] = wp.A * wp.code(aims[(h + shift) % 8](i, int(dil[h])), NB, c.D)[None]
    v = inp.normal((c.B, c.T, c.H, c.D), c.seed + 24)
    qb, kb, vb = wp.bf16(q), wp.bf16(k), inp.as_io(v, "bf16")
    banner(f"longformer window probe shift={shift} B={c.B} T={c.T} r={r}")
    o = bd.longformer(dev(qb), dev(kb), dev(vb), r, dil, g).cpu()
    torch.cuda.synchronize()
    _check_rows(o, oracle.swa_longformer, (inp.widen(qb), inp.widen(kb), inp.widen(vb)),
                np.arange(c.T), dict(r=r, dilation=dil, global_idx=g), f"longformer probe {shift}",
                chunk=256)


# ---------------------------------------------------------------- ring probes

def test_chunked_prefill_window_probe():
    # the chunked-prefill workload: slot keys carry the code of the position
    # they hold; the ring holds the stale position p - W for every row but the
    # first and the future position p + 1 for every row but the last
    c = inp.C6
    q0, kc, vc, sp, qp = inp.chunk_inputs(c)
    spn, qpn = sp.numpy(), qp.numpy()
    NB = 16
    kcode = np.broadcast_to(wp.code(np.maximum(spn, 0), NB, c.D)[:, None], (c.B, c.Hkv, c.S, c.D))
    p = qpn.astype(np.int64)
    offs = [-c.W + 1, -c.W, 0, 1, -c.W + 2, -1, -c.W - 1, 2]
    q = np.zeros((c.B, c.L, c.Hq, c.D), dtype=np.float32)
    for h in range(c.Hq):
        q[:, :, h] = wp.A * wp.code(p + offs[h % 8], NB, c.D)
    qb, kb = wp.bf16(q), wp.bf16(kcode)
    banner(f"chunked prefill window probe B={c.B} L={c.L} S={c.S} W={c.W}")
    o = bd.prefill_cached(dev(qb), dev(kb), dev(vc), dev(sp), dev(qp), c.W).cpu()
    torch.cuda.synchronize()
    _check_rows(o, oracle.swa_prefill_cached,
                (inp.widen(qb), inp.widen(kb), inp.widen(vc), spn, qpn), np.arange(c.L),
                dict(W=c.W), "chunked probe", chunk=16)


def test_decode_window_probe():
    # the decode workload with three slots changed per request: one holds the
    # stale position cur - W, one the future position cur + 1, one is empty
    # with a key that copies the newest key's code
    c = inp.C4
    q0, kc, vc, sp, cur = inp.decode_inputs(c)
    spn, curn = sp.numpy().copy(), cur.numpy().astype(np.int64)
    NB = 16
    for b in range(c.B):
        slot = lambda p: int(p % c.W)  # noqa: E731  (the full ring's slot of position p)
        spn[b, slot(curn[b] - c.W + 5)] = curn[b] - c.W
        spn[b, slot(curn[b] - c.W + 9)] = curn[b] + 1
        spn[b, slot(curn[b] - c.W + 13)] = -1
    codes = np.where(spn >= 0, spn, curn[:, None])           # the empty slot copies cur's code
    kcode = np.broadcast_to(wp.code(codes, NB, c.D)[:, None], (c.B, c.Hkv, c.W, c.D))
    offs = [-c.W + 1, -c.W, 0, 1, -c.W + 2, -1, -c.W + 5, -c.W + 13]
    q = np.zeros((c.B, c.Hq, c.D), dtype=np.float32)
    for h in range(c.Hq):
        q[:, h] = wp.A * wp.code(curn + offs[h % 8], NB, c.D)
    qb, kb = wp.bf16(q), wp.bf16(kcode)
    spt = torch.from_numpy(spn)
    banner(f"decode window probe B={c.B} W={c.W}")
    o, lse = bd.decode(dev(qb), dev(kb), dev(vc), dev(spt), dev(cur), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_decode(inp.widen(qb), inp.widen(kb), inp.widen(vc), spn, curn, c.W)
    assert max_err(host(o), ro) <= TOL_BF16


# ---------------------------------------------------------------- q = 0, exact lse

def _zero_q(shape_q, shape_kv, seed):
    q = torch.zeros(shape_q, dtype=torch.bfloat16)
    k = inp.as_io(inp.normal(shape_kv, seed + 11), "bf16")
    v = inp.as_io(inp.normal(shape_kv, seed + 12), "bf16")
    return q, k, v


def _prefix(x, axis):
    z = np.zeros_like(np.take(x, [0], axis=axis), dtype=np.float64)
    return np.concatenate([z, np.cumsum(x, axis=axis, dtype=np.float64)], axis=axis)


def test_dilated_zero_query_exact_counts():
    c = inp.C2
    dil = [1] * 16 + [2] * 8 + [4] * 8
    q, k, v = _zero_q((c.B, c.T, c.Hq, c.D), (c.B, c.T, c.Hkv, c.D), c.seed + 40)
    banner(f"dilated q = 0 every row T={c.T} W={c.W}")
    o, lse = bd.prefill_dilated(dev(q), dev(k), dev(v), c.W, dil, return_lse=True)
    torch.cuda.synchronize()
    vn = inp.widen(v).astype(np.float64)
    t = np.arange(c.T)
    group = c.Hq // c.Hkv
    lse_h, o_h = host(lse), o.cpu()
    for h in range(c.Hq):
        d = dil[h]
        want = np.empty((c.B, c.T, c.D))
        n = np.minimum(c.W, t // d + 1).astype(np.float64)   # |{t - i d >= 0 : i < W}|
        for rho in range(d):
            pos = np.arange(rho, c.T, d)
            cs = _prefix(vn[:, pos, h // group], axis=1)
            ci = np.arange(len(pos))
            lo = np.maximum(0, ci - c.W + 1)
            want[:, pos] = (cs[:, ci + 1] - cs[:, lo]) / (ci - lo + 1)[None, :, None]
        assert max_err(host(o_h[:, :, h]), want) <= TOL_BF16, f"head {h}"
        assert max_err(lse_h[:, h], np.log(n)[None]) <= TOL_LSE_EXACT, f"lse head {h}"


def test_sinks_zero_query_exact_counts():
    c = inp.C2
    n_sink = 4
    q, k, v = _zero_q((c.B, c.T, c.Hq, c.D), (c.B, c.T, c.Hkv, c.D), c.seed + 41)
    banner(f"sinks q = 0 every row T={c.T} W={c.W} n_sink={n_sink}")
    o, lse = bd.prefill_sinks(dev(q), dev(k), dev(v), c.W, n_sink=n_sink, return_lse=True)
    torch.cuda.synchronize()
    vn = inp.widen(v).astype(np.float64)
    t = np.arange(c.T)
    lo = np.maximum(0, t - c.W + 1)
    cs = _prefix(vn, axis=1)
    # window [lo, t] plus the sinks s < n_sink below lo
    extra = np.minimum(n_sink, lo)
    cs_sink = _prefix(vn[:, :n_sink], axis=1)
    num = cs[:, t + 1] - cs[:, lo] + cs_sink[:, extra]
    n = (t - lo + 1 + extra).astype(np.float64)
    want = num / n[None, :, None, None]
    group = c.Hq // c.Hkv
    o_h = o.cpu()
    for h in range(c.Hq):
        assert max_err(host(o_h[:, :, h]), want[:, :, h // group]) <= TOL_BF16, f"head {h}"
    assert max_err(host(lse), np.broadcast_to(np.log(n)[None, None], (c.B, c.Hq, c.T))) <= TOL_LSE_EXACT


def test_chunked_zero_query_exact_counts():
    c = inp.C6
    _, kc, vc, sp, qp = inp.chunk_inputs(c)
    q = torch.zeros(c.B, c.L, c.Hq, c.D, dtype=torch.bfloat16)
    banner(f"chunked prefill q = 0 B={c.B} L={c.L} S={c.S}")
    o, lse = bd.prefill_cached(dev(q), dev(kc), dev(vc), dev(sp), dev(qp), c.W, return_lse=True)
    torch.cuda.synchronize()
    spn, qpn = sp.numpy().astype(np.int64), qp.numpy().astype(np.int64)
    vn = inp.widen(vc).astype(np.float64)
    group = c.Hq // c.Hkv
    o_h, lse_h = host(o), host(lse)
    for b in range(c.B):
        att = (spn[b][None, :] >= 0) & (spn[b][None, :] > qpn[b][:, None] - c.W) & \
              (spn[b][None, :] <= qpn[b][:, None])                    # [L, S]
        n = att.sum(axis=1).astype(np.float64)
        for h in range(c.Hq):
            want = (att.astype(np.float64) @ vn[b, h // group]) / n[:, None]
            assert max_err(o_h[b, :, h], want) <= TOL_BF16, (b, h)
        assert max_err(lse_h[b], np.broadcast_to(np.log(n)[None], (c.Hq, c.L))) <= TOL_LSE_EXACT


def test_decode_zero_query_exact_counts():
    c = inp.C4
    _, kc, vc, sp, cur = inp.decode_inputs(c)
    spn = sp.numpy().copy()
    curn = cur.numpy().astype(np.int64)
    rng = np.random.default_rng(44)
    for b in range(c.B):   # a few stale, future and empty slots per request
        js = rng.choice(c.W, size=6, replace=False)
        spn[b, js[:2]] = curn[b] - c.W - rng.integers(0, 3, 2)
        spn[b, js[2:4]] = curn[b] + 1 + rng.integers(0, 3, 2)
        spn[b, js[4:]] = -1
    q = torch.zeros(c.B, c.Hq, c.D, dtype=torch.bfloat16)
    banner(f"decode q = 0 B={c.B} W={c.W}")
    o, lse = bd.decode(dev(q), dev(kc), dev(vc), dev(torch.from_numpy(spn)), dev(cur),
                       return_lse=True)
    torch.cuda.synchronize()
    att = (spn >= 0) & (spn > curn[:, None] - c.W) & (spn <= curn[:, None])   # [B, W]
    n = att.sum(axis=1).astype(np.float64)
    vn = inp.widen(vc).astype(np.float64)
    want = np.einsum("bw,bhwd->bhd", att.astype(np.float64), vn) / n[:, None, None]
    group = c.Hq // c.Hkv
    o_h = host(o)
    for h in range(c.Hq):
        assert max_err(o_h[:, h], want[:, h // group]) <= TOL_BF16, f"head {h}"
    assert max_err(host(lse), np.broadcast_to(np.log(n)[:, None], (c.B, c.Hq))) <= TOL_LSE_EXACT


# ------------------------------------------- 64-key tiles: windows around block edges
#
# At d_h = 64 a key tile holds two 32-key blocks, computed in turn, and a block
# outside every row of a wave is skipped.  Windows whose ends fall just before,
# on and just after 32- and 64-key boundaries move that skip between the first
# and the last tile of a wave; q = 0 reads every row's window size out exactly.

@pytest.mark.parametrize("W", [1, 31, 32, 33, 63, 64, 65, 96, 97, 128, 129, 200, 256, 257])
def test_causal_d64_zero_query_exact_counts(W):
    # two query heads per key/value head: waves at rows R and R + 32
    B, T, Hq, Hkv, D = 2, 700, 4, 2, 64
    q, k, v = _zero_q((B, T, Hq, D), (B, T, Hkv, D), 500 + W)
    banner(f"causal d64 q = 0 W={W}")
    o, lse = bd.prefill(dev(q), dev(k), dev(v), W, return_lse=True)
    torch.cuda.synchronize()
    vn = inp.widen(v).astype(np.float64)
    t = np.arange(T)
    lo = np.maximum(0, t - W + 1)
    n = (t - lo + 1).astype(np.float64)
    cs = _prefix(vn, axis=1)                                 # [B, T+1, Hkv, D]
    want = (cs[:, t + 1] - cs[:, lo]) / n[None, :, None, None]
    group = Hq // Hkv
    o_h, lse_h = host(o), host(lse)
    for h in range(Hq):
        assert max_err(o_h[:, :, h], want[:, :, h // group]) <= TOL_BF16, f"head {h}"
        assert max_err(lse_h[:, h], np.broadcast_to(np.log(n), (B, T))) <= TOL_LSE_EXACT, \
            f"lse head {h}"


@pytest.mark.parametrize("r", [1, 31, 32, 33, 63, 64, 65, 100, 128])
def test_symmetric_d64_zero_query_exact_counts(r):
    # dilations 1, 2, 3 (class lengths 600, 300, 200): bands starting and
    # ending mid-tile in every class
    B, T, H, D = 1, 600, 3, 64
    dil = [1, 2, 3]
    q, k, v = _zero_q((B, T, H, D), (B, T, H, D), 700 + r)
    banner(f"symmetric d64 q = 0 r={r}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), r, dil, return_lse=True)
    torch.cuda.synchronize()
    vn = inp.widen(v).astype(np.float64)
    o_h, lse_h = host(o), host(lse)
    for h in range(H):
        d = dil[h]
        want = np.empty((B, T, D))
        n = np.empty(T)
        for rho in range(d):
            pos = np.arange(rho, T, d)
            ci = np.arange(len(pos))
            lo = np.maximum(0, ci - r)
            hi = np.minimum(len(pos) - 1, ci + r)
            cs = _prefix(vn[:, pos, h], axis=1)
            want[:, pos] = (cs[:, hi + 1] - cs[:, lo]) / (hi - lo + 1)[None, :, None]
            n[pos] = hi - lo + 1
        assert max_err(o_h[:, :, h], want) <= TOL_BF16, f"head {h}"
        assert max_err(lse_h[:, h], np.log(n)[None]) <= TOL_LSE_EXACT, f"lse head {h}"
