"""GPU parity: swa_prefill_cached (a chunk of queries over a ring cache) and
swa_cache_append (multi-token ring write)."""

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _compare(q, kc, vc, sp, qp, W, dtype, rows=None):
    banner(f"prefill_cached {dtype} B={q.shape[0]} L={q.shape[1]} S={kc.shape[2]} W={W} "
           f"Hq={q.shape[2]} Hkv={kc.shape[1]} D={q.shape[3]}")
    o, lse = bd.prefill_cached(dev(q), dev(kc), dev(vc), dev(sp), dev(qp), W, return_lse=True)
    torch.cuda.synchronize()
    o, lse = host(o), host(lse)
    qq, spn, qpn = inp.widen(q), sp.numpy(), qp.numpy()
    if rows is not None:          # sampled (b, t) rows, all heads
        b_idx, t_idx = rows
        qq = np.stack([qq[b, t] for b, t in zip(b_idx, t_idx)])[:, None]
        o = np.stack([o[b, t] for b, t in zip(b_idx, t_idx)])[:, None]
        lse = np.stack([lse[b, :, t] for b, t in zip(b_idx, t_idx)])[:, :, None]
        kcw = np.stack([inp.widen(kc[b]) for b in b_idx])
        vcw = np.stack([inp.widen(vc[b]) for b in b_idx])
        spn = np.stack([spn[b] for b in b_idx])
        qpn = np.stack([qpn[b, t:t + 1] for b, t in zip(b_idx, t_idx)])
    else:
        kcw, vcw = inp.widen(kc), inp.widen(vc)
    ro, rl = oracle.swa_prefill_cached(qq, kcw, vcw, spn, qpn, W)
    tol, ltol = (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)
    assert max_err(o, ro) <= tol
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert max_err(lse[fin], rl[fin]) <= ltol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,S,W,Hq,Hkv,D,p_lo,p_hi", [
    (2, 37, 100, 64, 8, 2, 128, 64, 300),     # ring of W+L-1 slots, 4 heads per K/V head
    (1, 1, 256, 256, 4, 4, 64, 300, 400),     # one token: ring decode
    (3, 70, 102, 33, 4, 1, 128, 40, 90),      # ragged slot count, long chunk vs short window
    (2, 130, 629, 500, 16, 8, 64, 500, 2000),
    (2, 48, 64, 40, 4, 2, 128, 0, 10),        # ring not yet full (empty slots)
    (2, 40, 50, 40, 4, 2, 128, 100, 200),     # ring smaller than W+L-1: early queries lost keys
    (2, 64, 600, 40, 8, 2, 128, 1000, 1100),  # most slot tiles outside every window (skipped)
])
def test_cached_matches_oracle(dtype, B, L, S, W, Hq, Hkv, D, p_lo, p_hi):
    c = inp.ChunkCase(B=B, L=L, S=S, W=W, Hq=Hq, Hkv=Hkv, D=D, p_lo=p_lo, p_hi=p_hi, dtype=dtype,
                      seed=B * 131 + L + S)
    q, kc, vc, sp, qp = inp.chunk_inputs(c)
    _compare(q, kc, vc, sp, qp, W, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cached_stale_future_empty_shuffled_positions(dtype):
    B, L, S, W, Hq, Hkv, D = 3, 20, 90, 64, 8, 2, 128
    c = inp.ChunkCase(B=B, L=L, S=S, W=W, Hq=Hq, Hkv=Hkv, D=D, p_lo=200, p_hi=400, dtype=dtype,
                      seed=51)
    q, kc, vc, sp, qp = inp.chunk_inputs(c)
    sp, qp = sp.numpy().copy(), qp.numpy().copy()
    rng = np.random.default_rng(52)
    sp[0, 3] = qp[0, 0] - W          # stale for every query of the chunk
    sp[0, 4] = qp[0, -1] + 7         # future
    sp[0, 5] = -3                    # empty
    sp[1] = sp[1][rng.permutation(S)]
    qp[2] = qp[2][rng.permutation(L)]  # queries in any order
    qp[2, 4] = qp[2, 4] + 1000         # a query past every slot: empty window
    _compare(q, kc, vc, torch.from_numpy(sp), torch.from_numpy(qp), W, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_append_bit_exact(dtype):
    B, L, S, Hkv, D = 3, 13, 40, 2, 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = torch.zeros(B, Hkv, S, D, dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    ok = np.zeros((B, Hkv, S, D)); ov = np.zeros_like(ok); osp = np.full((B, S), -1)
    banner(f"cache_append {dtype}")
    p = 0
    for step in range(7):
        kn = torch.from_numpy(inp.normal((B, L, Hkv, D), 60 + step)).to(tdt)
        vn = torch.from_numpy(inp.normal((B, L, Hkv, D), 70 + step)).to(tdt)
        pos = torch.from_numpy(np.tile(np.arange(p, p + L, dtype=np.int32), (B, 1)))
        pos[1] += 5                                   # requests at different positions
        bd.cache_append(dev(kn), dev(vn), dev(pos), kc, vc, sp)
        oracle.ring_append(ok, ov, osp, inp.widen(kn), inp.widen(vn), pos.numpy())
        p += L
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), ok) and np.array_equal(host(vc), ov)
    assert np.array_equal(sp.cpu().numpy(), osp)


def test_chunks_through_ring_equal_prefill():
    # a sequence fed chunk by chunk (append, then attend) gives the prefill rows
    B, T, Hq, Hkv, D, W, L = 2, 300, 8, 2, 128, 64, 50
    S = W + L - 1
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, seed=53)
    q, k, v = inp.prefill_inputs(c)
    banner("chunks through the ring vs prefill")
    op = host(bd.prefill(dev(q), dev(k), dev(v), W))
    kc = torch.zeros(B, Hkv, S, D, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, S), -1, dtype=torch.int32, device="cuda")
    for t0 in range(0, T, L):
        pos = torch.arange(t0, t0 + L, dtype=torch.int32).repeat(B, 1)
        bd.cache_append(dev(k[:, t0:t0 + L].contiguous()), dev(v[:, t0:t0 + L].contiguous()),
                        dev(pos), kc, vc, sp)
        oc = host(bd.prefill_cached(dev(q[:, t0:t0 + L].contiguous()), kc, vc, sp, dev(pos), W))
        assert max_err(oc, op[:, t0:t0 + L]) <= TOL_BF16
    ro, _ = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W, rows=list(range(T - L, T)))
    assert max_err(oc, ro) <= TOL_BF16


def test_single_token_chunk_equals_decode():
    c = inp.DecodeCase(B=4, W=300, Hq=8, Hkv=2, D=128, cur_lo=300, cur_hi=2000, seed=54)
    q, kc, vc, sp, cur = inp.decode_inputs(c)
    banner("one-token chunk vs decode")
    od = host(bd.decode(dev(q), dev(kc), dev(vc), dev(sp), dev(cur)))
    oc = host(bd.prefill_cached(dev(q[:, None].contiguous()), dev(kc), dev(vc), dev(sp),
                                dev(cur[:, None].contiguous()), c.W))
    assert max_err(oc[:, 0], od) <= TOL_BF16
    ro, _ = oracle.swa_decode(inp.widen(q), inp.widen(kc), inp.widen(vc), sp.numpy(), cur.numpy(), c.W)
    assert max_err(oc[:, 0], ro) <= TOL_BF16


def test_cached_full_size_all_rows():
    # the timed chunked-prefill workload in the launch configuration bench.py
    # times; every (request, token) row and head against the oracle
    c = inp.C6
    q, kc, vc, sp, qp = inp.chunk_inputs(c)
    banner(f"prefill_cached full size B={c.B} L={c.L} S={c.S} W={c.W} all rows")
    o, lse = bd.prefill_cached(dev(q), dev(kc), dev(vc), dev(sp), dev(qp), c.W, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), host(lse)
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(oracle.swa_prefill_cached,
                                      (inp.widen(q), inp.widen(kc), inp.widen(vc), sp.numpy(),
                                       qp.numpy()), np.arange(c.L), dict(W=c.W)):
        e = max_err(host(o[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"tokens {rc[0]}..{rc[-1]} max err {e}"
        assert np.array_equal(np.isneginf(lse[:, :, rc]), np.isneginf(rl))
        fin = np.isfinite(rl)
        assert max_err(lse[:, :, rc][fin], rl[fin]) <= TOL_LSE_BF16, f"lse tokens {rc[0]}..{rc[-1]}"
    banner(f"prefill_cached: all {c.B * c.L} rows x all heads, max err {worst:.3e}")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,L,S,W,Hq,Hkv,D,p_lo,p_hi", [
    (2, 48, 64, 40, 4, 2, 128, 0, 10),        # ring not yet full
    (2, 37, 100, 64, 8, 2, 128, 64, 300),
    (3, 20, 130, 64, 4, 1, 64, 30, 60),       # ragged last slot tile
])
def test_cached_ignores_nonfinite_bits_of_empty_slots(dtype, B, L, S, W, Hq, Hkv, D, p_lo, p_hi):
    # Slots that hold no token (negative position) may contain any bits, e.g.
    # a cache from torch.empty: they must not reach the output.
    c = inp.ChunkCase(B=B, L=L, S=S, W=W, Hq=Hq, Hkv=Hkv, D=D, p_lo=p_lo, p_hi=p_hi, dtype=dtype,
                      seed=B * 7 + L + S)
    q, kc, vc, sp, qp = inp.chunk_inputs(c)
    spn = sp.numpy().copy()
    rng = np.random.default_rng(L + S)
    kn, vn = kc.clone(), vc.clone()
    for b in range(B):
        spn[b, rng.choice(S, size=5, replace=False)] = -1
        empty = np.nonzero(spn[b] < 0)[0]
        for i, j in enumerate(empty):
            fill = [float("nan"), float("inf"), float("-inf")][i % 3]
            kn[b, :, j] = fill
            vn[b, :, j] = fill
    _compare(q, kn, vn, torch.from_numpy(spn), qp, W, dtype)
