"""GPU parity: rotary positions (swa_rope) and causal prefill with fused RoPE
(swa_prefill_rope) against the fp64 oracle."""

import numpy as np
import pytest
import torch

import oracle
from oracle import pool
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,T,H,D,base,explicit", [(2, 300, 3, 128, 1e4, False),
                                                   (1, 257, 2, 64, 1e6, False),
                                                   (2, 50, 4, 128, 1e4, True),
                                                   (1, 33, 1, 64, 5e5, True)])
def test_rope_against_oracle(dtype, B, T, H, D, base, explicit):
    x = inp.as_io(inp.normal((B, T, H, D), T + H), dtype)
    pos = None
    if explicit:  # large, unsorted positions (long contexts)
        pos = torch.from_numpy(np.random.default_rng(T).integers(0, 200000, (B, T)).astype(np.int32))
    banner(f"rope {dtype} B={B} T={T} H={H} D={D} base={base} explicit={explicit}")
    y = host(bd.rope(dev(x), base, None if pos is None else dev(pos)))
    xw = inp.widen(x)
    want = np.stack([oracle.rope_rotate_half(xw[b], np.arange(T) if pos is None else pos[b].numpy(),
                                             base) for b in range(B)])
    if dtype == "bf16":
        # the result is rounded to bf16 once: within half an ulp of the exact value
        assert np.all(np.abs(y - want) <= 2.0 ** -8 * np.abs(want) + 1e-6)
    else:
        assert max_err(y, want) <= 2e-6


def test_rope_in_place_equals_out_of_place():
    x = inp.as_io(inp.normal((2, 100, 2, 128), 3), "bf16")
    banner("rope in place")
    a = bd.rope(dev(x), 1e4)
    xd = dev(x)
    bd.rope(xd, 1e4, out=xd)
    torch.cuda.synchronize()
    assert torch.equal(a, xd)


SMALL = [
    (1, 300, 4, 2, 128, 70, 1e4),
    (2, 333, 8, 2, 128, 40, 1e6),
    (1, 257, 8, 8, 64, 64, 1e4),
    (1, 129, 2, 1, 64, 1000, 1e4),
    (1, 700, 12, 4, 128, 128, 1e4),
]


def _run(case, dtype):
    B, T, Hq, Hkv, D, W, base = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype=dtype, seed=T + Hq + W)
    q, k, v = inp.prefill_inputs(c)
    banner(f"prefill_rope {dtype} {case}")
    qd, kd = dev(q), dev(k)
    o, lse = bd.prefill_rope(qd, kd, dev(v), W, base, return_lse=True)
    torch.cuda.synchronize()
    assert torch.equal(qd.cpu(), q) and torch.equal(kd.cpu(), k)  # inputs untouched
    ro, rl = oracle.swa_prefill(inp.widen(q), inp.widen(k), inp.widen(v), W, rope_base=base)
    return host(o), host(lse), ro, rl


def _lse_bound(q, k, W, base, rows=None):
    """Per-row lse tolerance of the bf16 path [B, H_q, R].  The MFMA products
    consume the rotated q and k rounded to bf16 (relative error <= 2^-9 each),
    so the score of (t, s) moves by at most scale * sum_i |q_ti k_si| *
    (2^-8 + 2^-18); lse moves by at most the largest such shift over the row's
    window, on top of the fp32 accumulation bound of the plain path."""
    B, T, Hq, D = q.shape
    group = Hq // k.shape[2]
    qr = np.abs(oracle.rope_rotate_half(inp.widen(q), np.arange(T), base))
    kr = np.abs(oracle.rope_rotate_half(inp.widen(k), np.arange(T), base))
    rows = np.arange(T) if rows is None else np.asarray(rows)
    t = rows[:, None]
    s_ = np.arange(T)[None, :]
    win = (s_ <= t) & (s_ > t - W)
    out = np.zeros((B, Hq, len(rows)))
    for b in range(B):
        for h in range(Hq):
            m = qr[b, rows, h] @ kr[b, :, h // group].T          # [R, T]
            out[b, h] = np.where(win, m, 0.0).max(axis=1)
    return TOL_LSE_BF16 + out / np.sqrt(D) * (2.0 ** -8 + 2.0 ** -18)


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_prefill_rope_bf16(case):
    o, lse, ro, rl = _run(case, "bf16")
    assert max_err(o, ro) <= TOL_BF16
    B, T, Hq, Hkv, D, W, base = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype="bf16", seed=T + Hq + W)
    q, k, _ = inp.prefill_inputs(c)
    assert np.all(np.abs(lse - rl) <= _lse_bound(q, k, W, base))


@pytest.mark.parametrize("case", SMALL, ids=[str(c) for c in SMALL])
def test_prefill_rope_equals_prefill_of_rotated_inputs(case):
    # Same arithmetic on the GPU, q rotated by swa_rope instead of in the
    # kernel's registers: the two may differ only where a rotated q element
    # rounds to a neighbouring bf16 value.
    B, T, Hq, Hkv, D, W, base = case
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, dtype="bf16", seed=T + Hq + W)
    q, k, v = (dev(x) for x in inp.prefill_inputs(c))
    banner(f"prefill_rope vs prefill(rope) {case}")
    o1, l1 = bd.prefill_rope(q, k, v, W, base, return_lse=True)
    o2, l2 = bd.prefill(bd.rope(q, base), bd.rope(k, base), v, W, return_lse=True)
    torch.cuda.synchronize()
    a, b = host(o1), host(o2)
    # outputs are bf16: allow one output rounding step (an ulp is at most
    # 2^-7 of the value) on top
    assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 1e-3)
    assert max_err(host(l1), host(l2)) <= 1e-3


@pytest.mark.parametrize("case", SMALL[:4], ids=[str(c) for c in SMALL[:4]])
def test_prefill_rope_f32(case):
    o, lse, ro, rl = _run(case, "f32")
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_LSE_F32


def test_prefill_rope_local_layer_fullsize_row_set():
    # the local-layer shape (B=2, T=32768, W=1024, H_q=32, H_kv=16) with the
    # rotation done inside the call instead of by the input generator; rows
    # [0, W+256), [T-256, T) and 4096 seeded random rows, all heads
    c = inp.PrefillCase(B=2, T=32768, Hq=32, Hkv=16, D=128, W=1024, seed=1002)
    q, k, v = inp.prefill_inputs(c)
    banner("prefill_rope local-layer full size")
    o, lse = bd.prefill_rope(dev(q), dev(k), dev(v), c.W, 1e4, return_lse=True)
    torch.cuda.synchronize()
    o, lse = o.cpu(), host(lse)
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([np.arange(0, c.W + 256), np.arange(c.T - 256, c.T),
                                     rng.integers(0, c.T, 4096)]))
    # the oracle's rotation (fp64) of k at every position and of q at the
    # compared rows, then the oracle's plain prefill over those rows: the same
    # as oracle.swa_prefill(..., rope_base=1e4) on them
    k_rot = oracle.rope_rotate_half(inp.widen(k), np.arange(c.T), 1e4)
    q_rot = np.zeros(q.shape, dtype=np.float64)
    q_rot[:, rows] = oracle.rope_rotate_half(inp.widen(q)[:, rows], rows, 1e4)
    # lse bound of _lse_bound with sum_i |q_i k_i| <= |q| |k| (Cauchy-Schwarz)
    # and the largest |k_s| of the row's window
    qn = np.linalg.norm(q_rot[:, rows], axis=-1)                 # [B, R, Hq]
    kn = np.linalg.norm(k_rot, axis=-1)                          # [B, T, Hkv]
    pad = np.concatenate([np.zeros((c.B, c.W - 1, c.Hkv)), kn], axis=1)
    kmax = np.lib.stride_tricks.sliding_window_view(pad, c.W, axis=1).max(axis=-1)  # [B, T, Hkv]
    group = c.Hq // c.Hkv
    bound = TOL_LSE_BF16 + (qn * np.repeat(kmax[:, rows], group, axis=2)).transpose(0, 2, 1) \
        / np.sqrt(c.D) * (2.0 ** -8 + 2.0 ** -18)                # [B, Hq, R]
    pos = {int(t): i for i, t in enumerate(rows)}
    worst = 0.0
    for rc, (ro, rl) in pool.run_rows(oracle.swa_prefill, (q_rot, k_rot, inp.widen(v)), rows,
                                      dict(W=c.W)):
        e = max_err(host(o[:, rc]), ro)
        worst = max(worst, e)
        assert e <= TOL_BF16, f"rows {rc[0]}..{rc[-1]} max err {e}"
        ix = [pos[int(t)] for t in rc]
        assert np.all(np.abs(lse[:, :, rc] - rl) <= bound[:, :, ix]), f"lse rows {rc[0]}..{rc[-1]}"
    banner(f"prefill_rope local-layer: {len(rows)} rows x all heads, max err {worst:.3e}")
