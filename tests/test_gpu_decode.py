"""GPU parity: swa_decode over the ring cache and swa_cache_write."""

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu


def _compare(q, kc, vc, sp, cur, W, dtype):
    banner(f"decode {dtype} B={q.shape[0]} W={W} Hq={q.shape[1]} Hkv={kc.shape[1]} D={q.shape[2]}")
    o, lse = bd.decode(dev(q), dev(kc), dev(vc), dev(sp), dev(cur), return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_decode(inp.widen(q), inp.widen(kc), inp.widen(vc), sp.numpy(),
                               cur.numpy(), W)
    tol, ltol = (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)
    assert max_err(host(o), ro) <= tol
    lse = host(lse)
    assert np.array_equal(np.isneginf(lse), np.isneginf(rl))
    fin = np.isfinite(rl)
    assert max_err(lse[fin], rl[fin]) <= ltol


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,W,Hq,Hkv,D", [(3, 8, 8, 2, 128), (2, 64, 4, 4, 64), (3, 100, 8, 2, 128),
                                          (2, 600, 32, 8, 128), (1, 1000, 12, 4, 64),
                                          (5, 513, 16, 1, 128)])
def test_decode_full_ring(dtype, B, W, Hq, Hkv, D):
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=W, cur_hi=8 * W, dtype=dtype,
                       seed=B * 31 + W)
    q, kc, vc, sp, cur = inp.decode_inputs(c)
    _compare(q, kc, vc, sp, cur, W, dtype)


# Batches with many (request, kv head) groups: the bf16 path then runs one
# workgroup per group whose waves split the ring and merge in LDS (1, 2, 4 or
# 8 waves by group count); cur_lo = 0 leaves some rings partly filled, and
# W = 600 over 8 waves leaves the last wave an empty split.
@pytest.mark.parametrize("B,W,Hq,Hkv,D,cur_lo", [
    (256, 100, 16, 8, 128, 100),   # 2048 groups: one wave each
    (128, 100, 8, 8, 128, 0),      # 1024 groups: two waves
    (64, 700, 32, 8, 128, 0),      # 512 groups: four waves
    (32, 600, 16, 4, 128, 300),    # 128 groups: eight waves, last split empty
    (32, 600, 32, 4, 64, 0),       # eight query heads per kv head
    (16, 333, 96, 8, 128, 0),      # twelve query heads per kv head: two passes
])
def test_decode_workgroup_merge(B, W, Hq, Hkv, D, cur_lo):
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=cur_lo, cur_hi=4 * W, seed=B + W + Hq)
    q, kc, vc, sp, cur = inp.decode_inputs(c)
    _compare(q, kc, vc, sp, cur, W, "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_partial_stale_future_shuffled(dtype):
    B, W, Hq, Hkv, D = 6, 96, 8, 2, 128
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=0, cur_hi=3 * W, dtype=dtype, seed=11)
    q, kc, vc, _, _ = inp.decode_inputs(c)
    rng = np.random.default_rng(12)
    cur = np.array([0, 5, 95, 96, 150, 287], dtype=np.int32)
    sp = inp.full_ring_positions(cur, W)          # rows 0..2: partially filled rings
    sp[3, 7] = 96 - W                              # stale: exactly one window behind
    sp[4, 10] = 150 + 3                            # future position
    sp[4, 11] = -5                                 # empty
    sp[5] = sp[5][rng.permutation(W)]              # positions shuffled over slots
    _compare(q, kc, vc, torch.from_numpy(sp), torch.from_numpy(cur), W, dtype)


def test_decode_empty_ring_gives_zero():
    B, W, Hq, Hkv, D = 2, 64, 4, 2, 128
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=0, cur_hi=10, seed=13)
    q, kc, vc, _, cur = inp.decode_inputs(c)
    sp = torch.full((B, W), -1, dtype=torch.int32)
    banner("decode empty ring")
    o, lse = bd.decode(dev(q), dev(kc), dev(vc), dev(sp), dev(cur), return_lse=True)
    torch.cuda.synchronize()
    assert bool((o == 0).all()) and bool(torch.isneginf(lse).all())


def test_decode_equals_prefill_row():
    # A ring filled by the write rule from a sequence gives the prefill row of
    # the current position (both on the GPU, both against the oracle).
    B, T, Hq, Hkv, D, W = 3, 400, 8, 2, 128, 128
    c = inp.PrefillCase(B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, W=W, seed=14)
    q, k, v = inp.prefill_inputs(c)
    cur = np.array([7, 200, 399])
    kc, vc, sp = oracle.ring_from_sequence(inp.widen(k), inp.widen(v), cur, W)
    kc_t = torch.from_numpy(kc.astype(np.float32)).to(torch.bfloat16)
    vc_t = torch.from_numpy(vc.astype(np.float32)).to(torch.bfloat16)
    qd = torch.stack([q[b, int(cur[b])] for b in range(B)])
    banner("decode vs prefill row")
    od = host(bd.decode(dev(qd), dev(kc_t), dev(vc_t), dev(torch.from_numpy(sp.astype(np.int32))),
                        dev(torch.from_numpy(cur.astype(np.int32)))))
    op = host(bd.prefill(dev(q), dev(k), dev(v), W))
    for b in range(B):
        ro, _ = oracle.swa_prefill(inp.widen(q[b:b + 1]), inp.widen(k[b:b + 1]),
                                   inp.widen(v[b:b + 1]), W, rows=[cur[b]])
        assert max_err(od[b], ro[0, 0]) <= TOL_BF16
        assert max_err(od[b], op[b, cur[b]]) <= TOL_BF16


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_cache_write_then_decode(dtype):
    # Append tokens one by one with swa_cache_write (slot = pos mod W) and check
    # the ring bit for bit against the oracle's write rule, then decode.
    B, T, Hkv, Hq, D, W = 2, 70, 2, 4, 64, 16
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    seq_k = torch.from_numpy(inp.normal((B, T, Hkv, D), 15)).to(tdt)
    seq_v = torch.from_numpy(inp.normal((B, T, Hkv, D), 16)).to(tdt)
    kc = torch.zeros(B, Hkv, W, D, dtype=tdt, device="cuda")
    vc = torch.zeros_like(kc)
    sp = torch.full((B, W), -1, dtype=torch.int32, device="cuda")
    ok = np.zeros((B, Hkv, W, D)); ov = np.zeros_like(ok); osp = np.full((B, W), -1)
    banner(f"cache write {dtype}")
    for p in range(T):
        pos = torch.full((B,), p, dtype=torch.int32)
        bd.cache_write(dev(seq_k[:, p].contiguous()), dev(seq_v[:, p].contiguous()), dev(pos),
                       kc, vc, sp)
        oracle.ring_write(ok, ov, osp, inp.widen(seq_k[:, p]), inp.widen(seq_v[:, p]), pos.numpy())
    torch.cuda.synchronize()
    assert np.array_equal(host(kc), ok) and np.array_equal(host(vc), ov)
    assert np.array_equal(sp.cpu().numpy(), osp)
    q = torch.from_numpy(inp.normal((B, Hq, D), 17)).to(tdt)
    _compare(q, kc.cpu(), vc.cpu(), sp.cpu(), torch.full((B,), T - 1, dtype=torch.int32), W, dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("B,W,Hq,Hkv,D", [(4, 200, 8, 2, 128), (64, 512, 32, 8, 128),
                                          (3, 96, 4, 4, 64)])
def test_decode_ignores_nonfinite_bits_of_unattended_slots(dtype, B, W, Hq, Hkv, D):
    # Empty, stale and future slots are outside the window: whatever bits they
    # hold (NaN, Inf) must not reach the output ([KB] §2 "KV cache": only the
    # positions of the window are attended).
    c = inp.DecodeCase(B=B, W=W, Hq=Hq, Hkv=Hkv, D=D, cur_lo=0, cur_hi=3 * W, dtype=dtype,
                       seed=B + W + D)
    q, kc, vc, sp, cur = inp.decode_inputs(c)
    spn = sp.numpy().copy()
    curn = cur.numpy().astype(np.int64)
    rng = np.random.default_rng(B * W)
    kn, vn = kc.clone(), vc.clone()
    for b in range(B):
        js = rng.choice(W, size=9, replace=False)
        spn[b, js[:3]] = -1                                    # empty
        spn[b, js[3:6]] = curn[b] - W - rng.integers(0, 5, 3)  # stale
        spn[b, js[6:]] = curn[b] + 1 + rng.integers(0, 5, 3)   # future
        bad = np.nonzero((spn[b] < 0) | (spn[b] <= curn[b] - W) | (spn[b] > curn[b]))[0]
        for i, j in enumerate(bad):
            fill = [float("nan"), float("inf"), float("-inf")][i % 3]
            kn[b, :, j] = fill
            vn[b, :, j] = fill
    _compare(q, kn, vn, torch.from_numpy(spn), cur, W, dtype)
