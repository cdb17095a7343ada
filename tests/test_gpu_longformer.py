"""GPU parity: swa_longformer (symmetric window, dilation, global tokens) and the
device-side window predicate, against the oracle."""

import os

import numpy as np
import pytest
import torch

import oracle
from sliding_window_attention_amd import binding as bd
from sliding_window_attention_amd import inputs as inp
from gpu_util import TOL_BF16, TOL_F32, TOL_LSE_BF16, TOL_LSE_F32, banner, dev, host, max_err

pytestmark = pytest.mark.gpu
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# B, T, H, D, r, dilation, globals
SMALL = [
    (1, 16, 1, 64, 2, [1], []),
    (1, 16, 2, 64, 2, [1, 2], [[0, 8]]),
    (2, 300, 4, 64, 20, [1, 2, 3, 1], [[0, 77], [5, 299]]),
    (2, 300, 4, 128, 20, [1, 2, 3, 1], [[10, 11], [0, 1]]),
    (1, 257, 3, 64, 0, [1, 2, 5], [[128]]),
    (1, 200, 2, 64, 300, [1, 2], []),
    (2, 520, 4, 64, 64, [1, 1, 2, 2], [[0, 8], [200, 519]]),
    (1, 129, 2, 128, 63, [4, 1], [[3, 64, 65, 100]]),
    (1, 90, 2, 64, 5, [100, 1], [[0]]),
    # 16 < G <= 32: two 16-row passes of the global-row block states, global
    # keys added after the band
    (1, 300, 2, 64, 9, [1, 3], [list(range(0, 300, 12))]),
    (1, 200, 2, 128, 30, [2, 1], [list(range(1, 200, 7))]),
    # more than 32 global tokens: the tile-of-global-keys path with shared projections
    (1, 300, 2, 64, 9, [1, 3], [list(range(0, 300, 7))]),
    (2, 260, 2, 128, 20, [2, 1], [list(range(3, 260, 6)), list(range(0, 43))]),
]


def _run(case, dtype):
    B, T, H, D, r, dil, gl = case
    c = inp.LongformerCase(B=B, T=T, H=H, D=D, r=r, dilation=dil,
                           globals_=gl[0] if gl else [], dtype=dtype, seed=T + 7 * H)
    q, k, v, dl, _ = inp.longformer_inputs(c)
    g = np.asarray(gl, dtype=np.int32).reshape(B, -1) if gl else None
    if g is not None and g.shape[0] != B:
        g = np.repeat(g, B, axis=0)
    banner(f"longformer {dtype} {case}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), r, dl, g, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), r, dl, g)
    return host(o), host(lse), ro, rl


@pytest.mark.parametrize("case", SMALL, ids=[str(c[:5]) for c in SMALL])
def test_longformer_bf16(case):
    o, lse, ro, rl = _run(case, "bf16")
    assert max_err(o, ro) <= TOL_BF16
    assert max_err(lse, rl) <= TOL_LSE_BF16


@pytest.mark.parametrize("case", SMALL, ids=[str(c[:5]) for c in SMALL])
def test_longformer_f32(case):
    o, lse, ro, rl = _run(case, "f32")
    assert max_err(o, ro) <= TOL_F32
    assert max_err(lse, rl) <= TOL_LSE_F32


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", [(1, 200, 2, 64, [1, 3], [[0, 150]]),
                                  (2, 129, 2, 128, [2, 1], [])], ids=str)
def test_longformer_radius_past_the_sequence(case, dtype):
    # r = 2^31 - 1 (where i + r leaves 32-bit range) reaches every key of the
    # row's class, as r = T does; the oracle runs at r = T
    B, T, H, D, dil, gl = case
    c = inp.LongformerCase(B=B, T=T, H=H, D=D, r=T, dilation=dil,
                           globals_=gl[0] if gl else [], dtype=dtype, seed=5 + T)
    q, k, v, dl, _ = inp.longformer_inputs(c)
    g = np.repeat(np.asarray(gl, dtype=np.int32).reshape(1, -1), B, axis=0) if gl else None
    banner(f"longformer {dtype} r=2^31-1 {case}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), 2**31 - 1, dl, g, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), T, dl, g)
    tol, tol_lse = (TOL_BF16, TOL_LSE_BF16) if dtype == "bf16" else (TOL_F32, TOL_LSE_F32)
    assert max_err(host(o), ro) <= tol
    assert max_err(host(lse), rl) <= tol_lse


def _class_blocks(T, dil, n=32):
    return sum(-(-len(range(rho, T, dil)) // n) for rho in range(dil))


# The bf16 global rows come from per-block partial states when the workspace
# holds them, else from a split-KV pass: both against the oracle and each other.
@pytest.mark.parametrize("case", [
    (2, 300, 4, 64, 20, [1, 2, 3, 1], [[0, 77], [5, 299]]),
    (1, 129, 2, 128, 63, [4, 1], [[3, 64, 65, 100]]),
    (1, 300, 2, 64, 9, [1, 3], [list(range(0, 300, 7))]),
    (1, 200, 2, 128, 30, [2, 1], [list(range(1, 200, 7))]),
], ids=["d64", "d128", "43globals", "29globals_d128"])
def test_longformer_global_rows_both_paths(case):
    B, T, H, D, r, dil, gl = case
    c = inp.LongformerCase(B=B, T=T, H=H, D=D, r=r, dilation=dil, globals_=gl[0], dtype="bf16",
                           seed=T + 11 * H)
    q, k, v, dl, _ = inp.longformer_inputs(c)
    g = np.repeat(np.asarray(gl, dtype=np.int32).reshape(len(gl), -1), B // len(gl), axis=0)
    G = g.shape[1]
    nb = max(_class_blocks(T, d) for d in dl)
    block_bytes = B * H * G * nb * (D + 4) * 4
    banner(f"longformer global-row paths {case[:5]} G={G}")
    qd, kd, vd = dev(q), dev(k), dev(v)
    ws_full = torch.empty(bd.longformer_workspace_size(B, T, H, D, G), dtype=torch.uint8, device="cuda")
    ws_small = torch.empty(block_bytes - 256, dtype=torch.uint8, device="cuda")
    o1, l1 = bd.longformer(qd, kd, vd, r, dl, g, workspace=ws_full, return_lse=True)
    o2, l2 = bd.longformer(qd, kd, vd, r, dl, g, workspace=ws_small, return_lse=True)
    torch.cuda.synchronize()
    ro, rl = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), r, dl, g)
    for o, lse in ((o1, l1), (o2, l2)):
        assert max_err(host(o), ro) <= TOL_BF16
        assert max_err(host(lse), rl) <= TOL_LSE_BF16
    rows = g[0]
    assert max_err(host(o1)[:, rows], host(o2)[:, rows]) <= TOL_BF16


# B, T, H, D, r, dilation, globals (separate global projections)
PROJ = [
    (1, 16, 2, 64, 2, [1, 2], [[0, 8]]),
    (2, 300, 4, 64, 20, [1, 2, 3, 1], [[0, 77], [5, 299]]),
    (2, 300, 2, 128, 20, [1, 2], [[10, 11], [0, 1]]),
    (1, 129, 2, 128, 63, [4, 1], [[3, 64, 65, 100]]),
    (2, 520, 4, 64, 64, [1, 1, 2, 2], [[0, 8], [200, 519]]),
    (1, 200, 2, 64, 300, [1, 2], [[7]]),
]


def _run_proj(case, dtype):
    B, T, H, D, r, dil, gl = case
    c = inp.LongformerCase(B=B, T=T, H=H, D=D, r=r, dilation=dil, globals_=[], dtype=dtype,
                           seed=3 * T + H)
    q, k, v, dl, _ = inp.longformer_inputs(c)
    # the global projections: independent seeded draws of the same shape
    qg, kg, vg = (inp.as_io(inp.normal(q.shape, c.seed + 101 + i), dtype) for i in range(3))
    g = np.asarray(gl, dtype=np.int32).reshape(B, -1)
    banner(f"longformer_proj {dtype} {case}")
    o, lse = bd.longformer(dev(q), dev(k), dev(v), r, dl, g, return_lse=True,
                           qg=dev(qg), kg=dev(kg), vg=dev(vg))
    torch.cuda.synchronize()
    W = inp.widen
    ro, rl = oracle.swa_longformer(W(q), W(k), W(v), r, dl, g, qg=W(qg), kg=W(kg), vg=W(vg))
    return host(o), host(lse), ro, rl


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("case", PROJ, ids=[str(c[:5]) for c in PROJ])
def test_longformer_separate_projections(case, dtype):
    o, lse, ro, rl = _run_proj(case, dtype)
    assert max_err(o, ro) <= (TOL_BF16 if dtype == "bf16" else TOL_F32)
    assert max_err(lse, rl) <= (TOL_LSE_BF16 if dtype == "bf16" else TOL_LSE_F32)


def test_longformer_proj_with_shared_tensors_is_longformer():
    # qg, kg, vg = q, k, v must reproduce the shared-projection call exactly
    # (the same arithmetic on the same operands).
    c = inp.LongformerCase(B=2, T=300, H=4, D=64, r=20, dilation=[1, 2, 3, 1], globals_=[],
                           dtype="bf16", seed=5)
    q, k, v, dl, _ = inp.longformer_inputs(c)
    g = np.asarray([[0, 77], [5, 299]], dtype=np.int32)
    banner("longformer_proj shared == longformer")
    a = bd.longformer(dev(q), dev(k), dev(v), c.r, dl, g)
    b = bd.longformer(dev(q), dev(k), dev(v), c.r, dl, g, qg=dev(q), kg=dev(k), vg=dev(v))
    torch.cuda.synchronize()
    ro, _ = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), c.r, dl, g)
    assert max_err(host(b), ro) <= TOL_BF16
    assert max_err(host(a), host(b)) <= 2 ** -7


def test_small_symmetric_workload_fp32():
    # n=16, r=2, d_h=64, float32, one head: the running example's shape
    c = inp.C1
    q, k, v, dl, _ = inp.longformer_inputs(c)
    banner("longformer n16 r2 fp32")
    o = host(bd.longformer(dev(q), dev(k), dev(v), c.r, dl, None))
    ro, _ = oracle.swa_longformer(inp.widen(q), inp.widen(k), inp.widen(v), c.r, dl, None)
    assert max_err(o, ro) <= TOL_F32


def _readout(dtype, r, dil, glist, n=16, D=64):
    q = torch.zeros(1, n, 1, D)
    k = torch.from_numpy(inp.normal((1, n, 1, D), 21))
    v = torch.zeros(1, n, 1, D)
    for s in range(n):
        v[0, s, 0, s] = 1.0
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    g = np.asarray([glist], dtype=np.int32) if glist else None
    o = host(bd.longformer(dev(q.to(tdt)), dev(k.to(tdt)), dev(v.to(tdt)), r, [dil], g))
    return o[0, :, 0]


def _table(name):
    rows = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.strip()
        if line and not line.startswith("#") and not line.startswith("total"):
            i, vals = line.split(":")
            rows[int(i)] = [int(x) for x in vals.split()]
    return rows


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("name,r,dil,gl,total", [
    ("pp_symmetric_n16_r2.txt", 2, 1, [], 74),
    ("pp_dilated_n16_r2_d2.txt", 2, 2, [], 68),
    ("pp_global_n16_r2_G0_8.txt", 2, 1, [0, 8], 120),
])
def test_index_readout_printed_tables(dtype, name, r, dil, gl, total):
    # q = 0 and one-hot v read the kernels' connectivity sets out exactly; they
    # must be the printed tables, row by row, and sum to the printed totals.
    banner(f"longformer readout {dtype} {name}")
    o = _readout(dtype, r, dil, gl)
    table = _table(name)
    count = 0
    for i in range(16):
        sup = np.nonzero(o[i])[0].tolist()
        count += len(sup)
        assert sup == oracle.longformer_index_set(i, 16, r, dil, gl).tolist()
        if i in table:
            assert sup == table[i]
        np.testing.assert_allclose(o[i][sup], 1.0 / len(sup), rtol=2 ** -8)
    assert count == total


@pytest.mark.parametrize("mode,T,w,dil,gl", [
    (0, 300, 70, 1, []), (0, 257, 1, 1, []), (0, 100, 500, 1, []),
    (1, 300, 20, 1, []), (1, 300, 20, 3, [0, 77, 299]), (1, 257, 64, 2, [128]),
    (1, 16, 2, 2, []), (1, 16, 2, 1, [0, 8]),
    # a window or radius of 2^31 - 1 covers everything, as w = T does
    (0, 100, 2**31 - 1, 1, []), (1, 100, 2**31 - 1, 3, [5]),
])
def test_device_predicate_matches_oracle(mode, T, w, dil, gl):
    banner(f"debug mask mode={mode} T={T} w={w} dil={dil}")
    m = bd.debug_index_mask(mode, T, w, dil, gl).cpu().numpy().astype(bool)
    w = min(w, T)
    want = oracle.causal_mask(T, w) if mode == 0 else oracle.longformer_mask(T, w, dil, gl)
    assert np.array_equal(m, want)
