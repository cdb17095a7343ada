"""Host-side checks of libswa.so (no GPU needed, no compute launched).

- the library loads and exports every function include/swa.h declares;
- argument validation returns the documented status before any HIP call;
- the band-tile schedule the kernels run matches the oracle's brute-force
  tile classification bit for bit.
"""

import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from sliding_window_attention_amd import binding as bd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "swa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, 1, 2, 3
P = ctypes.c_void_p(4096)  # aligned fake device pointer; never dereferenced on error paths
S0 = ctypes.c_void_p(0)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(swa_[a-z_0-9]+)\s*\(", text)))


def test_exports_every_declared_symbol():
    L = bd.lib()
    names = _declared()
    assert len(names) >= 10
    for n in names:
        assert hasattr(L, n), n
    assert L.swa_version() == 1


def test_status_strings():
    for c in range(5):
        assert bd.status_str(c)


def _prefill(**kw):
    a = dict(dt=0, q=P, k=P, v=P, o=P, lse=None, B=1, T=16, Hq=4, Hkv=2, D=128, W=8, sc=0.1)
    a.update(kw)
    return bd.lib().swa_prefill(a["dt"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["T"],
                                a["Hq"], a["Hkv"], a["D"], a["W"], a["sc"], S0)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(o=None), INVALID), (dict(q=ctypes.c_void_p(4098)), INVALID),
    (dict(lse=ctypes.c_void_p(4098)), INVALID),
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(W=0), INVALID), (dict(Hq=3), INVALID),
    (dict(Hkv=0), INVALID), (dict(sc=0.0), INVALID), (dict(sc=float("nan")), INVALID),
    (dict(sc=float("inf")), INVALID), (dict(dt=7), INVALID), (dict(D=96), UNSUPPORTED),
    (dict(D=256), UNSUPPORTED),
])
def test_prefill_validation(kw, code):
    assert _prefill(**kw) == code


def _decode(ws_bytes=None, **kw):
    a = dict(dt=0, B=2, W=64, Hq=8, Hkv=2, D=128, sc=0.1, sp=P, cur=P, ws=P)
    a.update(kw)
    need = bd.lib().swa_decode_workspace_size(a["B"], a["Hq"], a["Hkv"], a["W"], a["D"])
    nb = need if ws_bytes is None else ws_bytes
    return bd.lib().swa_decode(a["dt"], P, P, P, a["sp"], a["cur"], P, None, a["B"], a["W"],
                               a["Hq"], a["Hkv"], a["D"], a["sc"], a["ws"], nb, S0)


def test_decode_validation():
    assert bd.lib().swa_decode_workspace_size(2, 8, 2, 64, 128) > 0
    assert _decode(sp=None) == INVALID
    assert _decode(cur=ctypes.c_void_p(4098)) == INVALID
    assert _decode(W=0) == INVALID
    assert _decode(Hq=7) == INVALID
    assert _decode(D=32) == UNSUPPORTED
    assert _decode(ws_bytes=16) == WORKSPACE
    assert _decode(ws=None) == WORKSPACE


def _lf(dil=None, gl=None, G=0, ws_bytes=1 << 30, **kw):
    a = dict(dt=0, B=2, T=64, H=3, D=64, r=4, sc=0.1)
    a.update(kw)
    dp = None if dil is None else (ctypes.c_int32 * len(dil))(*dil)
    gp = None if gl is None else (ctypes.c_int32 * len(gl))(*gl)
    return bd.lib().swa_longformer(a["dt"], P, P, P, P, None, a["B"], a["T"], a["H"], a["D"],
                                   a["r"], dp, gp, G, a["sc"], P, ws_bytes, S0)


def test_longformer_validation():
    assert _lf(r=-1) == INVALID
    assert _lf(dil=[1, 0, 2]) == INVALID
    assert _lf(dil=[1, 70000, 2]) == INVALID
    assert _lf(gl=[0, 8, 9, 9], G=2) == INVALID          # not strictly increasing
    assert _lf(gl=[0, 64, 1, 2], G=2) == INVALID         # out of range
    assert _lf(gl=[3, 1, 1, 2], G=2) == INVALID          # decreasing
    assert _lf(gl=None, G=2) == INVALID
    assert _lf(gl=[0, 1, 2, 3], G=0) == INVALID
    assert _lf(D=80) == UNSUPPORTED
    assert _lf(H=300, dil=None) == UNSUPPORTED
    assert _lf(gl=[0, 8, 0, 8], G=2, ws_bytes=8) == WORKSPACE
    assert bd.lib().swa_longformer_workspace_size(2, 64, 3, 64, 0) == 0


def _class_blocks(T, dil, n=32):
    """32-key blocks over the residue classes of one head: sum over classes of
    ceil(class length / 32)."""
    return sum(-(-len(range(rho, T, dil)) // n) for rho in range(dil))


@pytest.mark.parametrize("B,T,H,D,G", [(2, 64, 3, 64, 2), (8, 4096, 12, 64, 2), (1, 90, 2, 128, 5),
                                       (3, 1000, 4, 128, 40)])
def test_longformer_workspace_holds_block_states(B, T, H, D, G):
    # the reported size holds one record of D + 4 floats per (batch, head,
    # global row, 32-key block) for every head dilation up to 16
    cap = max(_class_blocks(T, d) for d in range(1, 17))
    assert bd.lib().swa_longformer_workspace_size(B, T, H, D, G) >= B * H * G * cap * (D + 4) * 4


def _lfp(qg=P, kg=P, vg=P, **kw):
    a = dict(dt=0, B=2, T=64, H=3, D=64, r=4, sc=0.1, G=2)
    a.update(kw)
    gp = (ctypes.c_int32 * 4)(0, 8, 0, 8)
    return bd.lib().swa_longformer_proj(a["dt"], P, P, P, qg, kg, vg, P, None, a["B"], a["T"],
                                        a["H"], a["D"], a["r"], None, gp, a["G"], a["sc"], P,
                                        1 << 30, S0)


def test_prefill_dilated_validation():
    L = bd.lib()

    def call(dil, Hq=4, Hkv=2, D=128, W=8):
        dp = None if dil is None else (ctypes.c_int32 * len(dil))(*dil)
        return L.swa_prefill_dilated(0, P, P, P, P, None, 1, 16, Hq, Hkv, D, W, dp, 0.1, S0)

    assert call([1, 0, 2, 2]) == INVALID
    assert call([1, 70000, 2, 2]) == INVALID
    assert call([1, 2, 2, 2], W=0) == INVALID
    assert call([1, 2, 2, 2], Hq=3, Hkv=2) == INVALID
    assert call([1, 2, 2, 2], D=96) == UNSUPPORTED
    assert call([1, 2] * 150, Hq=300, Hkv=1) == UNSUPPORTED  # 300 single-head groups


def test_rope_validation():
    L = bd.lib()
    assert L.swa_rope(0, None, P, None, 1, 8, 2, 64, 1e4, S0) == INVALID
    assert L.swa_rope(0, P, P, ctypes.c_void_p(4098), 1, 8, 2, 64, 1e4, S0) == INVALID
    assert L.swa_rope(0, P, P, None, 1, 8, 2, 64, 0.0, S0) == INVALID
    assert L.swa_rope(0, P, P, None, 1, 8, 2, 64, float("inf"), S0) == INVALID
    assert L.swa_rope(0, P, P, None, 0, 8, 2, 64, 1e4, S0) == INVALID
    assert L.swa_rope(0, P, P, None, 1, 8, 2, 80, 1e4, S0) == UNSUPPORTED
    need = L.swa_prefill_rope_workspace_size(0, 2, 64, 3, 128)
    assert need == 2 * 64 * 3 * 128 * 2
    assert L.swa_prefill_rope_workspace_size(1, 2, 64, 3, 128) == 2 * need

    def pr(ws_bytes=need, base=1e4, **kw):
        a = dict(Hq=6, Hkv=3, W=8, D=128)
        a.update(kw)
        return L.swa_prefill_rope(0, P, P, P, P, None, 2, 64, a["Hq"], a["Hkv"], a["D"], a["W"],
                                  base, 0.1, P, ws_bytes, S0)

    assert pr(base=-1.0) == INVALID
    assert pr(W=0) == INVALID
    assert pr(Hq=5) == INVALID
    assert pr(D=96) == UNSUPPORTED
    assert pr(ws_bytes=need - 1) == WORKSPACE


def test_longformer_proj_validation():
    assert _lfp(qg=None) == INVALID
    assert _lfp(kg=None) == INVALID
    assert _lfp(vg=None) == INVALID
    assert _lfp(kg=ctypes.c_void_p(4100)) == INVALID     # misaligned
    assert _lfp(r=-1) == INVALID
    assert _lfp(D=96) == UNSUPPORTED


def test_cache_write_and_debug_validation():
    L = bd.lib()
    assert L.swa_cache_write(0, P, P, P, P, P, None, 1, 8, 1, 64, S0) == INVALID
    assert L.swa_cache_write(0, P, P, P, P, P, P, 1, 0, 1, 64, S0) == INVALID
    assert L.swa_cache_write(0, P, P, P, P, P, P, 1, 8, 1, 48, S0) == UNSUPPORTED
    assert L.swa_debug_index_mask(0, 16, 0, 1, None, 0, P, S0) == INVALID
    assert L.swa_debug_index_mask(5, 16, 2, 1, None, 0, P, S0) == INVALID
    assert L.swa_debug_index_mask(1, 16, 2, 0, None, 0, P, S0) == INVALID
    g = (ctypes.c_int32 * 1)(16)
    assert L.swa_debug_index_mask(1, 16, 2, 1, g, 1, P, S0) == INVALID


def _cached(**kw):
    a = dict(dt=0, q=P, kc=P, vc=P, sp=P, qp=P, o=P, lse=None, B=2, L=5, S=40, Hq=4, Hkv=2,
             D=128, W=16, ns=0, z=None, sc=0.1)
    a.update(kw)
    return bd.lib().swa_prefill_cached(a["dt"], a["q"], a["kc"], a["vc"], a["sp"], a["qp"],
                                       a["o"], a["lse"], a["B"], a["L"], a["S"], a["Hq"],
                                       a["Hkv"], a["D"], a["W"], a["ns"], a["z"], a["sc"], S0)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID), (dict(sp=None), INVALID), (dict(qp=None), INVALID),
    (dict(qp=ctypes.c_void_p(4098)), INVALID), (dict(kc=ctypes.c_void_p(4104)), INVALID),
    (dict(B=0), INVALID), (dict(L=0), INVALID), (dict(S=0), INVALID), (dict(W=0), INVALID),
    (dict(Hq=5), INVALID), (dict(sc=-1.0), INVALID), (dict(dt=3), INVALID),
    (dict(D=32), UNSUPPORTED), (dict(ns=-1), INVALID), (dict(z=ctypes.c_void_p(4098)), INVALID),
    (dict(dt=0, S=1 << 23, D=128), UNSUPPORTED),   # bf16 head slice of 2 GiB
])
def test_prefill_cached_validation(kw, code):
    assert _cached(**kw) == code


def test_cache_append_validation():
    L = bd.lib()
    ok = dict(dt=0, kn=P, vn=P, pos=P, kc=P, vc=P, sp=P, B=2, L=4, S=8, Hkv=2, D=64, ns=0)

    def call(**kw):
        a = dict(ok)
        a.update(kw)
        return L.swa_cache_append(a["dt"], a["kn"], a["vn"], a["pos"], a["kc"], a["vc"], a["sp"],
                                  a["B"], a["L"], a["S"], a["Hkv"], a["D"], a["ns"], S0)

    assert call(sp=None) == INVALID
    assert call(kn=ctypes.c_void_p(4100)) == INVALID
    assert call(L=0) == INVALID
    assert call(L=9) == INVALID          # more tokens than slots
    assert call(B=70000) == INVALID
    assert call(D=100) == UNSUPPORTED
    assert call(ns=-1) == INVALID
    assert call(ns=8) == INVALID         # no rolling slot left


def test_prefill_sinks_validation():
    L = bd.lib()

    def call(ns=4, z=None, D=128, W=8):
        return L.swa_prefill_sinks(0, P, P, P, P, None, 1, 16, 4, 2, D, W, ns, z, 0.1, S0)

    assert call(ns=-1) == INVALID
    assert call(ns=33) == INVALID        # sinks must fit the first key tile
    assert call(z=ctypes.c_void_p(4098)) == INVALID
    assert call(W=0) == INVALID
    assert call(D=96) == UNSUPPORTED


def test_tile_config():
    # 4 waves of 32 rows; 4 (2, 1) query heads share a K/V tile
    assert bd.tile_config("p", 32, 8, 128) == (32, 32)
    assert bd.tile_config("p", 32, 16, 128) == (64, 32)
    assert bd.tile_config("p", 12, 12, 64) == (128, 64)   # 64-key tiles at d_h = 64
    assert bd.tile_config("l", 12, 12, 64) == (128, 64)


# ------------------------------------------------------------ schedule vs brute force

def _bruteforce_triples(mode, T, w, BM, BN):
    got = oracle.band_tiles_bruteforce(mode, T, w, BM, BN)
    out = []
    for qi, (vis, edge) in enumerate(got):
        for kj in vis:
            out.append((qi, kj, 1 if kj in edge else 0))
    return out


@pytest.mark.parametrize("T", [1, 5, 16, 64, 100, 131])
@pytest.mark.parametrize("W", [1, 2, 15, 16, 17, 64, 200])
@pytest.mark.parametrize("BM,BN", [(16, 16), (32, 16), (8, 32), (32, 64)])
def test_causal_schedule_matches_bruteforce(T, W, BM, BN):
    assert bd.band_tiles(bd.SWA_MODE_CAUSAL, T, W, BM, BN) == _bruteforce_triples("causal", T, W, BM, BN)


@pytest.mark.parametrize("T", [1, 7, 16, 64, 100])
@pytest.mark.parametrize("r", [0, 1, 2, 15, 16, 40, 200])
@pytest.mark.parametrize("BM,BN", [(16, 16), (32, 16), (8, 32)])
def test_symmetric_schedule_matches_bruteforce(T, r, BM, BN):
    assert bd.band_tiles(bd.SWA_MODE_SYMMETRIC, T, r, BM, BN) == _bruteforce_triples("symmetric", T, r, BM, BN)


@pytest.mark.parametrize("T", [1, 7, 100])
def test_schedule_with_huge_window(T):
    # a window or radius past the sequence (up to INT_MAX, where r + i would
    # overflow 32-bit arithmetic) is full attention: same plan as W = T, r = T
    big = 2**31 - 1
    for BM, BN in ((16, 16), (32, 64)):
        assert bd.band_tiles(bd.SWA_MODE_CAUSAL, T, big, BM, BN) == _bruteforce_triples("causal", T, T, BM, BN)
        assert bd.band_tiles(bd.SWA_MODE_SYMMETRIC, T, big, BM, BN) == _bruteforce_triples("symmetric", T, T, BM, BN)


def test_schedule_at_kernel_tiling_small():
    # the kernels' real tile sizes on shapes small enough for brute force
    for (Hq, Hkv) in ((32, 8), (32, 16), (4, 4)):
        BM, BN = bd.tile_config("p", Hq, Hkv, 128)
        for T, W in ((300, 70), (257, 256), (200, 1000)):
            assert bd.band_tiles(0, T, W, BM, BN) == _bruteforce_triples("causal", T, W, BM, BN)
    BM, BN = bd.tile_config("l", 12, 12, 64)
    for T, r in ((300, 20), (257, 64), (130, 500)):
        assert bd.band_tiles(1, T, r, BM, BN) == _bruteforce_triples("symmetric", T, r, BM, BN)


def test_schedule_steady_state_counts_full_size():
    # full-size causal workload (T=16384, W=4096) at the kernel tiling (BM a
    # multiple of BN): every steady-state query tile visits (W + BM)/BN key
    # tiles, BM/BN partial ones at each edge of the band; ramp tiles have only
    # the BM/BN diagonal tiles partial.
    BM, BN = bd.tile_config("p", 32, 8, 128)
    assert BM % BN == 0
    nd = BM // BN
    T, W = 16384, 4096
    tr = np.array(bd.band_tiles(0, T, W, BM, BN))
    for qi in range(T // BM):
        rows = tr[tr[:, 0] == qi]
        m0 = qi * BM
        if m0 + BM <= W:
            assert rows[:, 2].sum() == nd and rows[-nd:, 2].all()
        elif m0 >= W:
            assert len(rows) == (W + BM) // BN and rows[:, 2].sum() == 2 * nd
            assert rows[:nd, 2].all() and rows[-nd:, 2].all()
        else:  # band reaches key 0 for some rows of the tile but not all
            assert rows[0, 1] == 0 and rows[-nd:, 2].all()
