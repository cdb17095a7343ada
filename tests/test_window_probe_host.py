"""CPU: the window probes of ``window_probe`` see a one-key window error.

The probes are run through the oracle at small sizes: with the correct window
an aimed key inside the window gives exactly its value row and one outside does
not; a window one key too wide or too narrow (a planted mistake: the oracle
called with W + 1 or W - 1, r + 1 or r - 1) moves some output by far more than
the 2e-2 gate.  This is what makes the full-size GPU probes a window-exactness
check.
"""

import numpy as np

import oracle
from sliding_window_attention_amd import inputs as inp
import window_probe as wp

GATE = 2e-2


def _causal_probe(T, W, Hq, Hkv, D, seed):
    NB = wp.nbits(T)
    k = np.broadcast_to(wp.code(np.arange(T), NB, D)[None, :, None, :], (1, T, Hkv, D)).copy()
    q = wp.causal_queries(1, T, Hq, D, W, NB)
    v = inp.widen(inp.as_io(inp.normal((1, T, Hkv, D), seed), "bf16"))
    return inp.widen(wp.bf16(q)), inp.widen(wp.bf16(k)), v


def test_causal_probe_inside_aims_return_the_aimed_value():
    T, W, Hq, Hkv, D = 200, 48, 8, 2, 128
    q, k, v = _causal_probe(T, W, Hq, Hkv, D, 3)
    o, _ = oracle.swa_prefill(q, k, v, W)
    names = [a[0] for a in wp.CAUSAL_AIMS]
    for h in range(Hq):
        name, aim = wp.CAUSAL_AIMS[h % len(wp.CAUSAL_AIMS)]
        for t in range(T):
            p = int(aim(np.int64(t), W))
            inside = max(0, t - W + 1) <= p <= t
            got = o[0, t, h]
            if inside:
                np.testing.assert_allclose(got, v[0, p, h // (Hq // Hkv)], atol=1e-6)
            elif 0 <= p < T:
                assert np.max(np.abs(got - v[0, p, h // (Hq // Hkv)])) > 0.1, (name, t)
    assert names == ["t-W", "t-W+1", "t", "t+1", "t-W+2", "t-1", "t-W-1", "0"]


def test_causal_probe_sees_a_one_key_window_error():
    T, W, Hq, Hkv, D = 200, 48, 8, 2, 128
    q, k, v = _causal_probe(T, W, Hq, Hkv, D, 4)
    o, _ = oracle.swa_prefill(q, k, v, W)
    for wrong in (W - 1, W + 1):
        ow, _ = oracle.swa_prefill(q, k, v, wrong)
        # every steady-state row shows the error on some head
        err = np.abs(ow - o).max(axis=(2, 3))[0]
        assert np.all(err[W + 1:] > GATE), wrong
    # a window shifted by one (same size, t-W <= s < t) is seen on every row too
    shifted = np.zeros_like(o)
    for t in range(1, T):
        S = np.arange(max(0, t - W), t)
        for h in range(Hq):
            shifted[0, t, h], _ = oracle.attend(q[0, t, h], k[0, S, h // 4], v[0, S, h // 4],
                                                1 / np.sqrt(D))
    assert np.all(np.abs(shifted - o).max(axis=(2, 3))[0, 1:] > GATE)


def test_longformer_probe_sees_a_one_step_radius_error():
    T, H, D, r = 160, 4, 64, 12
    dil = np.array([1, 2, 1, 2], dtype=np.int32)
    g = np.array([[0, 8]], dtype=np.int32)
    NB = wp.nbits(T)
    i = np.arange(T)
    k = np.broadcast_to(wp.code(i, NB, D)[None, :, None, :], (1, T, H, D)).copy()
    aims = [lambda i, d: i + r * d, lambda i, d: i + (r + 1) * d, lambda i, d: i - r * d,
            lambda i, d: i - (r + 1) * d]
    q = np.zeros((1, T, H, D), dtype=np.float32)
    for h in range(H):
        q[:, :, h] = wp.A * wp.code(aims[h](i, int(dil[h])), NB, D)[None]
    v = inp.widen(inp.as_io(inp.normal((1, T, H, D), 5), "bf16"))
    q, k = inp.widen(wp.bf16(q)), inp.widen(wp.bf16(k))
    o, _ = oracle.swa_longformer(q, k, v, r, dil, g)
    for wrong in (r - 1, r + 1):
        ow, _ = oracle.swa_longformer(q, k, v, wrong, dil, g)
        err = np.abs(ow - o).max(axis=3)[0]          # [T, H]
        # rows whose aimed key moves across the boundary, away from the ends
        mid = slice(3 * r, T - 3 * r)
        assert np.all(err[mid].max(axis=1) > GATE), wrong


def test_codes_are_exact_in_bf16():
    NB = 16
    c = wp.code(np.arange(1 << NB), NB, 128)
    assert set(np.unique(c[:, :NB])) == {-1.0, 1.0} and not c[:, NB:].any()
    wp.bf16(wp.A * c[:1000])
