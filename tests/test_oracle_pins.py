"""Pins for the CPU oracle: printed tables, closed forms, textbook special cases
and brute force.  None of these recomputes the oracle's own formula; each pits
the oracle against something fixed independently of it.  CPU only.
"""

import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

import oracle
from oracle import index_sets as ix
from sliding_window_attention_amd import inputs as inp

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows, total = {}, None
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, vals = line.split(":")
            if key == "total":
                total = int(vals)
            else:
                rows[int(key)] = [int(x) for x in vals.split()]
    return rows, total


# ---------------------------------------------------------------- printed tables

def test_symmetric_table_n16_r2():
    rows, total = _read_table("pp_symmetric_n16_r2.txt")
    for i, keys in rows.items():
        assert oracle.symmetric_index_set(i, 16, 2).tolist() == keys
    sizes = [len(oracle.symmetric_index_set(i, 16, 2)) for i in range(16)]
    assert sizes == [3, 4] + [5] * 12 + [4, 3]
    assert sum(sizes) == total == 74


def test_dilated_table_n16_r2_d2():
    rows, total = _read_table("pp_dilated_n16_r2_d2.txt")
    assert len(rows) == 16
    for i, keys in rows.items():
        assert oracle.longformer_index_set(i, 16, 2, 2).tolist() == keys
    assert sum(len(oracle.longformer_index_set(i, 16, 2, 2)) for i in range(16)) == total == 68


def test_global_table_n16_r2():
    rows, total = _read_table("pp_global_n16_r2_G0_8.txt")
    assert len(rows) == 16
    for i, keys in rows.items():
        assert oracle.longformer_index_set(i, 16, 2, 1, (0, 8)).tolist() == keys
    assert sum(len(oracle.longformer_index_set(i, 16, 2, 1, (0, 8))) for i in range(16)) == total == 120
    # the page's upper bound g*n + (n-g)(2r+1+g) holds
    assert total <= 2 * 16 + 14 * (5 + 2)


def test_counts_n16():
    with open(os.path.join(GOLDEN, "pp_counts_n16.txt")) as f:
        want = dict(l.split() for l in f if l.strip() and not l.startswith("#"))
    full = sum(len(oracle.symmetric_index_set(i, 16, 15)) for i in range(16))
    causal = sum(len(oracle.causal_index_set(t, 16)) for t in range(16))
    window = sum(len(oracle.symmetric_index_set(i, 16, 2)) for i in range(16))
    assert full == int(want["full_bidirectional"])
    assert causal == int(want["full_causal"])
    assert window == int(want["sliding_window_r2"])


def test_causal_examples():
    with open(os.path.join(GOLDEN, "causal_examples.txt")) as f:
        cases = [tuple(map(int, l.split())) for l in f if l.strip() and not l.startswith("#")]
    assert len(cases) == 3
    for t, W, first, last in cases:
        S = oracle.causal_index_set(t, W)
        assert S[0] == first and S[-1] == last and len(S) == last - first + 1


# ---------------------------------------------------------------- closed forms (brute force)

@pytest.mark.parametrize("T", [1, 2, 7, 16, 33])
@pytest.mark.parametrize("W", [1, 2, 3, 8, 16, 40])
def test_causal_count_closed_form(T, W):
    got = sum(len(oracle.causal_index_set(t, W)) for t in range(T))
    w = min(W, T)
    assert got == T * w - w * (w - 1) // 2


@pytest.mark.parametrize("n", [8, 16, 31])
@pytest.mark.parametrize("r", [0, 1, 2, 3])
@pytest.mark.parametrize("d", [1, 2, 3])
def test_dilated_count_closed_form(n, r, d):
    if r * d > n:
        pytest.skip("closed form assumes r*d <= n")
    got = sum(len(oracle.symmetric_index_set(i, n, r, d)) for i in range(n))
    assert got == (2 * r + 1) * n - d * r * (r + 1)


def test_dilated_is_residue_class_problem():
    # A dilated window on x equals d independent undilated windows on x[rho::d].
    n, r, d = 23, 3, 3
    for i in range(n):
        rho, ii = i % d, i // d
        m = len(range(rho, n, d))
        want = [rho + d * j for j in oracle.symmetric_index_set(ii, m, r, 1)]
        assert oracle.symmetric_index_set(i, n, r, d).tolist() == want


def test_masks_match_index_sets():
    T, W = 37, 9
    m = oracle.causal_mask(T, W)
    for t in range(T):
        assert np.nonzero(m[t])[0].tolist() == oracle.causal_index_set(t, W).tolist()
    lm = oracle.longformer_mask(20, 3, 2, (1, 12))
    for i in range(20):
        assert np.nonzero(lm[i])[0].tolist() == oracle.longformer_index_set(i, 20, 3, 2, (1, 12)).tolist()


# ---------------------------------------------------------------- values: textbook special cases

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v, causal, scale=None, mask=None):
    # q [B,T,H,D] -> torch [B,H,T,D], float64 on CPU; GQA via enable_gqa.
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x.transpose(0, 2, 1, 3))) for x in (q, k, v))
    gqa = tq.shape[1] != tk.shape[1]
    out = F.scaled_dot_product_attention(tq, tk, tv, attn_mask=mask, is_causal=causal,
                                         scale=scale, enable_gqa=gqa)
    return out.numpy().transpose(0, 2, 1, 3)


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (4, 1), (6, 3)])
def test_window_covering_sequence_is_dense_causal(Hq, Hkv):
    B, T, D = 2, 19, 8
    q, k, v = _rand((B, T, Hq, D), 1), _rand((B, T, Hkv, D), 2), _rand((B, T, Hkv, D), 3)
    want = _sdpa(q, k, v, causal=True)
    for W in (T, T + 5, 4 * T):
        o, _ = oracle.swa_prefill(q, k, v, W)
        np.testing.assert_allclose(o, want, rtol=0, atol=1e-12)


def test_explicit_scale_matches_library():
    B, T, H, D = 1, 11, 2, 16
    q, k, v = _rand((B, T, H, D), 4), _rand((B, T, H, D), 5), _rand((B, T, H, D), 6)
    o, _ = oracle.swa_prefill(q, k, v, T, scale=0.37)
    np.testing.assert_allclose(o, _sdpa(q, k, v, True, scale=0.37), rtol=0, atol=1e-12)


def test_symmetric_full_radius_is_dense_bidirectional():
    B, T, H, D = 2, 13, 3, 8
    q, k, v = _rand((B, T, H, D), 7), _rand((B, T, H, D), 8), _rand((B, T, H, D), 9)
    o, _ = oracle.swa_longformer(q, k, v, r=T - 1)
    np.testing.assert_allclose(o, _sdpa(q, k, v, causal=False), rtol=0, atol=1e-12)


def test_banded_values_match_library_with_boolean_mask():
    # The library applies a boolean mask built from the pages' printed tables
    # (global + window, n=16): values of the oracle must agree.
    rows, _ = _read_table("pp_global_n16_r2_G0_8.txt")
    mask = torch.zeros(16, 16, dtype=torch.bool)
    for i, keys in rows.items():
        mask[i, keys] = True
    B, T, H, D = 1, 16, 2, 64
    q, k, v = _rand((B, T, H, D), 10), _rand((B, T, H, D), 11), _rand((B, T, H, D), 12)
    o, _ = oracle.swa_longformer(q, k, v, r=2, global_idx=[[0, 8]])
    np.testing.assert_allclose(o, _sdpa(q, k, v, False, mask=mask), rtol=0, atol=1e-12)


def test_window_one_returns_own_value():
    B, T, H, D = 1, 10, 2, 4
    q, k, v = _rand((B, T, H, D), 13), _rand((B, T, H, D), 14), _rand((B, T, H, D), 15)
    o, lse = oracle.swa_prefill(q, k, v, 1)
    np.testing.assert_array_equal(o, v)
    want_lse = np.einsum("bthd,bthd->bht", q, k) / math.sqrt(D)
    np.testing.assert_allclose(lse, want_lse, rtol=0, atol=1e-12)


def test_zero_query_gives_window_mean():
    B, T, H, D, W = 1, 25, 1, 3, 6
    q = np.zeros((B, T, H, D))
    k, v = _rand((B, T, H, D), 16), _rand((B, T, H, D), 17)
    o, lse = oracle.swa_prefill(q, k, v, W)
    csum = np.concatenate([np.zeros((1, D)), np.cumsum(v[0, :, 0], axis=0)])
    for t in range(T):
        lo = max(0, t - W + 1)
        np.testing.assert_allclose(o[0, t, 0], (csum[t + 1] - csum[lo]) / (t + 1 - lo), atol=1e-12)
        assert abs(lse[0, 0, t] - math.log(t + 1 - lo)) < 1e-12


def test_constant_values_pass_through():
    B, T, H, D = 1, 17, 2, 5
    q, k = _rand((B, T, H, D), 18), _rand((B, T, H, D), 19)
    v = np.full((B, T, H, D), 2.5)
    o, _ = oracle.swa_prefill(q, k, v, 4)
    np.testing.assert_allclose(o, v, atol=1e-13)
    o, _ = oracle.swa_longformer(q, k, v, 2, [3, 2], [[0, 9]])
    np.testing.assert_allclose(o, v, atol=1e-13)


def test_dense_form_equals_index_set_form():
    T, D, W = 31, 6, 7
    q, k, v = _rand((T, D), 20), _rand((T, D), 21), _rand((T, D), 22)
    sc = 0.3
    dense = oracle.dense_masked_attention(q, k, v, oracle.causal_mask(T, W), sc)
    o, _ = oracle.swa_prefill(q[None, :, None], k[None, :, None], v[None, :, None], W, sc)
    np.testing.assert_allclose(o[0, :, 0], dense, atol=1e-13)
    mask = oracle.longformer_mask(T, 3, 2, (5, 20))
    dense = oracle.dense_masked_attention(q, k, v, mask, sc)
    o, _ = oracle.swa_longformer(q[None, :, None], k[None, :, None], v[None, :, None], 3, [2], [[5, 20]], sc)
    np.testing.assert_allclose(o[0, :, 0], dense, atol=1e-13)


def test_lse_is_logsumexp_and_merges():
    rng = np.random.default_rng(23)
    D, n = 8, 50
    q, K, V = rng.standard_normal(D), rng.standard_normal((n, D)), rng.standard_normal((n, D))
    sc = 0.5
    o, lse = oracle.attend(q, K, V, sc)
    assert abs(lse - logsumexp(K @ q * sc)) < 1e-12
    # splitting the key set and merging the two partial results by their lse
    # reproduces the whole (softmax associativity, used by split-KV kernels)
    cut = 17
    o1, l1 = oracle.attend(q, K[:cut], V[:cut], sc)
    o2, l2 = oracle.attend(q, K[cut:], V[cut:], sc)
    L = np.logaddexp(l1, l2)
    np.testing.assert_allclose(np.exp(l1 - L) * o1 + np.exp(l2 - L) * o2, o, atol=1e-13)
    assert abs(L - lse) < 1e-12


def test_empty_set():
    o, lse = oracle.attend(np.ones(4), np.zeros((0, 4)), np.zeros((0, 4)), 1.0)
    assert np.all(o == 0) and lse == -math.inf


# ---------------------------------------------------------------- ring cache / decode

def test_ring_slot_rule_and_generator_state():
    B, T, H, D, W = 3, 40, 2, 4, 8
    k, v = _rand((B, T, H, D), 24), _rand((B, T, H, D), 25)
    upto = np.array([3, 17, 39])
    kc, vc, sp = oracle.ring_from_sequence(k, v, upto, W)
    for b in range(B):
        for j in range(W):
            p = sp[b, j]
            if p >= 0:
                assert p % W == j and p <= upto[b] and p > upto[b] - W
                np.testing.assert_array_equal(kc[b, :, j], k[b, p])
    # the input generator's closed-form ring state is the replayed state
    np.testing.assert_array_equal(inp.full_ring_positions(upto, W), sp)


def test_ring_write_overwrites_position_minus_W():
    W = 4
    kc = np.zeros((1, 1, W, 2)); vc = np.zeros((1, 1, W, 2)); sp = np.full((1, W), -1)
    for p in range(9):
        oracle.ring_write(kc, vc, sp, np.full((1, 1, 2), p), np.full((1, 1, 2), -p), [p])
    assert sorted(sp[0].tolist()) == [5, 6, 7, 8]
    assert kc[0, 0, 8 % W, 0] == 8


@pytest.mark.parametrize("W", [1, 3, 8])
def test_decode_equals_prefill_row(W):
    B, T, Hq, Hkv, D = 3, 30, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 26), _rand((B, T, Hkv, D), 27), _rand((B, T, Hkv, D), 28)
    cur = np.array([0, 5, 29])
    kc, vc, sp = oracle.ring_from_sequence(k, v, cur, W)
    qd = np.stack([q[b, cur[b]] for b in range(B)])
    o, lse = oracle.swa_decode(qd, kc, vc, sp, cur, W)
    for b in range(B):
        op, lp = oracle.swa_prefill(q[b:b + 1], k[b:b + 1], v[b:b + 1], W, rows=[cur[b]])
        np.testing.assert_allclose(o[b], op[0, 0], atol=1e-13)
        np.testing.assert_allclose(lse[b], lp[0, :, 0], atol=1e-12)


def test_decode_ignores_slot_order_and_masks_stale_future_empty():
    rng = np.random.default_rng(29)
    B, Hq, Hkv, D, W = 1, 2, 1, 4, 6
    q = rng.standard_normal((B, Hq, D))
    kc, vc = rng.standard_normal((B, Hkv, W, D)), rng.standard_normal((B, Hkv, W, D))
    sp = np.array([[10, 11, 12, 4, 20, -1]])      # 4 stale, 20 future, -1 empty
    cur = np.array([12])
    o, _ = oracle.swa_decode(q, kc, vc, sp, cur, W)
    assert oracle.decode_index_set(sp[0], 12, W).tolist() == [0, 1, 2]
    perm = rng.permutation(W)
    o2, _ = oracle.swa_decode(q, kc[:, :, perm], vc[:, :, perm], sp[:, perm], cur, W)
    np.testing.assert_allclose(o, o2, atol=1e-14)
    # all slots invalid -> zero output
    o3, l3 = oracle.swa_decode(q, kc, vc, np.full((1, W), -1), cur, W)
    assert np.all(o3 == 0) and np.all(np.isneginf(l3))


# ---------------------------------------------------------------- chunked prefill over a ring

def test_ring_append_is_ordered_token_writes_and_keeps_latest():
    B, Hkv, D, S = 2, 2, 3, 7
    rng = np.random.default_rng(40)
    kc = np.zeros((B, Hkv, S, D)); vc = np.zeros_like(kc); sp = np.full((B, S), -1)
    kc2, vc2, sp2 = kc.copy(), vc.copy(), sp.copy()
    P = 0
    for L in (3, 5, 1, 7, 4):                      # chunks of consecutive positions
        pos = np.tile(np.arange(P, P + L), (B, 1))
        kn, vn = rng.standard_normal((B, L, Hkv, D)), rng.standard_normal((B, L, Hkv, D))
        oracle.ring_append(kc, vc, sp, kn, vn, pos)
        for t in range(L):
            oracle.ring_write(kc2, vc2, sp2, kn[:, t], vn[:, t], pos[:, t])
        P += L
    np.testing.assert_array_equal(kc, kc2)
    np.testing.assert_array_equal(sp, sp2)
    # slot j holds the latest position congruent to j (mod S)
    for j in range(S):
        assert sp[0, j] == max(p for p in range(P) if p % S == j)


@pytest.mark.parametrize("W,L,p0", [(8, 5, 20), (16, 16, 40), (5, 12, 3), (30, 1, 25)])
def test_prefill_cached_equals_prefill_rows(W, L, p0):
    # a ring of S = W + L - 1 slots holding tokens 0 .. p0+L-1 (appended chunk by
    # chunk, the last chunk being the queries' own tokens) gives prefill rows
    # p0 .. p0+L-1
    B, T, Hq, Hkv, D = 2, p0 + L, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 41), _rand((B, T, Hkv, D), 42), _rand((B, T, Hkv, D), 43)
    S = W + L - 1
    kc = np.zeros((B, Hkv, S, D)); vc = np.zeros_like(kc); sp = np.full((B, S), -1)
    cuts = list(range(0, p0, 7)) + [p0, T]
    for a, b_ in zip(cuts[:-1], cuts[1:]):
        pos = np.tile(np.arange(a, b_), (B, 1))
        oracle.ring_append(kc, vc, sp, k[:, a:b_], v[:, a:b_], pos)
    qpos = np.tile(np.arange(p0, T), (B, 1))
    o, lse = oracle.swa_prefill_cached(q[:, p0:T], kc, vc, sp, qpos, W)
    op, lp = oracle.swa_prefill(q, k, v, W, rows=list(range(p0, T)))
    np.testing.assert_allclose(o, op, atol=1e-12)
    np.testing.assert_allclose(lse, lp, atol=1e-12)


def test_prefill_cached_single_token_is_decode():
    B, Hq, Hkv, D, S, W = 3, 4, 2, 8, 12, 9
    rng = np.random.default_rng(44)
    q = rng.standard_normal((B, 1, Hq, D))
    kc, vc = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    sp = rng.integers(-3, 30, size=(B, S))
    cur = np.array([10, 25, 2])
    o, lse = oracle.swa_prefill_cached(q, kc, vc, sp, cur[:, None], W)
    od, ld = oracle.swa_decode(q[:, 0], kc, vc, sp, cur, W)
    np.testing.assert_allclose(o[:, 0], od, atol=1e-14)
    np.testing.assert_allclose(lse[:, :, 0], ld, atol=1e-14)


def test_prefill_cached_matches_position_mask_formula():
    # [G3] "How it works": mask from absolute positions, 1[s > t-W] 1[s < t+W]
    # times the causal factor 1[s <= t]; empty slots masked.  Checked against
    # torch SDPA in float64 with that boolean mask, on a ring too small for the
    # chunk (early queries have lost keys) and with stale / future / empty slots.
    B, L, Hq, Hkv, D, S, W = 2, 6, 2, 1, 8, 9, 7
    rng = np.random.default_rng(45)
    q = rng.standard_normal((B, L, Hq, D))
    kc, vc = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    sp = np.array([[13, 14, 15, 16, 17, 9, 10, 11, -1], [3, 30, 5, 6, -1, 8, 9, 1, 2]])
    qpos = np.array([[12, 13, 14, 15, 16, 17], [4, 5, 6, 7, 8, 9]])
    o, _ = oracle.swa_prefill_cached(q, kc, vc, sp, qpos, W)
    for b in range(B):
        t = qpos[b][:, None]
        s_ = sp[b][None, :]
        mask = (s_ > t - W) & (s_ < t + W) & (s_ <= t) & (s_ >= 0)
        for h in range(Hq):
            ref = _sdpa(q[b:b + 1, :, h:h + 1], kc[b, 0][None, :, None], vc[b, 0][None, :, None],
                        False, mask=torch.from_numpy(mask))
            np.testing.assert_allclose(o[b, :, h], ref[0, :, 0], atol=1e-12)


def test_prefill_cached_ignores_slot_order():
    B, L, Hq, Hkv, D, S, W = 1, 4, 2, 1, 4, 10, 6
    rng = np.random.default_rng(46)
    q = rng.standard_normal((B, L, Hq, D))
    kc, vc = rng.standard_normal((B, Hkv, S, D)), rng.standard_normal((B, Hkv, S, D))
    sp = rng.permutation(np.arange(S))[None] + 3
    qpos = np.array([[7, 8, 9, 12]])
    o, _ = oracle.swa_prefill_cached(q, kc, vc, sp, qpos, W)
    perm = rng.permutation(S)
    o2, _ = oracle.swa_prefill_cached(q, kc[:, :, perm], vc[:, :, perm], sp[:, perm], qpos, W)
    np.testing.assert_allclose(o, o2, atol=1e-14)


# ---------------------------------------------------------------- attention sinks

@pytest.mark.parametrize("T,W,n_sink", [(40, 6, 4), (40, 1, 3), (33, 10, 1), (20, 30, 4)])
def test_sink_window_against_sdpa_mask(T, W, n_sink):
    # union of the causal window and the first n_sink tokens, through torch SDPA
    # with the boolean mask written from the two definitions
    B, Hq, Hkv, D = 2, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 80), _rand((B, T, Hkv, D), 81), _rand((B, T, Hkv, D), 82)
    t = np.arange(T)[:, None]
    s_ = np.arange(T)[None, :]
    mask = ((s_ <= t) & (s_ > t - W)) | ((s_ < n_sink) & (s_ <= t))
    o, _ = oracle.swa_prefill(q, k, v, W, n_sink=n_sink)
    ref = _sdpa(q, k, v, False, mask=torch.from_numpy(mask))
    np.testing.assert_allclose(o, ref, atol=1e-12)
    # each key once: the set sizes
    for tt in range(T):
        n = len(oracle.causal_sink_index_set(tt, W, n_sink))
        assert n == min(tt + 1, W) + max(0, min(n_sink, tt + 1 - W))


def test_sink_logit_closed_forms():
    B, T, Hq, Hkv, D, W = 1, 12, 3, 1, 4, 5
    rng = np.random.default_rng(83)
    z = np.array([0.7, -2.0, 3.5])
    v = np.full((B, T, Hkv, D), 1.5)
    q = np.zeros((B, T, Hq, D))
    k = rng.standard_normal((B, T, Hkv, D))
    o, lse = oracle.swa_prefill(q, k, v, W, sink_logit=z)
    for t in range(T):
        n = min(t + 1, W)                       # q = 0: every score is 0
        for h in range(Hq):
            np.testing.assert_allclose(o[0, t, h], 1.5 * n / (n + math.exp(z[h])), rtol=1e-13)
            np.testing.assert_allclose(lse[0, h, t], math.log(n + math.exp(z[h])), rtol=1e-13)
    # lse with a sink = logaddexp(lse without, z); a very negative sink is no sink
    q = rng.standard_normal((B, T, Hq, D))
    o0, l0 = oracle.swa_prefill(q, k, v, W)
    o1, l1 = oracle.swa_prefill(q, k, v, W, sink_logit=z)
    np.testing.assert_allclose(l1, np.logaddexp(l0, z[None, :, None]), atol=1e-12)
    np.testing.assert_allclose(o1, o0 * np.exp(l0 - l1).transpose(0, 2, 1)[..., None], atol=1e-12)
    o2, _ = oracle.swa_prefill(q, k, v, W, sink_logit=np.full(Hq, -800.0))
    np.testing.assert_allclose(o2, o0, atol=1e-15)


def test_ring_slot_rule_with_sinks():
    S, n_sink = 9, 3
    kc = np.zeros((1, 1, S, 1)); vc = np.zeros_like(kc); sp = np.full((1, S), -1)
    P = 40
    pos = np.arange(P)[None]
    oracle.ring_append(kc, vc, sp, pos[:, :, None, None].astype(float),
                       -pos[:, :, None, None].astype(float), pos, n_sink=n_sink)
    assert sp[0, :n_sink].tolist() == [0, 1, 2]                  # pinned
    assert sorted(sp[0, n_sink:].tolist()) == list(range(P - (S - n_sink), P))  # rolling
    assert [oracle.ring_slot(p, S, 0) for p in (0, 8, 9, 20)] == [0, 8, 0, 2]


@pytest.mark.parametrize("W,L,p0,n_sink", [(8, 5, 30, 4), (16, 8, 40, 1), (6, 12, 9, 4)])
def test_sink_ring_chunks_equal_prefill_rows(W, L, p0, n_sink):
    # pinned sink slots + a rolling region of W + L - 1 slots, filled chunk by
    # chunk, give the prefill rows with the same sinks and sink logits
    B, T, Hq, Hkv, D = 2, p0 + L, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 84), _rand((B, T, Hkv, D), 85), _rand((B, T, Hkv, D), 86)
    z = np.array([0.3, -1.0, 2.0, 0.0])
    S = n_sink + W + L - 1
    kc = np.zeros((B, Hkv, S, D)); vc = np.zeros_like(kc); sp = np.full((B, S), -1)
    cuts = list(range(0, p0, 5)) + [p0, T]
    for a, b_ in zip(cuts[:-1], cuts[1:]):
        pos = np.tile(np.arange(a, b_), (B, 1))
        oracle.ring_append(kc, vc, sp, k[:, a:b_], v[:, a:b_], pos, n_sink=n_sink)
    qpos = np.tile(np.arange(p0, T), (B, 1))
    o, lse = oracle.swa_prefill_cached(q[:, p0:T], kc, vc, sp, qpos, W, n_sink=n_sink,
                                       sink_logit=z)
    op, lp = oracle.swa_prefill(q, k, v, W, rows=list(range(p0, T)), n_sink=n_sink, sink_logit=z)
    np.testing.assert_allclose(o, op, atol=1e-12)
    np.testing.assert_allclose(lse, lp, atol=1e-12)


# ---------------------------------------------------------------- Longformer global projections

def test_global_projections_equal_to_sliding_is_shared_form():
    # [PP] §5.3: global projections initialised from the sliding ones behave
    # exactly like the shared form
    B, T, H, D, r = 2, 24, 3, 8, 2
    q, k, v = _rand((B, T, H, D), 100), _rand((B, T, H, D), 101), _rand((B, T, H, D), 102)
    g = np.array([[0, 8, 13], [5, 6, 20]])
    dil = [1, 2, 3]
    o1, l1 = oracle.swa_longformer(q, k, v, r, dil, g)
    o2, l2 = oracle.swa_longformer(q, k, v, r, dil, g, qg=q.copy(), kg=k.copy(), vg=v.copy())
    np.testing.assert_allclose(o2, o1, atol=1e-13)
    np.testing.assert_allclose(l2, l1, atol=1e-13)


def test_global_projections_against_sdpa_on_stacked_keys():
    # Independent route: stack the two projections into 2T key/value rows
    # ([k; kg], [v; vg]) and give torch SDPA one boolean mask per row: a local
    # row sees its window positions that are not global in the first half and
    # every global position in the second half; a global row sees the whole
    # second half with its qg query.
    B, T, H, D, r = 1, 20, 2, 8, 2
    q, k, v = _rand((B, T, H, D), 103), _rand((B, T, H, D), 104), _rand((B, T, H, D), 105)
    qg, kg, vg = _rand((B, T, H, D), 106), _rand((B, T, H, D), 107), _rand((B, T, H, D), 108)
    G = [0, 9]
    dil = [1, 2]
    o, _ = oracle.swa_longformer(q, k, v, r, dil, np.array([G]), qg=qg, kg=kg, vg=vg)
    for h in range(H):
        d = dil[h]
        mask = np.zeros((T, 2 * T), dtype=bool)
        qrows = np.zeros((T, D))
        for i in range(T):
            if i in G:
                mask[i, T:] = True
                qrows[i] = qg[0, i, h]
            else:
                for j in range(T):
                    if (i - j) % d == 0 and abs(i - j) <= r * d and j not in G:
                        mask[i, j] = True
                for gpos in G:
                    mask[i, T + gpos] = True
                qrows[i] = q[0, i, h]
        K2 = np.concatenate([k[0, :, h], kg[0, :, h]])[None, :, None]
        V2 = np.concatenate([v[0, :, h], vg[0, :, h]])[None, :, None]
        ref = _sdpa(qrows[None, :, None], K2, V2, False, mask=torch.from_numpy(mask))
        np.testing.assert_allclose(o[0, :, h], ref[0, :, 0], atol=1e-12)


# ---------------------------------------------------------------- tiles

# ---------------------------------------------------------------- causal dilation ([KB] §2 "Dilation")

def test_causal_dilated_set_by_definition_and_count():
    # {t - i*d : 0 <= i < W} cut at 0: brute force over a grid of positions
    for d in (1, 2, 3, 7):
        for W in (1, 2, 5, 40):
            for t in range(0, 60):
                want = sorted(x for x in range(0, t + 1) if (t - x) % d == 0 and (t - x) // d < W)
                got = oracle.causal_dilated_index_set(t, W, d).tolist()
                assert got == want
                assert len(got) == min(W, t // d + 1)
    # d = 1 is the plain causal window
    for t in range(30):
        assert oracle.causal_dilated_index_set(t, 7, 1).tolist() == oracle.causal_index_set(t, 7).tolist()


def test_causal_dilated_is_residue_class_problem():
    # a dilated head is d independent causal problems on the subsequences
    # x[rho::d]: the window of t is rho + d * (causal window of t // d)
    for d in (2, 3, 5):
        for W in (1, 4, 9):
            for t in range(50):
                rho, i = t % d, t // d
                cls = rho + d * oracle.causal_index_set(i, W)
                assert oracle.causal_dilated_index_set(t, W, d).tolist() == cls.tolist()


def test_causal_dilated_attention_against_sdpa_per_class():
    # per residue class with a window covering the class, dilated SWA is dense
    # causal attention on that class subsequence (torch SDPA, float64)
    B, T, Hq, Hkv, D = 2, 23, 4, 2, 8
    q, k, v = _rand((B, T, Hq, D), 61), _rand((B, T, Hkv, D), 62), _rand((B, T, Hkv, D), 63)
    dil = [1, 3, 2, 3]
    o, _ = oracle.swa_prefill(q, k, v, T, dilation=dil)
    for h, d in enumerate(dil):
        kvh = h // (Hq // Hkv)
        for rho in range(d):
            sl = slice(rho, None, d)
            want = _sdpa(q[:, sl, h:h + 1], k[:, sl, kvh:kvh + 1], v[:, sl, kvh:kvh + 1], True,
                         scale=1 / math.sqrt(D))
            np.testing.assert_allclose(o[:, sl, h:h + 1], want, rtol=0, atol=1e-12)


def test_causal_dilated_zero_query_is_mean_over_dilated_window():
    B, T, H, D, W = 1, 40, 2, 4, 5
    q = np.zeros((B, T, H, D))
    k, v = _rand((B, T, H, D), 64), _rand((B, T, H, D), 65)
    o, _ = oracle.swa_prefill(q, k, v, W, dilation=[2, 4])
    for h, d in enumerate((2, 4)):
        for t in range(T):
            keys = [t - i * d for i in range(W) if t - i * d >= 0]
            np.testing.assert_allclose(o[0, t, h], v[0, keys, h].mean(axis=0), rtol=0, atol=1e-13)


# ---------------------------------------------------------------- rotary positions ([G3], [KB] §2)

def test_rope_is_complex_rotation():
    # the rotate-half pair (x_i, x_{i+d/2}) as the complex number x_i + j x_{i+d/2},
    # multiplied by exp(j p theta_i), theta_i = base^(-2i/d)
    T, H, D, base = 9, 3, 16, 1.0e4
    x = _rand((T, H, D), 66)
    pos = np.array([0, 1, 2, 5, 100, 4095, 16383, 32767, 70000])
    r = oracle.rope_rotate_half(x, pos, base)
    z = x[..., :D // 2] + 1j * x[..., D // 2:]
    th = base ** (-np.arange(D // 2) * 2.0 / D)
    zr = z * np.exp(1j * pos[:, None, None] * th[None, None, :])
    np.testing.assert_allclose(r[..., :D // 2], zr.real, rtol=0, atol=1e-9)
    np.testing.assert_allclose(r[..., D // 2:], zr.imag, rtol=0, atol=1e-9)


def test_rope_position_zero_identity_norms_and_relative_phase():
    T, H, D = 12, 2, 8
    x = _rand((1, T, H, D), 67)
    y = _rand((1, T, H, D), 68)
    pos = np.arange(T)
    rx = oracle.rope_rotate_half(x, pos, 1.0e6)
    ry = oracle.rope_rotate_half(y, pos, 1.0e6)
    np.testing.assert_array_equal(rx[:, 0], x[:, 0])                        # p = 0: no rotation
    np.testing.assert_allclose(np.linalg.norm(rx, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)
    # q_m . k_n depends on m - n only: shift both positions by 37
    sx = oracle.rope_rotate_half(x, pos + 37, 1.0e6)
    sy = oracle.rope_rotate_half(y, pos + 37, 1.0e6)
    for m in range(T):
        for n in range(T):
            a = rx[0, m, 0] @ ry[0, n, 0]
            b = sx[0, m, 0] @ sy[0, n, 0]
            assert abs(a - b) < 1e-11


def test_prefill_with_rope_equals_prefill_of_rotated_inputs():
    # the rope_base option is exactly "rotate q and k at their positions, then attend"
    B, T, Hq, Hkv, D, W = 1, 17, 2, 1, 8, 6
    q, k, v = _rand((B, T, Hq, D), 69), _rand((B, T, Hkv, D), 70), _rand((B, T, Hkv, D), 71)
    z = q[..., :D // 2] + 1j * q[..., D // 2:]
    th = 1.0e4 ** (-np.arange(D // 2) * 2.0 / D)
    ph = np.exp(1j * np.arange(T)[None, :, None, None] * th)
    qr = np.concatenate([(z * ph).real, (z * ph).imag], axis=-1)
    zk = k[..., :D // 2] + 1j * k[..., D // 2:]
    kr = np.concatenate([(zk * ph).real, (zk * ph).imag], axis=-1)
    o1, l1 = oracle.swa_prefill(q, k, v, W, rope_base=1.0e4)
    o2, l2 = oracle.swa_prefill(qr, kr, v, W)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-12)


def test_tiles_hand_example():
    # T=16, W=4, BM=BN=4 (causal): block 0 sees only the diagonal block; later
    # blocks see their diagonal block and the one before, both partly masked.
    got = oracle.band_tiles_bruteforce("causal", 16, 4, 4, 4)
    assert got[0] == ([0], [0])
    for qi in range(1, 4):
        assert got[qi] == ([qi - 1, qi], [qi - 1, qi])


@pytest.mark.parametrize("W,B_", [(8, 4), (12, 4), (16, 8)])
def test_tiles_causal_steady_state(W, B_):
    T = 64
    got = oracle.band_tiles_bruteforce("causal", T, W, B_, B_)
    for qi, (vis, edge) in enumerate(got):
        m0 = qi * B_
        if m0 + B_ <= W:               # ramp: only the diagonal block is partial
            assert vis == list(range(0, qi + 1)) and edge == [qi]
        else:                          # steady state: W/BN + 1 blocks, two partial
            assert len(vis) == W // B_ + 1 and len(edge) == 2
            assert edge == [vis[0], vis[-1]]


def test_tiles_ragged_tail_is_edge():
    got = oracle.band_tiles_bruteforce("causal", 10, 100, 4, 4)
    # last key block covers columns 8..11; 10, 11 are out of range -> partial
    assert got[2] == ([0, 1, 2], [2])
    assert got[1] == ([0, 1], [1])
