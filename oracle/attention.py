"""Masked softmax attention over explicit connectivity sets, in float64 (oracle).

Test infrastructure only (see ``oracle/__init__.py`` for the citation tags and
the list of who may import this).  The definition followed throughout is the
unified form of [PP] §11.1 and [KB] §2 (alpha^SWA, o^SWA): for a query position
t with connectivity set S_t,

    e_s = scale * (q_t . k_s),   alpha_ts = exp(e_s) / sum_{s' in S_t} exp(e_s'),
    o_t = sum_{s in S_t} alpha_ts v_s,

with scale = 1/sqrt(d_h) by default ([KB] §2, [MB] scaled dot product).
The softmax is the plain two-pass form (subtract the row maximum, exponentiate,
sum); there is no streaming, tiling or reordering.  ``lse`` is the natural log
of sum_s exp(e_s) (m + ln l), reported so split-softmax merges can be checked.

Inputs are arrays of the exact values the kernels consume (bf16 values widened
exactly to float32/float64 by the caller); everything is cast to float64 here.
"""

import math

import numpy as np

from .index_sets import (causal_dilated_index_set, causal_index_set, causal_sink_index_set,
                         decode_index_set, longformer_index_set)
from .rope import rope_rotate_half


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def attend(q_row, K, V, scale, sink_logit=None):
    """One query row over the key/value rows of its connectivity set.

    Returns (o [d_v], lse).  An empty set yields o = 0 and lse = -inf (a reading:
    the pages never produce an empty window; only an empty ring cache does).

    ``sink_logit`` (a reading of the learned per-head sink of [ST] "What's New"):
    a score z that joins the softmax denominator with no value row, i.e. an
    always-visible virtual position whose value is zero:
        o = sum_s exp(e_s) v_s / (exp(z) + sum_s exp(e_s)),
        lse = log(exp(z) + sum_s exp(e_s)).
    """
    q_row = _f64(q_row)
    K = _f64(K)
    V = _f64(V)
    z = None if sink_logit is None else float(sink_logit)
    if K.shape[0] == 0:
        if z is None:
            return np.zeros(V.shape[-1], dtype=np.float64), -math.inf
        return np.zeros(V.shape[-1], dtype=np.float64), z
    e = (K @ q_row) * float(scale)            # scores over S_t
    m = e.max() if z is None else max(e.max(), z)
    p = np.exp(e - m)                        # weights before normalisation
    l = p.sum() + (0.0 if z is None else math.exp(z - m))
    o = (p @ V) / l
    return o, m + math.log(l)


def _default_scale(d_h, scale):
    return 1.0 / math.sqrt(d_h) if scale is None else float(scale)


def swa_prefill(q, k, v, W, scale=None, rows=None, n_sink=0, sink_logit=None, dilation=None,
                rope_base=None):
    """Causal sliding-window prefill with grouped-query heads.

    q: [B, T, H_q, d_h]; k, v: [B, T, H_kv, d_h]; query head h reads key/value
    head h // (H_q / H_kv) (contiguous groups; [ST] "Combining SWA with GQA"
    fixes only that several query heads share one key/value head, the grouping
    is a reading).  S_t is the causal window of ``causal_index_set``.
    ``rows`` optionally restricts the computation to those query positions.
    ``n_sink`` > 0 adds the first n_sink positions to every window
    (``causal_sink_index_set``); ``sink_logit`` [H_q] gives each head a sink
    score in the denominator (see ``attend``).
    ``dilation`` [H_q] (ints >= 1) gives head h the dilated window
    {t - i*d_h : 0 <= i < W} of ``causal_dilated_index_set`` ([KB] §2 "Dilation").
    ``rope_base``: q and k are first rotated by rotary position embeddings at
    their token positions 0..T-1 (``rope.rope_rotate_half``; [G3] fixes the base
    1e4 for local layers, [KB] §2 1e4 local / 1e6 global).
    Returns o [B, R, H_q, d_h] and lse [B, H_q, R] (R = len(rows) or T).
    """
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    if Hq % Hkv:
        raise ValueError("H_q must be a multiple of H_kv")
    if n_sink and dilation is not None:
        raise ValueError("sinks and dilation are separate variants")
    if rope_base is not None:
        pos = np.arange(T)
        q = rope_rotate_half(q, pos, rope_base)
        k = rope_rotate_half(k, pos, rope_base)
    group = Hq // Hkv
    sc = _default_scale(D, scale)
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, len(rows), Hq, v.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, Hq, len(rows)), dtype=np.float64)
    for b in range(B):
        for ri, t in enumerate(rows):
            if n_sink:
                S_all = causal_sink_index_set(int(t), W, n_sink)
            elif dilation is None:
                S_all = causal_index_set(int(t), W)
            for h in range(Hq):
                kvh = h // group
                S = S_all if dilation is None else causal_dilated_index_set(int(t), W, int(dilation[h]))
                z = None if sink_logit is None else sink_logit[h]
                o[b, ri, h], lse[b, h, ri] = attend(q[b, t, h], k[b, S, kvh], v[b, S, kvh], sc, z)
    return o, lse


def swa_decode(q, k_cache, v_cache, slot_pos, cur_pos, W, scale=None):
    """One new query token per request over a ring cache of W slots.

    q: [B, H_q, d_h]; k_cache, v_cache: [B, H_kv, W, d_h]; slot_pos: [B, W]
    absolute position held by each slot (< 0 = empty); cur_pos: [B].
    Attended slots are those of ``decode_index_set`` ([KB] §2 "KV cache",
    [G3] "How it works").  Returns o [B, H_q, d_h], lse [B, H_q].
    """
    B, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    sc = _default_scale(D, scale)
    o = np.zeros((B, Hq, v_cache.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, Hq), dtype=np.float64)
    for b in range(B):
        S = decode_index_set(slot_pos[b], int(cur_pos[b]), W)
        for h in range(Hq):
            kvh = h // group
            o[b, h], lse[b, h] = attend(q[b, h], k_cache[b, kvh, S], v_cache[b, kvh, S], sc)
    return o, lse


def swa_prefill_cached(q, k_cache, v_cache, slot_pos, q_pos, W, scale=None, n_sink=0,
                       sink_logit=None, rows=None):
    """A chunk of L query tokens per request over a ring cache of S slots.

    [G3] "How it works": queries carry absolute positions ([B, L]) and the cache
    carries the position of each slot ([B, S]); the window is computed from
    those positions, so query t attends the slots holding a position p with
    q_pos[t]-W < p <= q_pos[t] (``decode_index_set`` with cur = q_pos[t]).  A
    single-token chunk is ring decode.  ``n_sink`` / ``sink_logit`` as in
    ``swa_prefill`` (slots holding one of the first n_sink positions stay visible).
    q: [B, L, H_q, d_h]; k_cache, v_cache: [B, H_kv, S, d_h]; slot_pos: [B, S]
    (< 0 = empty); q_pos: [B, L].  ``rows`` optionally restricts the computation
    to those query tokens.  Returns o [B, R, H_q, d_h], lse [B, H_q, R]
    (R = len(rows) or L).
    """
    B, L, Hq, D = q.shape
    Hkv = k_cache.shape[1]
    group = Hq // Hkv
    sc = _default_scale(D, scale)
    rows = np.arange(L) if rows is None else np.asarray(rows, dtype=np.int64)
    o = np.zeros((B, len(rows), Hq, v_cache.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, Hq, len(rows)), dtype=np.float64)
    for b in range(B):
        for ri, t in enumerate(rows):
            S_t = decode_index_set(slot_pos[b], int(q_pos[b, t]), W, n_sink)
            for h in range(Hq):
                kvh = h // group
                z = None if sink_logit is None else sink_logit[h]
                o[b, ri, h], lse[b, h, ri] = attend(q[b, t, h], k_cache[b, kvh, S_t],
                                                    v_cache[b, kvh, S_t], sc, z)
    return o, lse


def swa_longformer(q, k, v, r, dilation=None, global_idx=None, scale=None, rows=None, heads=None,
                   qg=None, kg=None, vg=None):
    """Longformer-style bidirectional attention: per-head dilated window + globals.

    q, k, v: [B, T, H, d_h]; dilation: [H] ints >= 1 (None = all 1);
    global_idx: [B, G] positions (None or G = 0 = no globals).
    S_i follows ``longformer_index_set`` ([PP] §1.1, §3.1, §4.3).
    ``rows``/``heads`` optionally restrict the computation.

    ``qg, kg, vg`` ([B, T, H, d_h], all three or none): the separate global
    projections of [PP] §5.2.  A global row uses qg for its query and kg, vg for
    every position; a local row keeps its sliding query q, reads its window
    positions that are not global through k, v, and every global position
    through kg, vg.  With qg, kg, vg equal to q, k, v this is the shared form
    ([PP] §5.3: the global projections start as copies of the sliding ones).
    Returns o [B, R, H', d_h], lse [B, H', R].
    """
    if qg is not None:
        return _longformer_two_proj(q, k, v, qg, kg, vg, r, dilation, global_idx, scale, rows, heads)
    B, T, H, D = q.shape
    sc = _default_scale(D, scale)
    dil = [1] * H if dilation is None else [int(x) for x in dilation]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((B, len(rows), len(heads), v.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, len(heads), len(rows)), dtype=np.float64)
    for b in range(B):
        G = () if global_idx is None else [int(g) for g in np.asarray(global_idx)[b]]
        for hi, h in enumerate(heads):
            for ri, i in enumerate(rows):
                S = longformer_index_set(int(i), T, r, dil[h], G)
                o[b, ri, hi], lse[b, hi, ri] = attend(q[b, i, h], k[b, S, h], v[b, S, h], sc)
    return o, lse


def _longformer_two_proj(q, k, v, qg, kg, vg, r, dilation, global_idx, scale, rows, heads):
    B, T, H, D = q.shape
    sc = _default_scale(D, scale)
    dil = [1] * H if dilation is None else [int(x) for x in dilation]
    rows = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = list(range(H)) if heads is None else list(heads)
    o = np.zeros((B, len(rows), len(heads), v.shape[-1]), dtype=np.float64)
    lse = np.zeros((B, len(heads), len(rows)), dtype=np.float64)
    for b in range(B):
        G = [] if global_idx is None else sorted(int(g) for g in np.asarray(global_idx)[b])
        for hi, h in enumerate(heads):
            for ri, i in enumerate(rows):
                if i in G:                          # [PP] §5.2: Q_g against K_g, V_g of all
                    o[b, ri, hi], lse[b, hi, ri] = attend(qg[b, i, h], kg[b, :, h], vg[b, :, h], sc)
                    continue
                S = longformer_index_set(int(i), T, r, dil[h], G)
                local = np.array([j for j in S if j not in G], dtype=np.int64)
                Kx = np.concatenate([_f64(k[b, local, h]).reshape(-1, D), _f64(kg[b, G, h]).reshape(-1, D)])
                Vx = np.concatenate([_f64(v[b, local, h]).reshape(-1, v.shape[-1]),
                                     _f64(vg[b, G, h]).reshape(-1, v.shape[-1])])
                o[b, ri, hi], lse[b, hi, ri] = attend(q[b, i, h], Kx, Vx, sc)
    return o, lse


def dense_masked_attention(q, k, v, mask, scale):
    """The literal dense form of [KB] §3 (and [MB]'s four steps): full [T, T]
    scores, masked_fill(~mask, -inf), row softmax, then weights @ V.

    q, k: [T, d]; v: [T, d_v]; mask: bool [T, T].  Used only to cross-check the
    index-set form on small inputs.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    scores = (q @ k.T) * float(scale)
    scores = np.where(mask, scores, -np.inf)
    mx = scores.max(axis=1, keepdims=True)
    p = np.exp(scores - mx)
    attn = p / p.sum(axis=1, keepdims=True)
    return attn @ v
