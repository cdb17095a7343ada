"""Connectivity sets S_t of sliding-window attention (oracle; test infrastructure).

Each function returns the sorted int64 array of key positions that query
position ``t`` attends.  Tags ([KB], [MB], [G3], [PP], [ST]) are defined in
``oracle/__init__.py``.
"""

import numpy as np


def causal_index_set(t: int, W: int) -> np.ndarray:
    """Causal window: keys s with max(0, t-W+1) <= s <= t (W keys, self included).

    [KB] §2 "Derivation": the window N_t = [max(0, t-W+1), t]; §3 "Reference
    implementation": the mask is 1 iff t-W < s <= t.  [G3] "How it works": the
    conjunction that fires is t-W < s <= t (t=2000, W=1024 keeps 977..2000).
    [ST] "The Mechanism": causal range [i-w+1, i].
    """
    if W < 1:
        raise ValueError("W must be >= 1")
    return np.arange(max(0, t - W + 1), t + 1, dtype=np.int64)


def causal_dilated_index_set(t: int, W: int, dilation: int = 1) -> np.ndarray:
    """Dilated causal window: keys t - i*d for 0 <= i < W that are >= 0.

    [KB] §2 "Dilation": the window N_t is replaced by {t - i*d : 0 <= i < W}
    with gap d >= 1 (heads may use different d).  Positions below 0 do not
    exist, so the set is cut there, as the undilated window is (a reading: the
    page does not spell out the start of the sequence).  d = 1 is the causal
    window of ``causal_index_set``.
    """
    if W < 1 or dilation < 1:
        raise ValueError("need W >= 1 and dilation >= 1")
    keys = [t - i * dilation for i in range(W) if t - i * dilation >= 0]
    return np.asarray(sorted(keys), dtype=np.int64)


def symmetric_index_set(i: int, n: int, r: int, dilation: int = 1) -> np.ndarray:
    """Symmetric (encoder) window with optional dilation, clipped to [0, n-1].

    [PP] §1.1: S_i = {j : |i-j| <= r} clipped to [0, n-1].
    [PP] §3.1: dilated S_i^(d) = {i + k*d : k in [-r, r]} clipped to [0, n-1].
    """
    if r < 0 or dilation < 1:
        raise ValueError("need r >= 0 and dilation >= 1")
    out = [i + k * dilation for k in range(-r, r + 1) if 0 <= i + k * dilation < n]
    return np.asarray(out, dtype=np.int64)


def longformer_index_set(i: int, n: int, r: int, dilation: int = 1, globals_=()) -> np.ndarray:
    """Window plus global attention, Longformer style.

    [PP] §4.3: a global position attends every position 0..n-1; a local position
    attends its window united with G.  The union counts a global key that is
    already inside the window once ([PP] §4.4 note under the table).
    [KB] §2 "Global attention augmentation" gives the same two rules.
    Dilation applies only to the window part (a reading: the pages are silent on
    globals combined with dilation).
    """
    G = sorted(set(int(g) for g in globals_))
    for g in G:
        if not 0 <= g < n:
            raise ValueError("global index out of range")
    if i in G:
        return np.arange(n, dtype=np.int64)
    window = set(symmetric_index_set(i, n, r, dilation).tolist())
    return np.asarray(sorted(window | set(G)), dtype=np.int64)


def causal_sink_index_set(t: int, W: int, n_sink: int) -> np.ndarray:
    """Causal window plus attention-sink tokens: the first n_sink positions stay
    visible to every later query alongside its rolling window ([KB] §4,
    "Failure mode 1": StreamingLLM keeps the first few KV slots pinned next to
    the rolling window; [ST] "What's New": sink positions every query sees).
    Union, each key once:
    (t-W, t] together with {s : s < n_sink, s <= t}.
    """
    win = causal_index_set(t, W)
    sinks = np.arange(min(n_sink, t + 1), dtype=np.int64)
    return np.union1d(sinks, win).astype(np.int64)


def decode_index_set(slot_pos_row, cur: int, W: int, n_sink: int = 0) -> np.ndarray:
    """Ring-cache slots attended by the query at absolute position ``cur``.

    The window is computed from the absolute token position stored in each slot,
    never from the slot's offset ([G3] "How it works": cache positions are kept
    with the cache so the mask uses true token indices).  A slot is attended iff
    it holds a position p with cur-W < p <= cur (the causal window of [KB] §2).
    Negative positions mark empty slots (a reading: the pages fix no sentinel).
    Returns slot indices.
    With n_sink > 0, slots holding one of the first n_sink positions (p <= cur)
    are attended too (pinned sink tokens, see ``causal_sink_index_set``).
    """
    sp = np.asarray(slot_pos_row, dtype=np.int64)
    ok = (sp >= 0) & (sp <= cur) & ((sp > cur - W) | (sp < n_sink))
    return np.nonzero(ok)[0].astype(np.int64)


def causal_mask(T: int, W: int) -> np.ndarray:
    """Dense boolean [T, T] causal-window mask, written as [KB] §3 builds it:
    causal = s <= t, window = s > t - W, mask = causal & window."""
    t_idx = np.arange(T).reshape(T, 1)
    s_idx = np.arange(T).reshape(1, T)
    return (s_idx <= t_idx) & (s_idx > t_idx - W)


def longformer_mask(n: int, r: int, dilation: int = 1, globals_=()) -> np.ndarray:
    """Dense boolean [n, n] mask from the Longformer connectivity sets ([PP] §4.3)."""
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        m[i, longformer_index_set(i, n, r, dilation, globals_)] = True
    return m
