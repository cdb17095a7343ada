"""Brute-force band-tile classification (oracle; test infrastructure).

A kernel that never materialises the T x T score grid visits, for each block of
BM query rows, only the key blocks of BN columns that intersect the band, and
needs a mask only where a visited block is partly outside the band ([PP] §6.1
and §6.3: only the banded entries are computed; [KB] §3 closing comment: the
band is iterated per query instead of the full grid; [ST] "The Mechanism":
out-of-window key/value blocks are skipped).

This module classifies every (query block, key block) pair by testing every
(t, s) element against the oracle's own connectivity sets — no interval
arithmetic — so a tile schedule can be compared with it bit for bit.
"""

import numpy as np

from .index_sets import causal_index_set, longformer_index_set


def _sets(mode, T, w_or_r, dil, globals_):
    if mode == "causal":
        return [set(causal_index_set(t, w_or_r).tolist()) for t in range(T)]
    if mode == "symmetric":
        return [set(longformer_index_set(t, T, w_or_r, dil, globals_).tolist()) for t in range(T)]
    raise ValueError(mode)


def band_tiles_bruteforce(mode, T, w_or_r, BM, BN, dil=1, globals_=()):
    """For every query block qi, the visited key blocks and which of them need a mask.

    visited(qi, kj): some valid (t, s) pair in the block pair is attended.
    edge(qi, kj):    visited, and some pair of the block pair — including columns
                     s >= T of a ragged last key block — is not attended.
    Rows t >= T of a ragged last query block are ignored (they are not outputs).

    Returns a list over query blocks of (visited_blocks, edge_blocks), each a
    sorted list of key-block indices.
    """
    sets = _sets(mode, T, w_or_r, dil, globals_)
    nq = -(-T // BM)
    nk = -(-T // BN)
    out = []
    for qi in range(nq):
        rows = range(qi * BM, min(T, (qi + 1) * BM))
        visited, edge = [], []
        for kj in range(nk):
            cols = range(kj * BN, (kj + 1) * BN)
            hit = np.array([[s < T and s in sets[t] for s in cols] for t in rows])
            if hit.any():
                visited.append(kj)
                if not hit.all():
                    edge.append(kj)
        out.append((visited, edge))
    return out
