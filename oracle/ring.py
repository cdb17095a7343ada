"""Rolling-buffer KV cache write rule (oracle; test infrastructure).

[KB] §2 "KV cache": the key and value of token i live in slot i mod W of a
fixed W-slot buffer, so writing token i overwrites token i - W.  Each slot also
records the absolute position it holds ([G3] "How it works": positions are
stored with the cache so the window is computed from true token indices).
Empty slots hold position -1 (a reading; the pages fix no sentinel).
"""

import numpy as np


def ring_write(k_cache, v_cache, slot_pos, k_new, v_new, pos):
    """Write one token per request into its ring slot, in place.

    k_cache, v_cache: [B, H_kv, W, d]; slot_pos: [B, W]; k_new, v_new: [B, H_kv, d];
    pos: [B] absolute positions.
    """
    W = slot_pos.shape[1]
    for b in range(slot_pos.shape[0]):
        j = int(pos[b]) % W
        k_cache[b, :, j] = k_new[b]
        v_cache[b, :, j] = v_new[b]
        slot_pos[b, j] = int(pos[b])


def ring_from_sequence(k_seq, v_seq, upto, W):
    """Replay tokens 0..upto[b] of a sequence through ``ring_write``.

    k_seq, v_seq: [B, T, H_kv, d] (sequence layout); upto: [B] last written position.
    Returns (k_cache, v_cache, slot_pos) after the writes, float64 caches.
    """
    B, T, Hkv, D = k_seq.shape
    k_cache = np.zeros((B, Hkv, W, D), dtype=np.float64)
    v_cache = np.zeros((B, Hkv, W, v_seq.shape[-1]), dtype=np.float64)
    slot_pos = np.full((B, W), -1, dtype=np.int64)
    for p in range(int(np.max(upto)) + 1):
        live = [b for b in range(B) if p <= int(upto[b])]
        for b in live:
            j = p % W
            k_cache[b, :, j] = k_seq[b, p]
            v_cache[b, :, j] = v_seq[b, p]
            slot_pos[b, j] = p
    return k_cache, v_cache, slot_pos


def ring_slot(p: int, S: int, n_sink: int = 0) -> int:
    """Slot of absolute position p in a cache of S slots.  Without sinks this is
    the rolling buffer's p mod S ([KB] §2 "KV cache").  With n_sink pinned sink
    tokens ([KB] §4 "Failure mode 1": the first few KV slots stay pinned next to a
    rolling window) positions p < n_sink keep slot p and the rest roll over the
    other S - n_sink slots (a reading: the pages fix no layout)."""
    if p < n_sink:
        return p
    return n_sink + (p - n_sink) % (S - n_sink)


def ring_append(k_cache, v_cache, slot_pos, k_new, v_new, pos, n_sink=0):
    """Write a chunk of tokens per request into a cache of S slots, in place.

    The same rule as ``ring_write`` applied to each token in order: token t of
    request b lands in slot ``ring_slot(pos[b, t], S, n_sink)`` ([KB] §2 "KV
    cache"; pos mod S without sinks) and the slot records pos[b, t] ([G3] "How
    it works").
    k_cache, v_cache: [B, H_kv, S, d]; slot_pos: [B, S];
    k_new, v_new: [B, L, H_kv, d]; pos: [B, L] absolute positions.
    """
    pos = np.asarray(pos)
    B, L = pos.shape
    S = slot_pos.shape[1]
    for t in range(L):
        for b in range(B):
            j = ring_slot(int(pos[b, t]), S, n_sink)
            k_cache[b, :, j] = k_new[b, t]
            v_cache[b, :, j] = v_new[b, t]
            slot_pos[b, j] = int(pos[b, t])

