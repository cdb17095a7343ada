"""Thin ctypes binding over libswa.so.

Argument marshalling only: tensors become device pointers, the current HIP
stream is passed through, and status codes become exceptions.  Every step of
the computation runs in the library's HIP kernels; there is no fallback.  If
the library has not been built, every call raises.
"""

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswa.so")

SWA_BF16, SWA_F32 = 0, 1
SWA_MODE_CAUSAL, SWA_MODE_SYMMETRIC = 0, 1

_lib = None


class SwaError(RuntimeError):
    def __init__(self, code, what):
        self.code = code
        super().__init__(f"{what}: {status_str(code)} ({code})")


def lib():
    """Load libswa.so once; raise if it is missing (no CPU fallback exists)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libswa.so not built ({LIB_PATH}); run "
                               "python -m sliding_window_attention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.swa_prefill.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
        L.swa_decode_workspace_size.argtypes = [i, i, i, i, i]
        L.swa_decode_workspace_size.restype = sz
        L.swa_decode.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp, sz, vp]
        L.swa_decode_noalloc.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, f, vp]
        L.swa_cache_write.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, vp]
        L.swa_cache_append.argtypes = [i, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
        L.swa_prefill_cached.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, i,
                                         vp, f, vp]
        L.swa_prefill_sinks.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, f, vp]
        L.swa_prefill_dilated.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp, f, vp]
        L.swa_rope.argtypes = [i, vp, vp, vp, i, i, i, i, f, vp]
        L.swa_prefill_rope_workspace_size.argtypes = [i, i, i, i, i]
        L.swa_prefill_rope_workspace_size.restype = sz
        L.swa_prefill_rope.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, i, f, f, vp, sz, vp]
        L.swa_longformer_workspace_size.argtypes = [i, i, i, i, i]
        L.swa_longformer_workspace_size.restype = sz
        L.swa_longformer.argtypes = [i, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp, i, f, vp, sz, vp]
        L.swa_longformer_proj.argtypes = [i, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, vp,
                                          i, f, vp, sz, vp]
        L.swa_tile_config.argtypes = [i, i, i, i, ctypes.POINTER(i), ctypes.POINTER(i)]
        L.swa_band_tiles.argtypes = [i, i, i, i, i, vp, i]
        L.swa_debug_index_mask.argtypes = [i, i, i, i, vp, i, vp, vp]
        L.swa_status_str.argtypes = [i]
        L.swa_status_str.restype = ctypes.c_char_p
        for name in ("swa_prefill", "swa_prefill_sinks", "swa_prefill_dilated", "swa_rope",
                     "swa_prefill_rope",
                     "swa_prefill_cached", "swa_decode", "swa_decode_noalloc",
                     "swa_cache_write", "swa_cache_append", "swa_longformer",
                     "swa_longformer_proj", "swa_tile_config", "swa_debug_index_mask"):
            getattr(L, name).restype = i
        L.swa_band_tiles.restype = i
        L.swa_version.restype = i
        _lib = L
    return _lib


def status_str(code):
    return lib().swa_status_str(code).decode()


def _check(code, what):
    if code != 0:
        raise SwaError(code, what)


def _dt(t):
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype == torch.float32:
        return SWA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t, name, ndim):
    if not t.is_cuda or not t.is_contiguous() or t.dim() != ndim:
        raise ValueError(f"{name} must be a contiguous {ndim}-d device tensor")


def prefill(q, k, v, W, scale=None, out=None, return_lse=False):
    """Causal sliding-window attention: q [B,T,Hq,D], k/v [B,T,Hkv,D] -> o [B,T,Hq,D]."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, T, device=q.device, dtype=torch.float32) if return_lse else None
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_prefill(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             B, T, Hq, Hkv, D, int(W), sc, _stream(q)), "swa_prefill")
    return (o, lse) if return_lse else o


def prefill_sinks(q, k, v, W, n_sink=0, sink_logit=None, scale=None, out=None,
                  return_lse=False):
    """Causal window plus the first n_sink tokens and an optional per-head sink
    score (sink_logit: float32 device tensor [Hq] or None)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    if sink_logit is not None:
        _need(sink_logit, "sink_logit", 1)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, T, device=q.device, dtype=torch.float32) if return_lse else None
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_prefill_sinks(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq,
                                   Hkv, D, int(W), int(n_sink), _ptr(sink_logit), sc, _stream(q)),
           "swa_prefill_sinks")
    return (o, lse) if return_lse else o


def prefill_dilated(q, k, v, W, dilation=None, scale=None, out=None, return_lse=False):
    """Causal windows {t - i*d : 0 <= i < W} with d = dilation[h] per query head
    (host int sequence [Hq] or None = all 1)."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    dil = None
    if dilation is not None:
        if len(dilation) != Hq:
            raise ValueError("dilation needs one entry per query head")
        dil = (ctypes.c_int32 * Hq)(*[int(x) for x in dilation])
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, T, device=q.device, dtype=torch.float32) if return_lse else None
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_prefill_dilated(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T,
                                     Hq, Hkv, D, int(W), dil, sc, _stream(q)),
           "swa_prefill_dilated")
    return (o, lse) if return_lse else o


def rope(x, base, pos=None, out=None):
    """Rotary positions (rotate-half pairs) of x [B,T,H,D] at positions pos
    (device int32 [B,T]) or t; out may be x (in place)."""
    _need(x, "x", 4)
    if pos is not None:
        _need(pos, "pos", 2)
    B, T, H, D = x.shape
    y = torch.empty_like(x) if out is None else out
    _check(lib().swa_rope(_dt(x), _ptr(x), _ptr(y), _ptr(pos), B, T, H, D, float(base),
                          _stream(x)), "swa_rope")
    return y


def prefill_rope_workspace_size(dtype_code, B, T, Hkv, D):
    return int(lib().swa_prefill_rope_workspace_size(dtype_code, B, T, Hkv, D))


def prefill_rope(q, k, v, W, rope_base, scale=None, out=None, workspace=None, return_lse=False):
    """swa_prefill of rope(q), rope(k), v: q rotated inside the kernel, k rotated
    once into the workspace."""
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, T, device=q.device, dtype=torch.float32) if return_lse else None
    need = prefill_rope_workspace_size(_dt(q), B, T, Hkv, D)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                            device=q.device)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_prefill_rope(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, T, Hq,
                                  Hkv, D, int(W), float(rope_base), sc, _ptr(ws),
                                  ws.numel() * ws.element_size(), _stream(q)), "swa_prefill_rope")
    return (o, lse) if return_lse else o


def decode_workspace_size(B, Hq, Hkv, W, D):
    return int(lib().swa_decode_workspace_size(B, Hq, Hkv, W, D))


def decode(q, k_cache, v_cache, slot_pos, cur_pos, scale=None, out=None, workspace=None,
           return_lse=False):
    """Ring-cache decode: q [B,Hq,D], caches [B,Hkv,W,D], slot_pos [B,W], cur_pos [B]."""
    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(slot_pos, "slot_pos", 2)
    _need(cur_pos, "cur_pos", 1)
    B, Hq, D = q.shape
    Hkv, W = k_cache.shape[1], k_cache.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32) if return_lse else None
    need = decode_workspace_size(B, Hq, Hkv, W, D)
    ws = workspace if workspace is not None else torch.empty(max(need, 1), dtype=torch.uint8,
                                                            device=q.device)
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_decode(_dt(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(slot_pos),
                            _ptr(cur_pos), _ptr(o), _ptr(lse), B, W, Hq, Hkv, D, sc, _ptr(ws),
                            ws.numel() * ws.element_size(), _stream(q)), "swa_decode")
    return (o, lse) if return_lse else o


# the size of the library's per-GPU scratch array (SWA_DECODE_NOALLOC_SCRATCH_BYTES)
DECODE_NOALLOC_SCRATCH_BYTES = 16 << 20


def decode_noalloc(q, k_cache, v_cache, slot_pos, cur_pos, scale=None, out=None,
                   return_lse=False):
    """Ring-cache decode through swa_decode_noalloc: as decode(), with the
    library's per-GPU scratch array instead of a workspace (only o and lse are
    allocated here, and not when `out` is given without return_lse)."""
    _need(q, "q", 3)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(slot_pos, "slot_pos", 2)
    _need(cur_pos, "cur_pos", 1)
    B, Hq, D = q.shape
    Hkv, W = k_cache.shape[1], k_cache.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, device=q.device, dtype=torch.float32) if return_lse else None
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_decode_noalloc(_dt(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(slot_pos),
                                    _ptr(cur_pos), _ptr(o), _ptr(lse), B, W, Hq, Hkv, D, sc,
                                    _stream(q)), "swa_decode_noalloc")
    return (o, lse) if return_lse else o


def cache_write(k_new, v_new, pos, k_cache, v_cache, slot_pos):
    """Append one token per request: slot pos mod W of the ring caches."""
    B, Hkv, W, D = k_cache.shape
    _check(lib().swa_cache_write(_dt(k_new), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(k_cache),
                                 _ptr(v_cache), _ptr(slot_pos), B, W, Hkv, D, _stream(k_new)),
           "swa_cache_write")


def cache_append(k_new, v_new, pos, k_cache, v_cache, slot_pos, n_sink=0):
    """Append a chunk per request: k_new/v_new [B,L,Hkv,D], pos [B,L] -> slots pos mod S
    (positions below n_sink keep their own slots; the rest roll over the others)."""
    _need(k_new, "k_new", 4)
    _need(v_new, "v_new", 4)
    _need(pos, "pos", 2)
    B, L, Hkv, D = k_new.shape
    S = k_cache.shape[2]
    _check(lib().swa_cache_append(_dt(k_new), _ptr(k_new), _ptr(v_new), _ptr(pos), _ptr(k_cache),
                                  _ptr(v_cache), _ptr(slot_pos), B, L, S, Hkv, D, int(n_sink),
                                  _stream(k_new)), "swa_cache_append")


def prefill_cached(q, k_cache, v_cache, slot_pos, q_pos, W, scale=None, out=None,
                   return_lse=False, n_sink=0, sink_logit=None):
    """Chunked prefill over a ring cache: q [B,L,Hq,D], caches [B,Hkv,S,D],
    slot_pos [B,S], q_pos [B,L] -> o [B,L,Hq,D] (lse [B,Hq,L])."""
    _need(q, "q", 4)
    _need(k_cache, "k_cache", 4)
    _need(v_cache, "v_cache", 4)
    _need(slot_pos, "slot_pos", 2)
    _need(q_pos, "q_pos", 2)
    B, L, Hq, D = q.shape
    Hkv, S = k_cache.shape[1], k_cache.shape[2]
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, Hq, L, device=q.device, dtype=torch.float32) if return_lse else None
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    _check(lib().swa_prefill_cached(_dt(q), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(slot_pos),
                                    _ptr(q_pos), _ptr(o), _ptr(lse), B, L, S, Hq, Hkv, D, int(W),
                                    int(n_sink), _ptr(sink_logit), sc, _stream(q)),
           "swa_prefill_cached")
    return (o, lse) if return_lse else o


def longformer_workspace_size(B, T, H, D, G):
    return int(lib().swa_longformer_workspace_size(B, T, H, D, G))


def longformer(q, k, v, r, dilation=None, global_idx=None, scale=None, out=None, workspace=None,
               return_lse=False, qg=None, kg=None, vg=None):
    """Bidirectional window |i-j| <= r (per-head dilation) plus global tokens.

    dilation: host int sequence [H] or None; global_idx: host int array [B, G] or None.
    qg, kg, vg (all three or none, shaped like q): separate global projections
    (swa_longformer_proj).
    """
    for t, n in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, n, 4)
    proj = (qg, kg, vg)
    if any(x is not None for x in proj):
        if any(x is None for x in proj):
            raise ValueError("qg, kg and vg go together")
        for t, n in zip(proj, ("qg", "kg", "vg")):
            _need(t, n, 4)
            if t.shape != q.shape or t.dtype != q.dtype:
                raise ValueError(f"{n} must match q in shape and dtype")
    B, T, H, D = q.shape
    dil = None
    if dilation is not None:
        dil = (ctypes.c_int32 * H)(*[int(x) for x in dilation])
    G = 0
    gl = None
    if global_idx is not None:
        rows = [[int(x) for x in row] for row in global_idx]
        G = len(rows[0]) if rows else 0
        if G:
            flat = [x for row in rows for x in row]
            gl = (ctypes.c_int32 * len(flat))(*flat)
    o = torch.empty_like(q) if out is None else out
    lse = torch.empty(B, H, T, device=q.device, dtype=torch.float32) if return_lse else None
    need = longformer_workspace_size(B, T, H, D, G)
    ws = workspace
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=q.device)
    ws_bytes = 0 if ws is None else ws.numel() * ws.element_size()
    sc = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if qg is None:
        _check(lib().swa_longformer(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                                    B, T, H, D, int(r), dil, gl, G, sc, _ptr(ws), ws_bytes,
                                    _stream(q)), "swa_longformer")
    else:
        _check(lib().swa_longformer_proj(_dt(q), _ptr(q), _ptr(k), _ptr(v), _ptr(qg), _ptr(kg),
                                         _ptr(vg), _ptr(o), _ptr(lse), B, T, H, D, int(r), dil,
                                         gl, G, sc, _ptr(ws), ws_bytes, _stream(q)),
               "swa_longformer_proj")
    return (o, lse) if return_lse else o


def tile_config(entry, Hq, Hkv, D):
    bm, bn = ctypes.c_int(), ctypes.c_int()
    _check(lib().swa_tile_config(ord(entry), Hq, Hkv, D, ctypes.byref(bm), ctypes.byref(bn)),
           "swa_tile_config")
    return bm.value, bn.value


def band_tiles(mode, T, w_or_r, BM, BN):
    """The kernels' tile schedule as a list of (qi, kj, needs_mask) triples (host call)."""
    n = lib().swa_band_tiles(mode, T, w_or_r, BM, BN, None, 0)
    if n < 0:
        raise ValueError("invalid band_tiles arguments")
    buf = (ctypes.c_int32 * max(1, 3 * n))()
    lib().swa_band_tiles(mode, T, w_or_r, BM, BN, buf, n)
    return [(buf[3 * i], buf[3 * i + 1], buf[3 * i + 2]) for i in range(n)]


def debug_index_mask(mode, T, w_or_r, dil=1, globals_=(), device="cuda"):
    """The kernels' window predicate evaluated on the device as a uint8 [T, T] matrix."""
    m = torch.empty(T, T, dtype=torch.uint8, device=device)
    G = len(globals_)
    gl = (ctypes.c_int32 * max(1, G))(*[int(x) for x in globals_]) if G else None
    _check(lib().swa_debug_index_mask(mode, T, w_or_r, dil, gl, G, _ptr(m), _stream(m)),
           "swa_debug_index_mask")
    return m
