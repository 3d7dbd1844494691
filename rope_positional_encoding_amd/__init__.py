"""Python binding of libwaveprune: WavePrune (RoPE first-period truncation)
attention on AMD MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libwaveprune.so, reached through its C ABI (include/waveprune.h)
with ctypes.  torch provides device memory and the current HIP stream.  If
the shared library is missing this module raises on first use -- there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

import torch

__all__ = [
    "WPError", "lib", "group_cutoffs", "rope_apply", "prefill", "decode", "decode_noalloc",
    "decode_num_splits", "decode_workspace_size", "prefill_tiling", "decode_tiling",
    "prefill_tile_counts", "decode_tile_counts", "FLAG_DENSE", "FLAG_COUNT", "NEVER_PRUNE",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwaveprune.so")

FLAG_DENSE = 1
FLAG_COUNT = 2
FLAG_MFMA16 = 4
NEVER_PRUNE = 2 ** 31 - 1
DTYPE_BF16 = 0
DTYPE_F32 = 1

_i32 = ctypes.c_int32
_i64 = ctypes.c_int64
_u32 = ctypes.c_uint32
_dbl = ctypes.c_double
_vp = ctypes.c_void_p
_sz = ctypes.c_size_t
_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)

_SIGNATURES = {
    "wp_group_cutoffs": (_i32, [_dbl, _i32, _i32, _dbl, _I32P, _i32]),
    "wp_cutoffs_from_freqs": (_i32, [ctypes.POINTER(ctypes.c_double), _i32, _dbl, _i32, _i32, _I32P, _i32]),
    "wp_rope_apply": (_i32, [_vp, _i32, _vp, _i32, _i32, _i32, _i32, _I64P, _I64P, _vp, _dbl, _dbl, _vp]),
    "wp_prefill": (_i32, [_vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _I64P, _I32P, _i32,
                          _u32, _vp, _vp]),
    "wp_decode": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _I64P, _I32P, _i32,
                         _i32, _vp, _sz, _u32, _vp, _vp]),
    "wp_decode_noalloc": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _I64P, _I32P,
                                 _i32, _i32, _u32, _vp, _vp]),
    "wp_kcache_layout": (_i32, [_i32, _i32, _i32, _I32P, _I32P, _I64P]),
    "wp_kcache_append": (_i32, [_vp, _i32, _i32, _i32, _i32, _I64P, _vp, _vp, _I64P, _i32, _I32P, _i32, _vp]),
    "wp_decode_kcache": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32, _I64P, _I32P,
                                _i32, _i32, _vp, _sz, _u32, _vp, _vp]),
    "wp_prefill_backward": (_i32, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _i32, _i32, _i32, _i32, _i32,
                                   _I64P, _I32P, _i32, _u32, _vp, _sz, _vp]),
    "wp_prefill_backward_workspace_size": (_sz, [_i32, _i32, _i32]),
    "wp_decode_num_splits": (_i32, [_i32, _i32, _i32]),
    "wp_decode_workspace_size": (_sz, [_i32, _i32, _i32, _i32, _i32, _i32]),
    "wp_prefill_tiling": (_i32, [_i32, _i32, _I32P, _I32P]),
    "wp_decode_tiling": (_i32, [_i32, _i32, _I32P]),
    "wp_prefill_tile_counts": (_i32, [_i32, _i32, _i32, _I32P, _I64P]),
    "wp_decode_tile_counts": (_i32, [_i32, _i32, _i32, _i32, _I32P, _I64P]),
    "wp_status_string": (ctypes.c_char_p, [_i32]),
    "wp_last_error": (ctypes.c_char_p, []),
    "wp_version": (ctypes.c_char_p, []),
}

_LIB: Optional[ctypes.CDLL] = None


class WPError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__("libwaveprune status %d: %s" % (status, message))
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libwaveprune.so (built in-tree by rope_positional_encoding_amd.build)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libwaveprune.so is not built (%s); run "
                               "`python -m rope_positional_encoding_amd.build`" % LIB_PATH)
        # torch is imported first, so the HIP runtime torch loaded is the one
        # this library binds to (same soname), and stream handles are shared.
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB


def _check(status: int) -> None:
    if status != 0:
        msg = lib().wp_last_error().decode()
        raise WPError(status, msg or lib().wp_status_string(status).decode())


def _i64arr(vals: Sequence[int]):
    return (ctypes.c_int64 * len(vals))(*[int(v) for v in vals])


def _i32arr(vals: Sequence[int]):
    return (ctypes.c_int32 * len(vals))(*[int(v) for v in vals])


def _cut(cutoffs: Sequence[int], d_h: int, G: int):
    """The group cutoff table as a C array; the library reads d_h / G entries."""
    if G > 0 and d_h % G == 0 and len(cutoffs) != d_h // G:
        raise ValueError("expected %d cutoffs (d_h / G), got %d" % (d_h // G, len(cutoffs)))
    return _i32arr(cutoffs)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype=None, ndim=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if not t.is_cuda:
        raise ValueError("%s must be a device (HIP) tensor" % name)
    if dtype is not None and t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dims, got shape %s" % (name, ndim, tuple(t.shape)))
    if t.stride(-1) != 1:
        raise ValueError("%s: the head dim must be contiguous" % name)


# ----------------------------------------------------------------------------
def group_cutoffs(theta: float, d_h: int, G: int, pos_scale: float = 1.0) -> list:
    """D'_g table (host computation in the library)."""
    if G <= 0 or d_h % G:
        raise ValueError("G must divide d_h")
    ng = d_h // G
    out = (ctypes.c_int32 * max(ng, 1))()
    _check(lib().wp_group_cutoffs(float(theta), int(d_h), int(G), float(pos_scale), out, ng))
    return [int(v) for v in out[:ng]]


def cutoffs_from_freqs(freqs: Sequence[float], G: int, alpha: float = 2.0,
                       trunc_channels: Optional[int] = None) -> list:
    """Group cutoff table from a per-channel frequency vector (radians per
    position, scaling applied), the window alpha*pi/f and the number of
    leading channels that are truncated (default: all)."""
    n_ch = len(freqs)
    if trunc_channels is None:
        trunc_channels = n_ch
    if G <= 0 or (2 * n_ch) % G:
        raise ValueError("G must divide 2 * len(freqs)")
    ng = 2 * n_ch // G
    f = (ctypes.c_double * max(n_ch, 1))(*[float(x) for x in freqs])
    out = (ctypes.c_int32 * max(ng, 1))()
    _check(lib().wp_cutoffs_from_freqs(f, n_ch, float(alpha), int(trunc_channels), int(G), out, ng))
    return [int(v) for v in out[:ng]]


def prefill_tiling(d_h: int, G: int):
    bm, bn = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().wp_prefill_tiling(d_h, G, ctypes.byref(bm), ctypes.byref(bn)))
    return bm.value, bn.value


def decode_tiling(d_h: int, G: int) -> int:
    bn = ctypes.c_int32()
    _check(lib().wp_decode_tiling(d_h, G, ctypes.byref(bn)))
    return bn.value


def prefill_tile_counts(n: int, d_h: int, G: int, cutoffs: Sequence[int]):
    ng = d_h // G
    out = (ctypes.c_int64 * (3 * ng + 1))()
    _check(lib().wp_prefill_tile_counts(n, d_h, G, _cut(cutoffs, d_h, G), out))
    return [int(v) for v in out]


def decode_tile_counts(q_pos: int, cache_len: int, d_h: int, G: int, cutoffs: Sequence[int]):
    ng = d_h // G
    out = (ctypes.c_int64 * (3 * ng + 1))()
    _check(lib().wp_decode_tile_counts(q_pos, cache_len, d_h, G, _cut(cutoffs, d_h, G), out))
    return [int(v) for v in out]


def decode_num_splits(B: int, Lmax: int, Hkv: int) -> int:
    return int(lib().wp_decode_num_splits(B, Lmax, Hkv))


def decode_workspace_size(B: int, Lmax: int, Hq: int, Hkv: int, d_h: int, num_splits: int = 0) -> int:
    return int(lib().wp_decode_workspace_size(B, Lmax, Hq, Hkv, d_h, num_splits))


# ----------------------------------------------------------------------------
def rope_apply(x: torch.Tensor, theta: float, pos_scale: float = 1.0,
               pos_start: Optional[torch.Tensor] = None,
               out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Rotate x [B, n, H, d_h] (bf16 or fp32) -> bf16 [B, n, H, d_h]."""
    _need(x, "x", ndim=4)
    if x.dtype == torch.bfloat16:
        xd = DTYPE_BF16
    elif x.dtype == torch.float32:
        xd = DTYPE_F32
    else:
        raise TypeError("x must be bf16 or fp32")
    B, n, H, d = x.shape
    if out is None:
        out = torch.empty((B, n, H, d), dtype=torch.bfloat16, device=x.device)
    _need(out, "out", torch.bfloat16, 4)
    if pos_start is not None:
        _need(pos_start, "pos_start", torch.int64, 1)
    _check(lib().wp_rope_apply(
        _ptr(x), xd, _ptr(out), B, n, H, d, _i64arr(x.stride()[:3]), _i64arr(out.stride()[:3]),
        _ptr(pos_start), float(theta), float(pos_scale), _stream(x)))
    return out


def prefill(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, cutoffs: Optional[Sequence[int]],
            G: int, dense: bool = False, return_lse: bool = False,
            counters: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
            lse: Optional[torch.Tensor] = None, variant: Optional[str] = None):
    """Causal WavePrune attention.  q [B, n, Hq, d_h], k/v [B, n, Hkv, d_h]
    (bf16, q/k rotated).  counters: device int64 [3*(d_h/G)+1] to add tile
    counts into (enables WP_FLAG_COUNT).  variant "mfma16x16x32" selects the
    v_mfma_f32_16x16x32_bf16 kernel (d_h = 128, G = 32: WP_FLAG_MFMA16)."""
    if variant not in (None, "mfma16x16x32"):
        raise ValueError("unknown prefill variant %r" % (variant,))
    for t, nm in ((q, "q"), (k, "k"), (v, "v")):
        _need(t, nm, torch.bfloat16, 4)
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    if tuple(k.shape) != (B, n, Hkv, d) or tuple(v.shape) != (B, n, Hkv, d):
        raise ValueError("k and v must be [B, n, Hkv, d_h] matching q")
    if out is None:
        out = torch.empty_like(q, memory_format=torch.contiguous_format)
    _need(out, "out", torch.bfloat16, 4)
    if return_lse and lse is None:
        lse = torch.empty((B, Hq, n), dtype=torch.float32, device=q.device)
    flags = ((FLAG_DENSE if dense else 0) | (FLAG_COUNT if counters is not None else 0)
             | (FLAG_MFMA16 if variant == "mfma16x16x32" else 0))
    cut = None if cutoffs is None else _cut(cutoffs, d, G)
    strides = list(q.stride()[:3]) + list(k.stride()[:3]) + list(v.stride()[:3]) + list(out.stride()[:3])
    _check(lib().wp_prefill(
        _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, n, Hq, Hkv, d, _i64arr(strides), cut,
        int(G), flags, _ptr(counters), _stream(q)))
    return (out, lse) if return_lse else out


def prefill_backward(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
                     dout: torch.Tensor, lse: torch.Tensor, cutoffs: Optional[Sequence[int]], G: int,
                     dense: bool = False, workspace: Optional[torch.Tensor] = None,
                     out: Optional[Sequence[torch.Tensor]] = None):
    """Gradients (dq, dk, dv) of <dout, o> for wp_prefill's inputs; o and lse
    [B, Hq, n] (natural log) from the forward pass.  out: optional (dq, dk,
    dv) tensors (views allowed) to write into."""
    for t, nm in ((q, "q"), (k, "k"), (v, "v"), (o, "o"), (dout, "dout")):
        _need(t, nm, torch.bfloat16, 4)
    _need(lse, "lse", torch.float32, 3)
    B, n, Hq, d = q.shape
    Hkv = k.shape[2]
    if (tuple(k.shape) != (B, n, Hkv, d) or tuple(v.shape) != (B, n, Hkv, d)
            or tuple(o.shape) != (B, n, Hq, d) or tuple(dout.shape) != (B, n, Hq, d)):
        raise ValueError("q/o/dout [B, n, Hq, d_h] and k/v [B, n, Hkv, d_h] must match")
    if tuple(lse.shape) != (B, Hq, n) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous [B, Hq, n] tensor")
    need = lib().wp_prefill_backward_workspace_size(B, n, Hq)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
        dk = torch.empty_like(k, memory_format=torch.contiguous_format)
        dv = torch.empty_like(v, memory_format=torch.contiguous_format)
    else:
        dq, dk, dv = out
        for t, nm in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
            _need(t, nm, torch.bfloat16, 4)
        if tuple(dq.shape) != (B, n, Hq, d) or tuple(dk.shape) != (B, n, Hkv, d) or tuple(dv.shape) != (B, n, Hkv, d):
            raise ValueError("out must be (dq [B, n, Hq, d_h], dk [B, n, Hkv, d_h], dv [B, n, Hkv, d_h])")
    strides = []
    for t in (q, k, v, o, dout, dq, dk, dv):
        strides += list(t.stride()[:3])
    cut = None if cutoffs is None else _cut(cutoffs, d, G)
    _check(lib().wp_prefill_backward(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk), _ptr(dv),
        B, n, Hq, Hkv, d, _i64arr(strides), cut, int(G), FLAG_DENSE if dense else 0, _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q)))
    return dq, dk, dv


def decode(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
           cache_len: torch.Tensor, q_pos: torch.Tensor, cutoffs: Optional[Sequence[int]], G: int,
           dense: bool = False, num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
           counters: Optional[torch.Tensor] = None,
           out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """One query token per sequence.  q [B, Hq, d_h]; caches [B, Lmax, Hkv,
    d_h]; cache_len, q_pos: device int32 [B]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, Hq, d = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Lmax, Hkv, d) or tuple(v_cache.shape) != (B, Lmax, Hkv, d):
        raise ValueError("k_cache and v_cache must be [B, Lmax, Hkv, d_h]")
    need = decode_workspace_size(B, Lmax, Hq, Hkv, d, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    flags = (FLAG_DENSE if dense else 0) | (FLAG_COUNT if counters is not None else 0)
    cut = None if cutoffs is None else _cut(cutoffs, d, G)
    strides = (list(q.stride()[:2]) + list(k_cache.stride()[:3]) + list(v_cache.stride()[:3])
               + list(out.stride()[:2]))
    _check(lib().wp_decode(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(cache_len), _ptr(q_pos), B, Lmax, Hq,
        Hkv, d, _i64arr(strides), cut, int(G), int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), flags, _ptr(counters), _stream(q)))
    return out


def decode_noalloc(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                   cache_len: torch.Tensor, q_pos: torch.Tensor, cutoffs: Optional[Sequence[int]], G: int,
                   dense: bool = False, num_splits: int = 0, counters: Optional[torch.Tensor] = None,
                   out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """wp_decode_noalloc: decode with the partial results in the library's
    fixed device scratch (no workspace).  With `out` given, the call
    allocates nothing on the device."""
    _need(q, "q", torch.bfloat16, 3)
    _need(k_cache, "k_cache", torch.bfloat16, 4)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, Hq, d = q.shape
    Lmax, Hkv = k_cache.shape[1], k_cache.shape[2]
    if tuple(k_cache.shape) != (B, Lmax, Hkv, d) or tuple(v_cache.shape) != (B, Lmax, Hkv, d):
        raise ValueError("k_cache and v_cache must be [B, Lmax, Hkv, d_h]")
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    flags = (FLAG_DENSE if dense else 0) | (FLAG_COUNT if counters is not None else 0)
    cut = None if cutoffs is None else _cut(cutoffs, d, G)
    strides = (list(q.stride()[:2]) + list(k_cache.stride()[:3]) + list(v_cache.stride()[:3])
               + list(out.stride()[:2]))
    _check(lib().wp_decode_noalloc(
        _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(out), _ptr(cache_len), _ptr(q_pos), B, Lmax, Hq,
        Hkv, d, _i64arr(strides), cut, int(G), int(num_splits), flags, _ptr(counters), _stream(q)))
    return out


def kcache_layout(Lmax: int, d_h: int, G: int, cutoffs: Sequence[int]):
    """Ring sizes (caps[ng]) and element offsets (offsets[ng+1]) of the
    group-major compact K store of one (sequence, kv head)."""
    ng = d_h // G
    caps = (ctypes.c_int32 * max(ng, 1))()
    offs = (ctypes.c_int64 * (ng + 1))()
    _check(lib().wp_kcache_layout(int(Lmax), int(d_h), int(G), _cut(cutoffs, d_h, G), caps, offs))
    return [int(v) for v in caps[:ng]], [int(v) for v in offs]


def kcache_empty(B: int, Hkv: int, Lmax: int, d_h: int, G: int, cutoffs: Sequence[int],
                 device=None) -> torch.Tensor:
    """An uninitialised compact K store [B, Hkv, elements] (bf16)."""
    _, offs = kcache_layout(Lmax, d_h, G, cutoffs)
    return torch.empty((B, Hkv, offs[-1]), dtype=torch.bfloat16, device=device)


def kcache_append(k: torch.Tensor, pos0: torch.Tensor, store: torch.Tensor, Lmax: int,
                  cutoffs: Sequence[int], G: int) -> torch.Tensor:
    """Write k [B, T, Hkv, d_h] (rotated bf16) at positions pos0[b] + t
    (device int32 [B]) into the compact store [B, Hkv, elements]."""
    _need(k, "k", torch.bfloat16, 4)
    _need(pos0, "pos0", torch.int32, 1)
    _need(store, "store", torch.bfloat16, 3)
    B, T, Hkv, d = k.shape
    if store.shape[0] != B or store.shape[1] != Hkv or store.stride(2) != 1:
        raise ValueError("store must be [B, Hkv, elements] (elements contiguous) matching k")
    _check(lib().wp_kcache_append(
        _ptr(k), B, T, Hkv, d, _i64arr(list(k.stride()[:3])), _ptr(pos0), _ptr(store),
        _i64arr(list(store.stride()[:2])), int(Lmax), _cut(cutoffs, d, G), int(G), _stream(k)))
    return store


def decode_kcache(q: torch.Tensor, store: torch.Tensor, v_cache: torch.Tensor,
                  cache_len: torch.Tensor, q_pos: torch.Tensor, cutoffs: Sequence[int], G: int,
                  num_splits: int = 0, workspace: Optional[torch.Tensor] = None,
                  counters: Optional[torch.Tensor] = None,
                  out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """wp_decode with K from the compact store [B, Hkv, elements]; v_cache
    [B, Lmax, Hkv, d_h]."""
    _need(q, "q", torch.bfloat16, 3)
    _need(store, "store", torch.bfloat16, 3)
    _need(v_cache, "v_cache", torch.bfloat16, 4)
    _need(cache_len, "cache_len", torch.int32, 1)
    _need(q_pos, "q_pos", torch.int32, 1)
    B, Hq, d = q.shape
    Lmax, Hkv = v_cache.shape[1], v_cache.shape[2]
    if (tuple(v_cache.shape) != (B, Lmax, Hkv, d) or store.shape[0] != B or store.shape[1] != Hkv
            or store.stride(2) != 1):
        raise ValueError("v_cache must be [B, Lmax, Hkv, d_h] and store [B, Hkv, elements]")
    need = decode_workspace_size(B, Lmax, Hq, Hkv, d, num_splits)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    if out is None:
        out = torch.empty((B, Hq, d), dtype=torch.bfloat16, device=q.device)
    _need(out, "out", torch.bfloat16, 3)
    flags = FLAG_COUNT if counters is not None else 0
    strides = (list(q.stride()[:2]) + list(store.stride()[:2]) + list(v_cache.stride()[:3])
               + list(out.stride()[:2]))
    _check(lib().wp_decode_kcache(
        _ptr(q), _ptr(store), _ptr(v_cache), _ptr(out), _ptr(cache_len), _ptr(q_pos), B, Lmax, Hq,
        Hkv, d, _i64arr(strides), _cut(cutoffs, d, G), int(G), int(num_splits), _ptr(workspace),
        workspace.numel() * workspace.element_size(), flags, _ptr(counters), _stream(q)))
    return out
