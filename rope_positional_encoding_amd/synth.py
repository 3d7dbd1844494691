"""Seeded synthetic inputs and the workload table.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
callers.  It holds random-number generation, bf16 rounding of the generated
values and the workload shapes -- nothing of the attention method itself.

Every tensor is generated in chunks of ``CHUNK_ROWS`` rows along its first
(flattened) axis; chunk ``c`` of tensor ``tid`` under workload seed ``seed``
comes from ``numpy.random.default_rng([seed, tid, c])``.  A caller that needs
only a few rows (the sampled-row oracle at 128K) can therefore regenerate just
the chunks that hold them, bit-identically.

Tensor ids: Q = 0, K = 1, V = 2, per-channel std = 3, sampled rows = 4.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Iterable, Sequence

import numpy as np

CHUNK_ROWS = 1024
TID_Q, TID_K, TID_V, TID_STD, TID_ROWS = 0, 1, 2, 3, 4


# ----------------------------------------------------------------------------
# bf16 rounding (round-to-nearest-even), done on the host for every input
# ----------------------------------------------------------------------------
def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> float32 holding the nearest bf16 value (ties to even)."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 (already bf16-exact) -> int16 raw bf16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16).view(np.int16)


def bits_to_f32(b: np.ndarray) -> np.ndarray:
    """int16/uint16 raw bf16 bit patterns -> float32 values."""
    return (np.asarray(b).view(np.uint16).astype(np.uint32) << 16).view(np.float32)


# ----------------------------------------------------------------------------
# chunked normal draws
# ----------------------------------------------------------------------------
def _chunk(seed: int, tid: int, c: int, rows: int, inner: Sequence[int]) -> np.ndarray:
    rng = np.random.default_rng([seed, tid, c])
    return rng.standard_normal((rows, *inner), dtype=np.float32)


def channel_std(seed: int, tid: int, d_h: int) -> np.ndarray:
    """One std per 2-D channel, U[0.5, 2], expanded onto dims (2c, 2c+1)."""
    rng = np.random.default_rng([seed, TID_STD, tid])
    s = rng.uniform(0.5, 2.0, size=d_h // 2).astype(np.float32)
    return np.repeat(s, 2)


def normal_rows(seed: int, tid: int, total_rows: int, inner: Sequence[int],
                rows: Iterable[int] | None = None, std: np.ndarray | None = None,
                round_bf16: bool = True) -> np.ndarray:
    """Rows of an N(0,1) tensor of shape (total_rows, *inner).

    ``rows=None`` returns the whole tensor; otherwise only the listed rows, in
    the order given.  ``std`` (length inner[-1]) scales the last axis.
    """
    inner = tuple(int(v) for v in inner)
    if rows is None:
        out = np.empty((total_rows, *inner), dtype=np.float32)
        for c in range((total_rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
            r0 = c * CHUNK_ROWS
            r1 = min(total_rows, r0 + CHUNK_ROWS)
            out[r0:r1] = _chunk(seed, tid, c, r1 - r0, inner)
    else:
        rows = np.asarray(list(rows), dtype=np.int64)
        out = np.empty((len(rows), *inner), dtype=np.float32)
        cache: dict[int, np.ndarray] = {}
        for k, r in enumerate(rows):
            c = int(r) // CHUNK_ROWS
            if c not in cache:
                r0 = c * CHUNK_ROWS
                r1 = min(total_rows, r0 + CHUNK_ROWS)
                cache[c] = _chunk(seed, tid, c, r1 - r0, inner)
            out[k] = cache[c][int(r) - c * CHUNK_ROWS]
    if std is not None:
        out *= std.astype(np.float32)
    return bf16_round(out) if round_bf16 else out


def normal_bits(seed: int, tid: int, total_rows: int, inner: Sequence[int],
                std: np.ndarray | None = None) -> np.ndarray:
    """Whole tensor as raw bf16 bits (int16), generated chunk by chunk so the
    float32 intermediate never exceeds one chunk."""
    inner = tuple(int(v) for v in inner)
    out = np.empty((total_rows, *inner), dtype=np.int16)
    for c in range((total_rows + CHUNK_ROWS - 1) // CHUNK_ROWS):
        r0 = c * CHUNK_ROWS
        r1 = min(total_rows, r0 + CHUNK_ROWS)
        x = _chunk(seed, tid, c, r1 - r0, inner)
        if std is not None:
            x *= std.astype(np.float32)
        out[r0:r1] = bf16_bits(bf16_round(x))
    return out


# ----------------------------------------------------------------------------
# workloads
# ----------------------------------------------------------------------------
@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str            # "prefill" | "decode"
    seed: int
    B: int
    n: int               # prefill: sequence length; decode: cache length
    Hq: int
    Hkv: int
    d_h: int
    theta: float
    G: int
    pos_scale: float = 1.0
    fp32_inputs: bool = False     # tiny case: Q, K fed to RoPE as fp32
    channel_std: bool = False     # per-channel std U[0.5, 2]
    q_pos: int = 0                # decode: position of the new query token
    oracle_rows: int = 0          # prefill: sampled rows (0 = all rows)


WORKLOADS = {
    "tiny256": Workload("tiny256", "prefill", 1, 1, 256, 1, 1, 64, 1e4, 16,
                        fp32_inputs=True),
    "prefill4k": Workload("prefill4k", "prefill", 2, 1, 4096, 32, 8, 128, 1e6, 16,
                          channel_std=True),
    "prefill32k_g16": Workload("prefill32k_g16", "prefill", 3, 1, 32768, 32, 8, 128,
                               1e6, 16, oracle_rows=256),
    "prefill32k_g32": Workload("prefill32k_g32", "prefill", 3, 1, 32768, 32, 8, 128,
                               1e6, 32, oracle_rows=256),
    "decode32k": Workload("decode32k", "decode", 4, 16, 32768, 32, 8, 128, 1e6, 16,
                          q_pos=32768),
    # the same two shapes under the exact per-channel rule (G = 2)
    "prefill32k_exact": Workload("prefill32k_exact", "prefill", 6, 1, 32768, 32, 8, 128,
                                 1e6, 2, oracle_rows=256),
    "decode32k_exact": Workload("decode32k_exact", "decode", 7, 16, 32768, 32, 8, 128,
                                1e6, 2, q_pos=32768),
    "prefill128k_s4": Workload("prefill128k_s4", "prefill", 5, 1, 131072, 64, 8, 128,
                               1e6, 16, pos_scale=4.0, oracle_rows=128),
}


def sample_rows(n: int, count: int, seed: int, special: Iterable[int] = (),
                tile: int = 64) -> np.ndarray:
    """Sorted, unique query rows: 0, n-1, the caller's special rows (e.g. rows
    at and just past each cutoff) and tile edges, topped up with seeded uniform
    draws to ``count``."""
    picks = {0, n - 1}
    for s in special:
        if 0 <= int(s) < n:
            picks.add(int(s))
    edges = [tile - 1, tile, n // 2 - 1, n // 2, n - tile, n - tile - 1]
    picks.update(e for e in edges if 0 <= e < n)
    rng = np.random.default_rng([seed, TID_ROWS])
    while len(picks) < min(count, n):
        picks.add(int(rng.integers(0, n)))
    return np.array(sorted(picks), dtype=np.int64)


def prefill_shapes(w: Workload):
    """(rows, inner) for Q and for K/V: tensors are [B, n, H, d_h] flattened
    to (B*n, H, d_h)."""
    return (w.B * w.n, (w.Hq, w.d_h)), (w.B * w.n, (w.Hkv, w.d_h))
