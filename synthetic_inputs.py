"""Seeded synthetic inputs for the video-DiT attention workloads.

This module is shared by the tests, the benchmark and the oracle checks, and it
holds none of the attention arithmetic: it only draws normal numbers, rounds
them to bfloat16 bit patterns, draws the key length of the cross-attention case
and picks the query rows that a sampled check looks at.

Recipe (the same for every workload):
  * values are float32 standard normals times ``sigma``, rounded to bfloat16 by
    round-to-nearest-even;
  * a tensor is drawn in C order of its own layout ([N, H, d] or the packed
    [N, 3, H, d]), in chunks of ``CHUNK`` elements; chunk ``c`` of stream ``s``
    under seed ``seed`` comes from PCG64 seeded with SeedSequence([seed, s, c]),
    so the result does not depend on the number of worker threads;
  * q, k and v of one workload use streams 0, 1 and 2 (a packed tensor uses
    stream 0 for the whole [N, 3, H, d] draw).
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

CHUNK = 1 << 22

STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaN inputs map to a quiet NaN.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    bias = np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    out = ((u + bias) >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = np.uint16(0x7FC0)
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _worker_count() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def normal_bf16(shape, seed: int, stream: int, sigma: float = 1.0) -> np.ndarray:
    """Draw a bfloat16 tensor of i.i.d. N(0, sigma^2) values; returns uint16 bits."""
    shape = tuple(int(s) for s in shape)
    total = int(np.prod(shape)) if shape else 1
    out = np.empty(total, dtype=np.uint16)
    nchunks = (total + CHUNK - 1) // CHUNK
    sig = np.float32(sigma)

    def fill(c: int) -> None:
        lo = c * CHUNK
        hi = min(total, lo + CHUNK)
        rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, stream, c])))
        x = rng.standard_normal(hi - lo, dtype=np.float32)
        if sig != np.float32(1.0):
            x *= sig
        out[lo:hi] = f32_to_bf16_bits(x)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(max_workers=_worker_count()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def key_length(seed: int, lo: int = 64, hi: int = 512) -> int:
    """Valid key length drawn uniformly from the integers in [lo, hi]."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 1_000_000])))
    return int(rng.integers(lo, hi + 1))


def sample_rows(n: int, count: int, seed: int, forced=()) -> np.ndarray:
    """Sorted distinct query rows: ``count`` drawn without replacement plus ``forced``.

    Forced rows outside [0, n) are dropped; if ``count >= n`` every row is returned.
    """
    if count >= n:
        return np.arange(n, dtype=np.int64)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 2_000_000])))
    rows = rng.choice(n, size=count, replace=False)
    extra = np.array([r for r in forced if 0 <= r < n], dtype=np.int64)
    return np.unique(np.concatenate([rows.astype(np.int64), extra]))


def tile_edge_rows(n: int) -> tuple:
    """Rows at the 64/128-row tile edges and at the ragged end of an n-row sequence."""
    cands = [0, 1, 63, 64, 127, 128, 255, 256, n - 81, n - 80, n - 65, n - 64, n - 2, n - 1]
    return tuple(sorted({c for c in cands if 0 <= c < n}))
