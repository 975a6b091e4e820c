"""Float64 reference for non-causal multi-head attention with optional key-length
mask, head-group selection and 3D RoPE — test infrastructure only (see package
docstring). Nothing here is tuned for speed beyond using numpy's matmul as the
dot-product primitive.
"""
from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64.

    A bfloat16 value is the top 16 bits of a float32, so placing the pattern in
    the high half of a 32-bit word gives the float32 value exactly.
    """
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def ulysses_head_range(heads_total: int, degree: int, rank: int) -> tuple[int, int]:
    """Head share [begin, begin + count) of ``rank`` under Ulysses sequence parallelism.

    fal.ai, "Generate video with WAN 2.2 across four GPUs", section "Splitting one
    generation across four GPUs": after the all-to-all each of the four GPUs holds
    the whole sequence for 10 of the 40 heads. Section "Tuning cost and GPU count":
    the degree has to divide the head count. Ranks take consecutive equal shares.
    Pinned by the page's own numbers (tests/golden/ulysses_head_shares.json).
    """
    if degree <= 0 or heads_total <= 0 or heads_total % degree != 0:
        raise ValueError("Ulysses degree must be positive and divide the head count")
    if not 0 <= rank < degree:
        raise ValueError("rank out of range")
    count = heads_total // degree
    return rank * count, count


# ---------------------------------------------------------------------------
# 3D RoPE. Reading used (the pages do not write it down): token n of a
# (T, H, W) latent grid, w fastest, sits at t = n // (H*W), y = (n // W) % H,
# x = n % W. The head dimension is cut into three consecutive bands of widths
# (D_t, D_h, D_w) (44/42/42 at d = 128); band b is an ordinary 1-D rotary
# embedding of its own position, rotating the adjacent pair (2i, 2i+1) of the
# band by theta = pos * base^(-2i / D_b), i in [0, D_b / 2).
# Parity with any real model's RoPE convention is unpinned (no model here).
# ---------------------------------------------------------------------------

def rope_grid_position(tokens, grid) -> np.ndarray:
    """Integer (t, y, x) of each token index on a (T, H, W) grid, w fastest."""
    T, H, W = (int(g) for g in grid)
    n = np.asarray(tokens, dtype=np.int64)
    t = n // (H * W)
    y = (n // W) % H
    x = n % W
    return np.stack([t, y, x], axis=-1)


def rope_pair_bands(head_dim: int, dims) -> np.ndarray:
    """For each rotated pair p in [0, head_dim/2): (band, i, band_width)."""
    dims = [int(v) for v in dims]
    if sum(dims) != head_dim or any(v <= 0 or v % 2 for v in dims):
        raise ValueError("bands must be positive, even and sum to the head dim")
    rows = []
    for band, width in enumerate(dims):
        for i in range(width // 2):
            rows.append((band, i, width))
    return np.array(rows, dtype=np.int64)


def rope_index_table(tokens, grid, head_dim: int, dims) -> np.ndarray:
    """int32 [len(tokens), head_dim/2, 5]: (t, y, x, band, i) for each (token, pair)."""
    pos = rope_grid_position(tokens, grid)              # [R, 3]
    pb = rope_pair_bands(head_dim, dims)                # [P, 3]
    R, P = pos.shape[0], pb.shape[0]
    out = np.empty((R, P, 5), dtype=np.int32)
    out[:, :, 0:3] = pos[:, None, :]
    out[:, :, 3] = pb[None, :, 0]
    out[:, :, 4] = pb[None, :, 1]
    return out


def rope_apply(u: np.ndarray, tokens, grid, dims, base: float) -> np.ndarray:
    """Rotate the last axis of ``u`` (float64, [R, ..., d]) for tokens ``tokens`` [R].

    Pair (a, b) = (u[o + 2i], u[o + 2i + 1]) of band (pos, o, D) becomes
    (a cos(theta) - b sin(theta), a sin(theta) + b cos(theta)),
    theta = pos * base ** (-2 i / D).
    """
    u = np.asarray(u, dtype=np.float64)
    d = u.shape[-1]
    pos = rope_grid_position(tokens, grid).astype(np.float64)   # [R, 3]
    out = u.copy()
    offset = 0
    for band, width in enumerate(int(v) for v in dims):
        i = np.arange(width // 2, dtype=np.float64)
        inv_freq = float(base) ** (-2.0 * i / width)             # [D/2]
        theta = pos[:, band][:, None] * inv_freq[None, :]         # [R, D/2]
        shape = (u.shape[0],) + (1,) * (u.ndim - 2) + (width // 2,)
        c = np.cos(theta).reshape(shape)
        s = np.sin(theta).reshape(shape)
        a = u[..., offset:offset + width:2]
        b = u[..., offset + 1:offset + width:2]
        out[..., offset:offset + width:2] = a * c - b * s
        out[..., offset + 1:offset + width:2] = a * s + b * c
        offset += width
    if offset != d:
        raise ValueError("bands must cover the head dim")
    return out


# ---------------------------------------------------------------------------
# Attention.
# ---------------------------------------------------------------------------

def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                   key_len: int | None = None, row_block: int = 256) -> np.ndarray:
    """Exact two-pass softmax attention for one head: q [R, d], k/v [Nk, d] -> [R, d]."""
    L = k.shape[0] if key_len is None else int(key_len)
    if not 1 <= L <= k.shape[0]:
        raise ValueError("key length must be in [1, Nk]")
    kL, vL = k[:L], v[:L]
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for r0 in range(0, q.shape[0], row_block):
        qb = q[r0:r0 + row_block]
        s = (qb @ kL.T) * scale                 # pass 1: scores and their max
        m = s.max(axis=1, keepdims=True)
        e = np.exp(s - m)                       # pass 2: weights, their sum, weighted values
        l = e.sum(axis=1, keepdims=True)
        out[r0:r0 + row_block] = (e @ vL) / l
    return out


def _split_inputs(q_bits, k_bits, v_bits, layout: str):
    if layout == "NHD":
        return q_bits, k_bits, v_bits
    if layout == "N3HD":
        if k_bits is not None or v_bits is not None:
            raise ValueError("packed layout takes the [N, 3, H, d] tensor alone")
        return q_bits[:, 0], q_bits[:, 1], q_bits[:, 2]
    raise ValueError("layout must be 'NHD' or 'N3HD'")


def mha_reference(q_bits, k_bits=None, v_bits=None, *, layout: str = "NHD",
                  head_begin: int = 0, head_count: int | None = None,
                  rows=None, key_len: int | None = None, scale: float | None = None,
                  rope=None, progress=None) -> np.ndarray:
    """Float64 attention output [R, head_count, d] for the selected query rows.

    q_bits/k_bits/v_bits are bfloat16 bit patterns (uint16) in [N, H, d] layout, or
    one packed [N, 3, H, d] tensor in ``q_bits`` (layout "N3HD"). ``rows`` selects
    the query tokens (default: all). ``rope`` is None or a dict with keys
    ``grid`` (T, H, W), ``dims`` (three even band widths) and ``base``; it rotates
    q and k, never v. The result is not rounded.
    """
    qb, kb, vb = _split_inputs(q_bits, k_bits, v_bits, layout)
    Nq, Ht, d = qb.shape
    hc = Ht - head_begin if head_count is None else int(head_count)
    if not (0 <= head_begin and hc >= 1 and head_begin + hc <= Ht):
        raise ValueError("head range out of bounds")
    if kb.shape[1] != Ht or vb.shape != kb.shape or kb.shape[2] != d:
        raise ValueError("q, k, v shapes disagree")
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    Nk = kb.shape[0]
    L = Nk if key_len is None else int(key_len)
    out = np.empty((rows.shape[0], hc, d), dtype=np.float64)
    key_tokens = np.arange(L, dtype=np.int64)
    for j, h in enumerate(range(head_begin, head_begin + hc)):
        q = bf16_bits_to_f64(qb[rows, h, :])
        k = bf16_bits_to_f64(kb[:L, h, :])
        v = bf16_bits_to_f64(vb[:L, h, :])
        if rope is not None:
            q = rope_apply(q, rows, rope["grid"], rope["dims"], rope["base"])
            k = rope_apply(k, key_tokens, rope["grid"], rope["dims"], rope["base"])
        out[:, j, :] = attention_rows(q, k, v, sc, L)
        if progress is not None:
            progress(j + 1, hc)
    return out
