"""Block-sparse attention over 64-token tiles (video sparse attention) — test
infrastructure only (see the package docstring).

Source: FastVideo "Pair two NVIDIA DGX Sparks". Its section "3. Generate one FastH3
clip on both GPUs" names the VSA attention kernels, and its section "Released V2,
FastH3-QAD-v2 and Trim NVFP4 stacks" runs them at sparsity 0.8 with tiles of 64
tokens. The pages state nothing more about the method. The reading implemented here,
the plainest one those two facts support (it is the two-stage scheme of the
published video sparse attention method, without its learned gates), is:

  * tiles are runs of 64 consecutive tokens in the order the tensors hold them;
    the last tile of a sequence whose length is not a multiple of 64 is shorter;
  * coarse stage: each tile of q and of k is summarised by the mean of its
    tokens, and the coarse score of (query tile i, key tile j) is the dot product
    of the two means (the positive softmax scale changes no ranking, so it is
    left out);
  * selection: query tile i keeps the ``keep`` key tiles of highest coarse score,
    keep = ceil((1 - sparsity) * tiles), at least 1; equal scores rank the lower
    tile index first;
  * fine stage: every query of tile i attends, with an exact softmax, over the
    keys of its kept tiles only; its output is that attention alone (the coarse
    attention output and the gates that mix it in need trained weights).

A second tiling, for tokens that lie on a latent video grid (T frames of H x W, token
index (t H + y) W + x, the order the RoPE oracle uses): tiles are 4 x 4 x 4 cubes of the
grid, as in the published video sparse attention method. Cube (ct, cy, cx) holds the
tokens with t // 4 = ct, y // 4 = cy, x // 4 = cx; cubes are numbered with cx fastest, then
cy, then ct. Where a grid side is not a multiple of 4 the last cube along it is thinner
(45 = 4 * 11 + 1 rows: the twelfth row of cubes is one token high), so cubes hold 1 to 64
tokens. The method's reference code pads such cubes to the full tile and masks the pad;
the plainest reading of that, taken here, is that a ragged cube is a tile of its actual
tokens only: its mean divides by its own token count and its keys are its own tokens.
Every other step is the same for both tilings.

The selection is an integer decided by floating point, so this file takes it in
float32, in the order the library computes it:

  mean(tile)[c] = float32(sum) / float32(n), the sum accumulated in float32 one token
                  at a time in ascending token order (n = tokens in the tile)
  score(i, j)   = sum over c of mean_q(i)[c] * mean_k(j)[c], each product and each
                  partial sum rounded to float32, c = 0, 1, ..., d-1 (no fused
                  multiply-add); -0 counts as +0 and NaN as the lowest score

Everything after the selection is float64. Pins: tests/test_oracle_vsa_pins.py
(hand-computed selections with ties, brute force on tiny inputs, the dense
special case, tile-permutation invariance; for cubes: hand-computed cube token lists,
means, scores and selections on a ragged grid, brute force over grid coordinates,
the dense special case, and whole cubes reducing to 64-token tiles of the cube-ordered
tokens).
"""
from __future__ import annotations

import math

import numpy as np

from .attention import _split_inputs, attention_rows, bf16_bits_to_f64

TILE = 64
CUBE = 4


def keep_count(sparsity: float, tiles: int) -> int:
    """Key tiles kept per query tile: ceil((1 - sparsity) * tiles), clamped to [1, tiles]."""
    if not 0.0 <= sparsity < 1.0:
        raise ValueError("sparsity must be in [0, 1)")
    return max(1, min(tiles, math.ceil((1.0 - sparsity) * tiles)))


def run_tiles(n: int, tile: int = TILE) -> list:
    """Token indices of each tile of ``tile`` consecutive tokens (the last may be shorter)."""
    return [np.arange(s, min(s + tile, n), dtype=np.int64) for s in range(0, n, tile)]


def cube_tiles(grid) -> list:
    """Token indices of each 4 x 4 x 4 cube of a (T, H, W) latent grid, cubes numbered
    with cx fastest, then cy, then ct; each cube's tokens ascending."""
    T, H, W = (int(g) for g in grid)
    if min(T, H, W) < 1:
        raise ValueError("grid sides must be positive")
    out = []
    for ct in range(0, T, CUBE):
        for cy in range(0, H, CUBE):
            for cx in range(0, W, CUBE):
                t = np.arange(ct, min(ct + CUBE, T))[:, None, None]
                y = np.arange(cy, min(cy + CUBE, H))[None, :, None]
                x = np.arange(cx, min(cx + CUBE, W))[None, None, :]
                out.append(((t * H + y) * W + x).reshape(-1).astype(np.int64))
    return out


def tiles_of(n: int, grid=None) -> list:
    """The tiling of n tokens: runs of 64 tokens, or the cubes of ``grid``."""
    if grid is None:
        return run_tiles(n)
    if int(np.prod([int(g) for g in grid])) != n:
        raise ValueError("grid does not hold n tokens")
    return cube_tiles(grid)


def group_means_f32(x_bits: np.ndarray, groups) -> np.ndarray:
    """float32 [len(groups), d] means of the bfloat16 rows x [n, d] listed in each group."""
    x = bf16_bits_to_f64(x_bits).astype(np.float32)   # exact: bfloat16 -> float32
    d = x.shape[1]
    count = np.array([len(g) for g in groups], dtype=np.int64)
    idx = np.zeros((len(groups), int(count.max())), dtype=np.int64)
    for i, g in enumerate(groups):
        idx[i, :len(g)] = g
    s = np.zeros((len(groups), d), dtype=np.float32)
    for r in range(idx.shape[1]):                       # token order, float32 adds
        live = r < count
        s[live] = s[live] + x[idx[live, r]]
    return s / count.astype(np.float32)[:, None]        # float32 division


def tile_means_f32(x_bits: np.ndarray, tile: int = TILE) -> np.ndarray:
    """float32 [ceil(n / tile), d] tile means of one head's bfloat16 rows x [n, d]."""
    return group_means_f32(x_bits, run_tiles(x_bits.shape[0], tile))


def coarse_scores_f32(qm: np.ndarray, km: np.ndarray) -> np.ndarray:
    """float32 [Tq, Tk] dot products of tile means, summed over c in order."""
    qm = np.asarray(qm, dtype=np.float32)
    km = np.asarray(km, dtype=np.float32)
    acc = np.zeros((qm.shape[0], km.shape[0]), dtype=np.float32)
    for c in range(qm.shape[1]):
        prod = qm[:, c, None] * km[None, :, c]          # rounded to float32
        acc = acc + prod                                # rounded to float32
    return acc


def select_tiles(scores: np.ndarray, keep: int) -> np.ndarray:
    """int32 [Tq, keep]: per row the ``keep`` highest scores' tile indices, ascending."""
    s = np.asarray(scores, dtype=np.float32) + np.float32(0.0)   # -0 -> +0
    s = np.where(np.isnan(s), np.float32(-np.inf), s)
    tq, tk = s.shape
    if not 1 <= keep <= tk:
        raise ValueError("keep must be in [1, key tiles]")
    out = np.empty((tq, keep), dtype=np.int32)
    idx = np.arange(tk)
    for i in range(tq):
        # primary key: score, descending; secondary: tile index, ascending
        order = np.lexsort((idx, -s[i].astype(np.float64)))
        out[i] = np.sort(order[:keep])
    return out


def vsa_select(q_bits, k_bits=None, *, layout: str = "NHD", head_begin: int = 0,
               head_count: int | None = None, keep: int, grid=None) -> np.ndarray:
    """int32 [head_count, Tq, keep]: kept key tiles of every (head, query tile).
    ``grid`` (T, H, W): cube tiles of that latent grid instead of 64-token runs."""
    if layout == "N3HD":
        qb, kb, _ = _split_inputs(q_bits, None, None, layout)
    else:
        qb, kb = q_bits, k_bits
    Ht = qb.shape[1]
    hc = Ht - head_begin if head_count is None else int(head_count)
    if not (0 <= head_begin and hc >= 1 and head_begin + hc <= Ht):
        raise ValueError("head range out of bounds")
    qg, kg = tiles_of(qb.shape[0], grid), tiles_of(kb.shape[0], grid)
    out = np.empty((hc, len(qg), keep), dtype=np.int32)
    for j, h in enumerate(range(head_begin, head_begin + hc)):
        s = coarse_scores_f32(group_means_f32(qb[:, h, :], qg), group_means_f32(kb[:, h, :], kg))
        out[j] = select_tiles(s, keep)
    return out


def sparse_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
                q_tiles: np.ndarray, tiles: np.ndarray, key_groups=None) -> np.ndarray:
    """float64 [R, d]: each query row r (of query tile q_tiles[r]) attends over the
    keys of the key tiles tiles[q_tiles[r]] (exact softmax). ``key_groups`` lists the
    keys of each tile (default: runs of 64)."""
    kg = run_tiles(k.shape[0]) if key_groups is None else key_groups
    out = np.empty((q.shape[0], v.shape[1]), dtype=np.float64)
    for t in np.unique(q_tiles):
        sel = np.flatnonzero(q_tiles == t)
        keys = np.concatenate([kg[b] for b in tiles[t]])
        out[sel] = attention_rows(q[sel], k[keys], v[keys], scale)
    return out


def vsa_reference(q_bits, k_bits=None, v_bits=None, *, layout: str = "NHD",
                  head_begin: int = 0, head_count: int | None = None, rows=None,
                  keep: int | None = None, sparsity: float | None = None,
                  tiles=None, scale: float | None = None, grid=None):
    """Float64 output [R, head_count, d] of block-sparse attention, and the tiles used.

    ``tiles`` (int [head_count, Tq, keep]) overrides the selection; otherwise it is
    ``vsa_select`` with ``keep`` (or ``keep_count(sparsity, Tk)``). ``grid`` (T, H, W)
    selects the cube tiling of that latent grid. Returns (out, tiles).
    """
    qb, kb, vb = _split_inputs(q_bits, k_bits, v_bits, layout)
    Nq, Ht, d = qb.shape
    hc = Ht - head_begin if head_count is None else int(head_count)
    qg, kg = tiles_of(Nq, grid), tiles_of(kb.shape[0], grid)
    if tiles is None:
        if keep is None:
            keep = keep_count(0.0 if sparsity is None else sparsity, len(kg))
        tiles = vsa_select(qb, kb, head_begin=head_begin, head_count=hc, keep=keep, grid=grid)
    tiles = np.asarray(tiles)
    tile_of_token = np.empty(Nq, dtype=np.int64)
    for i, g in enumerate(qg):
        tile_of_token[g] = i
    sc = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rows = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.empty((rows.shape[0], hc, d), dtype=np.float64)
    for j, h in enumerate(range(head_begin, head_begin + hc)):
        q = bf16_bits_to_f64(qb[rows, h, :])
        k = bf16_bits_to_f64(kb[:, h, :])
        v = bf16_bits_to_f64(vb[:, h, :])
        out[:, j, :] = sparse_rows(q, k, v, sc, tile_of_token[rows], tiles[j], kg)
    return out, tiles
