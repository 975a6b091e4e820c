"""Pins of the block-sparse (64-token tile) oracle, oracle/vsa.py, against things
other than itself:

  * hand-computed tile means, coarse scores and selections with ties
    (tests/golden/vsa_tile_selection.json);
  * a closed form of the fine stage on the same inputs (keys and values constant
    per tile: the output is a weighted mean of a few distinct values);
  * the float32 selection equals the exact (float64) top-k wherever the gap at the
    cut exceeds the float32 error bound;
  * keeping every tile reduces to the dense attention oracle;
  * brute force (explicit loops, math.exp) on tiny random inputs;
  * permuting whole key tiles permutes the selection and leaves the output alone;
  * cube tiles of a latent grid: hand-computed cube token lists, means, scores and
    selections on a ragged grid (tests/golden/vsa_cube_selection.json), brute force
    over grid coordinates, keep-all equal to dense attention, and whole cubes equal to
    64-token tiles of the cube-ordered tokens.

Mutations planted on the CPU (ties broken the other way, the ragged tile divided
by 64, the query tile used as the key tile) show that the pins catch them.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import vsa
import synthetic_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def fixture():
    with open(os.path.join(ROOT, "tests", "golden", "vsa_tile_selection.json")) as f:
        return json.load(f)


def build_tiles(fx, key, n, d, heads=1):
    """bfloat16 bit patterns [n, heads, d]: tile t cycles through fx[key][t]."""
    x = np.zeros((n, heads, d), dtype=np.float32)
    for t, toks in enumerate(fx[key]):
        for r in range(t * 64, min((t + 1) * 64, n)):
            x[r, :, :len(toks[0])] = toks[(r - t * 64) % len(toks)]
    return si.f32_to_bf16_bits(x)


def build_values(fx, n, d):
    x = np.zeros((n, 1, d), dtype=np.float32)
    for t, val in enumerate(fx["v_tile_value"]):
        x[t * 64:min((t + 1) * 64, n), 0, :len(val)] = val
    return si.f32_to_bf16_bits(x)


def test_keep_count_values():
    assert vsa.keep_count(0.8, 1182) == 237      # 236.4 rounded up
    assert vsa.keep_count(0.8, 5) == 1
    assert vsa.keep_count(0.0, 7) == 7
    assert vsa.keep_count(0.5, 3) == 2
    assert vsa.keep_count(0.75, 4) == 1
    assert vsa.keep_count(0.999, 10) == 1
    with pytest.raises(ValueError):
        vsa.keep_count(1.0, 4)


def test_hand_means_scores_and_selection():
    fx = fixture()
    n, d = fx["n"], fx["d"]
    q = build_tiles(fx, "q_tile_tokens", n, d)[:, 0, :]
    k = build_tiles(fx, "k_tile_tokens", n, d)[:, 0, :]
    qm, km = vsa.tile_means_f32(q), vsa.tile_means_f32(k)
    assert qm.tolist() == fx["q_tile_means"]
    assert km.tolist() == fx["k_tile_means"]
    assert vsa.coarse_scores_f32(qm, km).tolist() == fx["coarse_scores"]
    for keep, want in fx["selection"].items():
        got = oracle.vsa_select(q[:, None, :], k[:, None, :], keep=int(keep))
        assert got.shape == (1, 4, int(keep))
        assert got[0].tolist() == want, f"keep={keep}"


def test_hand_fine_stage_closed_form():
    """Keys take at most two distinct values per tile and values are constant per
    tile, so out = sum over distinct (key, value) groups of count * e^(s) * value,
    divided by sum of count * e^(s)."""
    fx = fixture()
    n, d = fx["n"], fx["d"]
    q = build_tiles(fx, "q_tile_tokens", n, d)
    k = build_tiles(fx, "k_tile_tokens", n, d)
    v = build_values(fx, n, d)
    scale = 0.5
    for keep in (1, 2, 3):
        out, tiles = oracle.vsa_reference(q, k, v, keep=keep, scale=scale)
        sel = fx["selection"][str(keep)]
        assert tiles[0].tolist() == sel
        for row in (0, 63, 64, 130, 192, 193, 199):
            qv = fx["q_tile_tokens"][row // 64]
            qrow = qv[(row - (row // 64) * 64) % len(qv)]
            num = [0.0] * d
            den = 0.0
            for j in sel[row // 64]:
                toks = fx["k_tile_tokens"][j]
                cnt = min(64, n - j * 64)
                for m, kv in enumerate(toks):
                    c = sum(1 for r in range(cnt) if r % len(toks) == m)
                    w = c * math.exp(scale * sum(a * b for a, b in zip(qrow, kv)))
                    den += w
                    for e in range(d):
                        num[e] += w * fx["v_tile_value"][j][e]
            want = [x / den for x in num]
            assert np.allclose(out[row, 0], want, rtol=1e-13, atol=1e-15), (keep, row)


def test_selection_matches_exact_topk_outside_the_error_bound():
    n, ht, d = 64 * 37 + 19, 2, 128
    q = si.normal_bf16((n, ht, d), 2101, si.STREAM_Q)
    k = si.normal_bf16((n, ht, d), 2101, si.STREAM_K)
    keep = 9
    sel = oracle.vsa_select(q, k, keep=keep)
    checked = 0
    for h in range(ht):
        qx = oracle.bf16_bits_to_f64(q[:, h, :])
        kx = oracle.bf16_bits_to_f64(k[:, h, :])
        tq = (n + 63) // 64
        qm = np.stack([qx[t * 64:(t + 1) * 64].mean(axis=0) for t in range(tq)])
        km = np.stack([kx[t * 64:(t + 1) * 64].mean(axis=0) for t in range(tq)])
        qa = np.stack([np.abs(qx[t * 64:(t + 1) * 64]).mean(axis=0) for t in range(tq)])
        ka = np.stack([np.abs(kx[t * 64:(t + 1) * 64]).mean(axis=0) for t in range(tq)])
        exact = qm @ km.T
        # float32 error bound: a mean of n terms is off by at most (n + 1) u mean|x|,
        # a d-term dot product by d u sum|a b| (u = 2^-24), doubled for the cross terms
        u = 2.0 ** -24
        bound = 2 * u * (65 * (qa @ np.abs(km).T + np.abs(qm) @ ka.T) + d * (np.abs(qm) @ np.abs(km).T))
        for i in range(tq):
            order = np.argsort(-exact[i], kind="stable")
            gap = exact[i, order[keep - 1]] - exact[i, order[keep]]
            if gap > 2 * bound[i].max():
                assert sel[h, i].tolist() == sorted(order[:keep].tolist()), (h, i)
                checked += 1
    assert checked > 60


def test_keep_all_tiles_is_dense_attention():
    n, ht, d = 64 * 3 + 21, 3, 64
    q = si.normal_bf16((n, ht, d), 2102, si.STREAM_Q)
    k = si.normal_bf16((n, ht, d), 2102, si.STREAM_K)
    v = si.normal_bf16((n, ht, d), 2102, si.STREAM_V)
    out, tiles = oracle.vsa_reference(q, k, v, head_begin=1, head_count=2, sparsity=0.0)
    assert tiles.shape == (2, 4, 4) and (tiles == np.arange(4)).all()
    dense = oracle.mha_reference(q, k, v, head_begin=1, head_count=2)
    assert np.allclose(out, dense, rtol=1e-12, atol=1e-14)


def test_brute_force_tiny():
    n, d = 150, 8
    q = si.normal_bf16((n, 1, d), 2103, si.STREAM_Q)
    k = si.normal_bf16((n, 1, d), 2103, si.STREAM_K)
    v = si.normal_bf16((n, 1, d), 2103, si.STREAM_V)
    rows = [0, 5, 63, 64, 100, 127, 128, 149]
    out, tiles = oracle.vsa_reference(q, k, v, keep=2, rows=rows)
    qx, kx, vx = (oracle.bf16_bits_to_f64(t[:, 0, :]).tolist() for t in (q, k, v))
    scale = 1.0 / math.sqrt(d)
    for r_i, r in enumerate(rows):
        keys = [j for j in range(n) if j // 64 in tiles[0][r // 64]]
        s = [scale * sum(qx[r][c] * kx[j][c] for c in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        want = [sum(wi * vx[j][c] for wi, j in zip(w, keys)) / sum(w) for c in range(d)]
        assert np.allclose(out[r_i, 0], want, rtol=1e-12, atol=1e-14), r


def test_key_tile_permutation_invariance():
    n, ht, d = 64 * 6, 1, 64
    q = si.normal_bf16((n, ht, d), 2104, si.STREAM_Q)
    k = si.normal_bf16((n, ht, d), 2104, si.STREAM_K)
    v = si.normal_bf16((n, ht, d), 2104, si.STREAM_V)
    perm = np.array([3, 0, 5, 1, 4, 2])
    rows_of = np.concatenate([np.arange(p * 64, (p + 1) * 64) for p in perm])
    out, tiles = oracle.vsa_reference(q, k, v, keep=2)
    out_p, tiles_p = oracle.vsa_reference(q, k[rows_of], v[rows_of], keep=2)
    # new tile t holds old tile perm[t]
    assert [sorted(perm[t].tolist()) for t in tiles_p[0]] == tiles[0].tolist()
    assert np.allclose(out, out_p, rtol=1e-12, atol=1e-14)


def test_nan_scores_rank_lowest_and_negative_zero_ties():
    s = np.array([[np.nan, -0.0, 0.0, -1.0]], dtype=np.float32)
    assert vsa.select_tiles(s, 1).tolist() == [[1]]      # -0 and +0 tie: lower index
    assert vsa.select_tiles(s, 3).tolist() == [[1, 2, 3]]
    assert vsa.select_tiles(s, 4).tolist() == [[0, 1, 2, 3]]


def cube_fixture():
    with open(os.path.join(ROOT, "tests", "golden", "vsa_cube_selection.json")) as f:
        return json.load(f)


def cube_inputs(grid):
    """q = (t, y, x, 1) and k = (2 [t = 4], 2 [y = 4], 0, w) per token, as bfloat16 bits [n, 1, 4]."""
    T, H, W = grid
    q = np.zeros((T * H * W, 1, 4), dtype=np.float32)
    k = np.zeros_like(q)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                n = (t * H + y) * W + x
                q[n, 0] = (t, y, x, 1)
                w = -6.0 if (t == 4 and y == 4) else x - 1.5
                k[n, 0] = (2.0 if t == 4 else 0.0, 2.0 if y == 4 else 0.0, 0.0, w)
    return si.f32_to_bf16_bits(q), si.f32_to_bf16_bits(k)


def test_hand_cube_tokens_means_scores_and_selection():
    fx = cube_fixture()
    grid = tuple(fx["grid"])
    cubes = vsa.cube_tiles(grid)
    assert [c.tolist() for c in cubes] == fx["cube_tokens"]
    q, k = cube_inputs(grid)
    qm = vsa.group_means_f32(q[:, 0, :], cubes)
    km = vsa.group_means_f32(k[:, 0, :], cubes)
    assert qm.tolist() == fx["q_cube_means"]
    assert km.tolist() == fx["k_cube_means"]
    assert vsa.coarse_scores_f32(qm, km).tolist() == fx["coarse_scores"]
    for keep, want in fx["selection"].items():
        got = oracle.vsa_select(q, k, keep=int(keep), grid=grid)
        assert got.shape == (1, 4, int(keep))
        assert got[0].tolist() == want, f"keep={keep}"


def test_cube_brute_force_ragged_grid():
    """Grid 5 x 6 x 7 cuts cubes on all three sides (8 cubes of 64, 48, 32, 24, 16, 12,
    8 and 6 tokens). Brute force: cube membership from each token's coordinates,
    float32 means and scores one operation at a time, a sorted() selection, and the
    fine stage with math.exp."""
    grid = (5, 6, 7)
    T, H, W = grid
    n, d, keep = T * H * W, 8, 3
    q = si.normal_bf16((n, 1, d), 2105, si.STREAM_Q)
    k = si.normal_bf16((n, 1, d), 2105, si.STREAM_K)
    v = si.normal_bf16((n, 1, d), 2105, si.STREAM_V)
    qx, kx, vx = (oracle.bf16_bits_to_f64(a[:, 0, :]) for a in (q, k, v))
    ncx, ncy = (W + 3) // 4, (H + 3) // 4
    members = {}
    for tok in range(n):
        t, y, x = tok // (H * W), (tok // W) % H, tok % W
        members.setdefault((t // 4 * ncy + y // 4) * ncx + x // 4, []).append(tok)
    cubes = [members[c] for c in sorted(members)]
    assert sorted(len(c) for c in cubes) == [6, 8, 12, 16, 24, 32, 48, 64]

    def mean32(x, toks):
        out = []
        for c in range(d):
            s = np.float32(0.0)
            for tok in toks:
                s = np.float32(s + np.float32(x[tok, c]))
            out.append(np.float32(s / np.float32(len(toks))))
        return out

    qm = [mean32(qx, c) for c in cubes]
    km = [mean32(kx, c) for c in cubes]
    want_tiles = []
    for i in range(len(cubes)):
        sc = []
        for j in range(len(cubes)):
            s = np.float32(0.0)
            for c in range(d):
                s = np.float32(s + np.float32(qm[i][c] * km[j][c]))
            sc.append(float(s))
        want_tiles.append(sorted(sorted(range(len(cubes)), key=lambda j: (-sc[j], j))[:keep]))
    rows = [0, 3, 27, 41, 100, 167, 168, 209]
    out, tiles = oracle.vsa_reference(q, k, v, keep=keep, rows=rows, grid=grid)
    assert tiles[0].tolist() == want_tiles
    scale = 1.0 / math.sqrt(d)
    cube_of = {tok: ci for ci, c in enumerate(cubes) for tok in c}
    for r_i, r in enumerate(rows):
        keys = [tok for j in want_tiles[cube_of[r]] for tok in cubes[j]]
        s = [scale * sum(qx[r, c] * kx[j, c] for c in range(d)) for j in keys]
        m = max(s)
        w = [math.exp(x - m) for x in s]
        want = [sum(wi * vx[j, c] for wi, j in zip(w, keys)) / sum(w) for c in range(d)]
        assert np.allclose(out[r_i, 0], want, rtol=1e-12, atol=1e-14), r


def test_cube_keep_all_is_dense_attention():
    grid = (3, 5, 9)
    n = 3 * 5 * 9
    q = si.normal_bf16((n, 2, 16), 2106, si.STREAM_Q)
    k = si.normal_bf16((n, 2, 16), 2106, si.STREAM_K)
    v = si.normal_bf16((n, 2, 16), 2106, si.STREAM_V)
    out, tiles = oracle.vsa_reference(q, k, v, sparsity=0.0, grid=grid)
    assert tiles.shape == (2, 6, 6) and (tiles == np.arange(6)).all()
    assert np.allclose(out, oracle.mha_reference(q, k, v), rtol=1e-12, atol=1e-14)


def test_whole_cubes_are_64_token_tiles_in_cube_order():
    grid = (8, 4, 8)
    n = 256
    q = si.normal_bf16((n, 1, 32), 2107, si.STREAM_Q)
    k = si.normal_bf16((n, 1, 32), 2107, si.STREAM_K)
    v = si.normal_bf16((n, 1, 32), 2107, si.STREAM_V)
    perm = np.concatenate(vsa.cube_tiles(grid))
    assert sorted(perm.tolist()) == list(range(n)) and perm.tolist() != list(range(n))
    out_c, tiles_c = oracle.vsa_reference(q, k, v, keep=2, grid=grid)
    out_r, tiles_r = oracle.vsa_reference(q[perm], k[perm], v[perm], keep=2)
    assert tiles_c.tolist() == tiles_r.tolist()
    assert np.array_equal(out_c[perm], out_r)


# ---- planted mistakes: each must fail a pin above

def test_mutation_ties_to_higher_index_is_caught(monkeypatch):
    def select_desc(scores, keep):
        s = np.asarray(scores, dtype=np.float32) + np.float32(0.0)
        out = []
        for row in s:
            order = np.lexsort((-np.arange(row.size), -row.astype(np.float64)))
            out.append(sorted(order[:keep].tolist()))
        return np.array(out, dtype=np.int32)
    monkeypatch.setattr(vsa, "select_tiles", select_desc)
    with pytest.raises(AssertionError):
        test_hand_means_scores_and_selection()


def test_mutation_ragged_tile_divided_by_64_is_caught(monkeypatch):
    def means_64(x_bits, groups):
        x = oracle.bf16_bits_to_f64(x_bits).astype(np.float32)
        return np.stack([x[g].sum(axis=0, dtype=np.float32) / np.float32(64) for g in groups])
    monkeypatch.setattr(vsa, "group_means_f32", means_64)
    with pytest.raises(AssertionError):
        test_hand_means_scores_and_selection()
    with pytest.raises(AssertionError):
        test_hand_cube_tokens_means_scores_and_selection()


def test_mutation_query_tile_as_key_tile_is_caught(monkeypatch):
    real = vsa.sparse_rows

    def wrong(q, k, v, scale, q_tiles, tiles, key_groups=None):
        diag = np.stack([np.full(tiles.shape[1], t) for t in range(tiles.shape[0])])
        return real(q, k, v, scale, q_tiles, np.minimum(diag, (k.shape[0] - 1) // 64), key_groups)
    monkeypatch.setattr(vsa, "sparse_rows", wrong)
    with pytest.raises(AssertionError):
        test_brute_force_tiny()


def test_mutation_cubes_numbered_ct_fastest_is_caught(monkeypatch):
    real = vsa.cube_tiles

    def transposed(grid):
        cubes = real(grid)
        T, H, W = (int(g) for g in grid)
        nct, ncy, ncx = (T + 3) // 4, (H + 3) // 4, (W + 3) // 4
        return [cubes[(ct * ncy + cy) * ncx + cx] for cx in range(ncx) for cy in range(ncy) for ct in range(nct)]
    monkeypatch.setattr(vsa, "cube_tiles", transposed)
    with pytest.raises(AssertionError):
        test_hand_cube_tokens_means_scores_and_selection()
