"""GPU: block-sparse attention over 4x4x4 cubes of the latent grid (vsa_cubes)
against the oracle.

As for 64-token tiles, the cube selection is decided in float32 with a fixed order
on both sides and must match the oracle exactly; the output is held to the dense
path's parity tolerances (max |d| <= 2e-2, relL1 <= 2e-3 against the unrounded
float64 oracle). Grids with sides that are not multiples of 4 give thin edge cubes
(1 to 64 tokens), whose keys past their token count the kernel masks.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import vsa as ovsa
import synthetic_inputs as si
from test_gpu_parity import as_f64, check, down, note, up

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import long_sequence_attention_amd as vd
    vd.load_library()
    return torch.device("cuda:0")


def vdm():
    import long_sequence_attention_amd as vd
    return vd


def inputs(n, ht, d, seed, sigma=1.0):
    return (si.normal_bf16((n, ht, d), seed, si.STREAM_Q, sigma),
            si.normal_bf16((n, ht, d), seed, si.STREAM_K, sigma),
            si.normal_bf16((n, ht, d), seed, si.STREAM_V, sigma))


def ncubes(grid):
    return len(ovsa.cube_tiles(grid))


def cube_rows(grid, cubes, rng, per_cube=6):
    """Query rows of the listed cubes: each cube's first and last token and a few drawn
    at random."""
    tiles = ovsa.cube_tiles(grid)
    rows = []
    for c in cubes:
        toks = tiles[c]
        rows += [toks[0], toks[-1]] + list(rng.choice(toks, min(per_cube, len(toks)), replace=False))
    return np.unique(np.array(rows, dtype=np.int64))


def test_hand_fixture_selection_and_output(dev):
    """tests/golden/vsa_cube_selection.json (grid 5 x 5 x 4, cubes of 64, 16, 16 and 4
    tokens), embedded in d = 64 (zeros elsewhere)."""
    vd = vdm()
    with open(os.path.join(ROOT, "tests", "golden", "vsa_cube_selection.json")) as f:
        fx = json.load(f)
    grid = tuple(fx["grid"])
    T, H, W = grid
    n, d = T * H * W, 64
    note(f"vsa cubes hand fixture grid={grid} d={d}")
    q = np.zeros((n, 1, d), dtype=np.float32)
    k = np.zeros_like(q)
    v = np.zeros_like(q)
    for t in range(T):
        for y in range(H):
            for x in range(W):
                i = (t * H + y) * W + x
                q[i, 0, :4] = (t, y, x, 1)
                k[i, 0, :4] = (2.0 if t == 4 else 0.0, 2.0 if y == 4 else 0.0, 0.0,
                               -6.0 if (t == 4 and y == 4) else x - 1.5)
                v[i, 0, :3] = (t, y, x)
    q, k, v = (si.f32_to_bf16_bits(a) for a in (q, k, v))
    attn = vd.Attention(n, n, 1, d, scale=0.5, vsa_cubes=grid)
    assert attn.q_tiles == attn.k_tiles == 4
    for keep, want in fx["selection"].items():
        tiles = attn.vsa_select(up(q, dev), up(k, dev), keep=int(keep))
        torch.cuda.synchronize()
        assert tiles.cpu().numpy()[0].tolist() == want, f"keep={keep}"
        out = attn.vsa_attend(up(q, dev), up(k, dev), up(v, dev), tiles=tiles)
        torch.cuda.synchronize()
        ref, _ = oracle.vsa_reference(q, k, v, tiles=np.array([want]), scale=0.5, grid=grid)
        check(as_f64(out), ref, f"cube hand fixture keep={keep}")


@pytest.mark.parametrize("grid,ht,d,h0,hc,keep,seed", [
    ((5, 9, 12), 3, 128, 1, 2, 5, 4001),      # thin cubes along t and y, head share
    ((6, 7, 10), 2, 64, 0, 2, 7, 4002),       # thin along all three sides, d = 64
    ((3, 5, 7), 1, 128, 0, 1, 1, 4003),       # one cube along t (3 frames), one kept cube
    ((8, 16, 16), 2, 128, 0, 2, 4, 4004),     # whole cubes only
])
def test_selection_and_output_match_oracle(dev, grid, ht, d, h0, hc, keep, seed):
    vd = vdm()
    n = int(np.prod(grid))
    note(f"vsa cubes grid={grid} Ht={ht} d={d} heads {h0}-{h0 + hc - 1} keep={keep} seed {seed}")
    q, k, v = inputs(n, ht, d, seed)
    attn = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc, vsa_cubes=grid)
    assert attn.q_tiles == ncubes(grid)
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    tiles = attn.vsa_select(qd, kd, keep=keep)
    out = attn.vsa_attend(qd, kd, vd_, tiles=tiles)
    out2 = attn.vsa_forward(qd, kd, vd_, keep=keep)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, k, head_begin=h0, head_count=hc, keep=keep, grid=grid)
    got = tiles.cpu().numpy()
    assert got.shape == want.shape
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"selection differs at (head, query cube) {bad[:5].tolist()}"
    assert np.array_equal(down(out), down(out2)), "vsa_forward differs from select + attend"
    ref, _ = oracle.vsa_reference(q, k, v, head_begin=h0, head_count=hc, tiles=want, grid=grid)
    check(as_f64(out), ref, f"vsa cubes grid={grid} keep={keep}")


def test_thin_cube_listed_first(dev):
    """Grid 8 x 5 x 8: cubes 2, 3, 6 and 7 are one row high (16 tokens), so in the first
    kept tile of the lists below the second key half is empty; the two waves of a
    query block share the reference of the whole tile. Also a thin cube kept alone."""
    vd = vdm()
    grid = (8, 5, 8)
    n, ht, d = 320, 2, 128
    q, k, v = inputs(n, ht, d, 4010)
    attn = vd.Attention(n, n, ht, d, vsa_cubes=grid)
    tq = attn.q_tiles
    assert [len(c) for c in ovsa.cube_tiles(grid)] == [64, 64, 16, 16, 64, 64, 16, 16]
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    first = np.tile(np.array([2, 4, 5], dtype=np.int32), (ht, tq, 1))
    alone = np.full((ht, tq, 1), 7, dtype=np.int32)
    for name, tl in (("thin cube listed first", first), ("thin cube alone", alone)):
        note(f"vsa cubes {name}")
        out = attn.vsa_attend(qd, kd, vd_, tiles=torch.from_numpy(tl).to(dev))
        torch.cuda.synchronize()
        ref, _ = oracle.vsa_reference(q, k, v, tiles=tl, grid=grid)
        check(as_f64(out), ref, f"vsa cubes {name}")


def test_keep_all_cubes_matches_dense_attention(dev):
    vd = vdm()
    grid = (5, 9, 12)
    n, ht, d = 540, 2, 128
    note(f"vsa cubes keep-all grid={grid}")
    q, k, v = inputs(n, ht, d, 4020)
    attn = vd.Attention(n, n, ht, d, vsa_cubes=grid)
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    out = attn.vsa_forward(qd, kd, vd_, sparsity=0.0)
    dense = attn.forward(qd, kd, vd_)
    torch.cuda.synchronize()
    ref = oracle.mha_reference(q, k, v)
    check(as_f64(out), ref, "vsa cubes keep-all vs oracle")
    check(as_f64(dense), ref, "dense call of a cube plan vs oracle")


def test_batch_and_head_share_equal_single_calls(dev):
    """Batch entries and a head share give the rows of the matching single calls bit
    for bit (the per-row arithmetic does not depend on the batch or the head count)."""
    vd = vdm()
    grid = (6, 9, 8)
    B, n, ht, d, keep = 2, 432, 4, 128, 5
    note(f"vsa cubes batch B={B} grid={grid}")
    qkv = [inputs(n, ht, d, 4030 + i) for i in range(B)]
    attn = vd.Attention(n, n, ht, d, batch=B, vsa_cubes=grid)
    qb, kb, vb = (up(np.stack([x[j] for x in qkv]), dev) for j in range(3))
    out = attn.vsa_forward(qb, kb, vb, keep=keep)
    share = vd.Attention(n, n, ht, d, head_begin=1, head_count=2, vsa_cubes=grid)
    one = vd.Attention(n, n, ht, d, vsa_cubes=grid)
    for i in range(B):
        q, k, v = (up(a, dev) for a in qkv[i])
        o1 = one.vsa_forward(q, k, v, keep=keep)
        osh = share.vsa_forward(q, k, v, keep=keep)
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(o1)), f"batch entry {i}"
        assert np.array_equal(down(osh), down(o1[:, 1:3])), f"head share, entry {i}"


@pytest.mark.timeout(900)
def test_ulysses_share_n75600_cubes_sparsity_08(dev):
    """The workload's grid, 21 x 45 x 80: 6 x 12 x 20 = 1440 cubes (thin along t and y:
    21 = 4 * 5 + 1 frames, 45 = 4 * 11 + 1 rows), keep = 288 at sparsity 0.8."""
    vd = vdm()
    grid = (21, 45, 80)
    n, ht, h0, hc, d = 75600, 40, 0, 10, 128
    q, k, v = inputs(n, ht, d, 1003)
    attn = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc, vsa_cubes=grid)
    keep = attn.vsa_keep(0.8)
    assert attn.q_tiles == 1440 and keep == 288
    note(f"vsa cubes N={n} grid={grid} heads 0-9 of 40 keep={keep}")
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    tiles = attn.vsa_select(qd, kd, keep=keep)
    out = attn.vsa_attend(qd, kd, vd_, tiles=tiles)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, k, head_begin=h0, head_count=hc, keep=keep, grid=grid)
    got = tiles.cpu().numpy()
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"selection differs at (head, query cube) {bad[:5].tolist()}"
    # rows of the first and last cube, thin cubes (the last frame, the last row of
    # cubes) and cubes drawn at random: at least 4096 rows
    rng = np.random.default_rng(1003)
    tq = attn.q_tiles
    cubes = np.unique(np.concatenate([[0, 19, 220, 239, 1200, 1439], rng.choice(tq, 320, replace=False)]))
    rows = cube_rows(grid, cubes, rng, per_cube=14)
    assert len(rows) >= 4096
    ref, _ = oracle.vsa_reference(q, k, v, head_begin=h0, head_count=hc, rows=rows, tiles=want, grid=grid)
    check(as_f64(out[torch.from_numpy(rows).to(dev)]), ref, f"vsa cubes N={n} ({len(rows)} rows x {hc} heads)")


def test_packed_layout_equals_separate(dev):
    """The packed [N, 3, Ht, d] layout with cube tiles gives the separate layout's bits."""
    vd = vdm()
    grid = (5, 6, 9)
    n, ht, d, keep = 270, 2, 128, 3
    note(f"vsa cubes packed grid={grid} keep={keep}")
    qkv = si.normal_bf16((n, 3, ht, d), 4040, si.STREAM_Q)
    packed = vd.Attention(n, n, ht, d, layout="N3HD", vsa_cubes=grid)
    sep = vd.Attention(n, n, ht, d, vsa_cubes=grid)
    both = up(qkv, dev)
    tp = packed.vsa_select(both, keep=keep)
    op = packed.vsa_forward(both, keep=keep)
    q, k, v = (up(np.ascontiguousarray(qkv[:, j]), dev) for j in range(3))
    ts = sep.vsa_select(q, k, keep=keep)
    os_ = sep.vsa_forward(q, k, v, keep=keep)
    torch.cuda.synchronize()
    assert torch.equal(tp, ts)
    assert np.array_equal(down(op), down(os_))
    want = oracle.vsa_select(qkv, layout="N3HD", keep=keep, grid=grid)
    assert np.array_equal(tp.cpu().numpy(), want)
    ref, _ = oracle.vsa_reference(qkv, layout="N3HD", tiles=want, grid=grid)
    check(as_f64(op), ref, "vsa cubes packed")
