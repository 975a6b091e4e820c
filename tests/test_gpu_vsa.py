"""GPU: block-sparse attention over 64-token tiles (vdit_vsa_*) against the oracle.

The tile selection is an integer decided in float32 with a fixed order on both
sides, so it must match the oracle exactly; the attention output is held to the
parity tolerances of the dense path (max |d| <= 2e-2, relL1 <= 2e-3 against the
unrounded float64 oracle). Keeping every tile must give dense attention.
"""
import ctypes
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


def test_hand_fixture_selection_and_output(dev):
    """tests/golden/vsa_tile_selection.json, embedded in d = 64 (zeros elsewhere)."""
    vd = vdm()
    with open(os.path.join(ROOT, "tests", "golden", "vsa_tile_selection.json")) as f:
        fx = json.load(f)
    n, d = fx["n"], 64
    note(f"vsa hand fixture n={n} d={d}")
    x = {key: np.zeros((n, 1, d), dtype=np.float32) for key in ("q", "k", "v")}
    for key, name in (("q", "q_tile_tokens"), ("k", "k_tile_tokens")):
        for t, toks in enumerate(fx[name]):
            for r in range(t * 64, min((t + 1) * 64, n)):
                x[key][r, 0, :len(toks[0])] = toks[(r - t * 64) % len(toks)]
    for t, val in enumerate(fx["v_tile_value"]):
        x["v"][t * 64:min((t + 1) * 64, n), 0, :len(val)] = val
    q, k, v = (si.f32_to_bf16_bits(x[key]) for key in ("q", "k", "v"))
    attn = vd.Attention(n, n, 1, d, scale=0.5)
    for keep, want in fx["selection"].items():
        tiles = attn.vsa_select(up(q, dev), up(k, dev), keep=int(keep))
        torch.cuda.synchronize()
        assert tiles.cpu().numpy()[0].tolist() == want, f"keep={keep}"
        out = attn.vsa_attend(up(q, dev), up(k, dev), up(v, dev), tiles=tiles)
        torch.cuda.synchronize()
        ref, _ = oracle.vsa_reference(q, k, v, tiles=np.array([want]), scale=0.5)
        check(as_f64(out), ref, f"hand fixture keep={keep}")


@pytest.mark.parametrize("n,ht,d,h0,hc,keep,seed", [
    (4096, 10, 128, 0, 10, 13, 3001),          # the N=4096 workload at sparsity 0.8
    (64 * 37 + 19, 3, 64, 1, 2, 9, 3002),      # ragged last tile, head share, d = 64
    (64 * 5 + 1, 2, 128, 0, 2, 1, 3003),       # one-token last tile, one kept tile
])
def test_selection_and_output_match_oracle(dev, n, ht, d, h0, hc, keep, seed):
    vd = vdm()
    note(f"vsa n={n} Ht={ht} d={d} heads {h0}-{h0 + hc - 1} keep={keep} seed {seed}")
    q, k, v = inputs(n, ht, d, seed)
    attn = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc)
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    tiles = attn.vsa_select(qd, kd, keep=keep)
    out = attn.vsa_attend(qd, kd, vd_, tiles=tiles)
    out2 = attn.vsa_forward(qd, kd, vd_, keep=keep)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, k, head_begin=h0, head_count=hc, keep=keep)
    got = tiles.cpu().numpy()
    assert got.shape == want.shape
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"selection differs at (head, query tile) {bad[:5].tolist()}"
    assert np.array_equal(down(out), down(out2)), "vsa_forward differs from select + attend"
    ref, _ = oracle.vsa_reference(q, k, v, head_begin=h0, head_count=hc, tiles=want)
    check(as_f64(out), ref, f"vsa n={n} keep={keep}")


def test_selection_with_many_ties_across_chunks(dev):
    """600 key tiles (the select kernel holds them in chunks of 256 per thread block)
    whose tiles are constant vectors of small integers, so the coarse scores are
    small exact integers with many ties: the kept tiles must still equal the
    oracle's, ties going to the lower tile."""
    vd = vdm()
    n, d, keep = 64 * 600, 64, 100
    rng = np.random.default_rng(3050)
    qt = rng.integers(-1, 2, (600, 1, 4)).astype(np.float32)
    kt = rng.integers(0, 3, (600, 1, 4)).astype(np.float32)
    q = np.zeros((n, 1, d), dtype=np.float32)
    k = np.zeros((n, 1, d), dtype=np.float32)
    q[:, :, :4] = np.repeat(qt, 64, axis=0)
    k[:, :, :4] = np.repeat(kt, 64, axis=0)
    qb, kb = si.f32_to_bf16_bits(q), si.f32_to_bf16_bits(k)
    attn = vd.Attention(n, n, 1, d)
    tiles = attn.vsa_select(up(qb, dev), up(kb, dev), keep=keep)
    torch.cuda.synchronize()
    want = oracle.vsa_select(qb, kb, keep=keep)
    scores = np.repeat(qt[:, 0], 1, axis=0) @ kt[:, 0].T
    assert len(np.unique(scores)) < 20   # the test really is about ties
    assert np.array_equal(tiles.cpu().numpy(), want)


def test_selection_n131072_2048_tiles(dev):
    """The packed RoPE workload's length without RoPE: 2048 key tiles, two heads."""
    vd = vdm()
    n, ht, d = 32 * 64 * 64, 2, 128
    q = si.normal_bf16((n, ht, d), 3060, si.STREAM_Q)
    k = si.normal_bf16((n, ht, d), 3060, si.STREAM_K)
    attn = vd.Attention(n, n, ht, d)
    keep = attn.vsa_keep(0.8)
    note(f"vsa selection N={n} tiles={attn.k_tiles} keep={keep}")
    tiles = attn.vsa_select(up(q, dev), up(k, dev), keep=keep)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, k, keep=keep)
    assert np.array_equal(tiles.cpu().numpy(), want)


@pytest.mark.parametrize("n", [1, 63, 64, 65, 129, 200])
@pytest.mark.parametrize("d", [64, 128])
def test_degenerate_and_ragged_sizes(dev, n, d):
    """One token, one partial tile, exactly one tile, a one-token last tile..., with
    one kept tile and with all of them."""
    vd = vdm()
    q, k, v = inputs(n, 2, d, 3070 + n)
    attn = vd.Attention(n, n, 2, d)
    for keep in sorted({1, attn.k_tiles}):
        out = attn.vsa_forward(up(q, dev), up(k, dev), up(v, dev), keep=keep)
        tiles = attn.vsa_select(up(q, dev), up(k, dev), keep=keep)
        torch.cuda.synchronize()
        want = oracle.vsa_select(q, k, keep=keep)
        assert np.array_equal(tiles.cpu().numpy(), want), (n, d, keep)
        ref, _ = oracle.vsa_reference(q, k, v, tiles=want)
        check(as_f64(out), ref, f"vsa n={n} d={d} keep={keep}")


def test_keep_count_matches_oracle(dev):
    vd = vdm()
    for n, s in ((75600, 0.8), (4096, 0.8), (4096, 0.0), (131072, 0.8), (130, 0.5), (64, 0.9)):
        attn = vd.Attention(n, n, 1, 64)
        assert attn.vsa_keep(s) == ovsa.keep_count(s, (n + 63) // 64), (n, s)
    with pytest.raises(vd.VditError):
        attn.vsa_keep(1.0)


@pytest.mark.parametrize("n", [4096, 64 * 9 + 30])
def test_keeping_every_tile_matches_dense_attention(dev, n):
    """All tiles kept: the oracle's dense attention, and the dense kernel within
    the parity bound (the sparse kernel splits each tile's keys between two waves
    with their own softmax references, so the roundings differ)."""
    vd = vdm()
    ht, d = 4, 128
    note(f"vsa keep all tiles n={n}")
    q, k, v = inputs(n, ht, d, 3010 + n)
    attn = vd.Attention(n, n, ht, d)
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    tk = attn.k_tiles
    tiles = torch.arange(tk, dtype=torch.int32, device=dev).repeat(ht, attn.q_tiles, 1).contiguous()
    sparse = attn.vsa_attend(qd, kd, vd_, tiles=tiles)
    dense = attn.forward(qd, kd, vd_)
    sel = attn.vsa_select(qd, kd, keep=tk)
    torch.cuda.synchronize()
    assert (sel == tiles).all()
    ref = oracle.mha_reference(q, k, v)
    check(as_f64(sparse), ref, f"all tiles kept n={n}")
    assert float((sparse.float() - dense.float()).abs().max()) <= 2e-2


def test_masked_key_half_and_retry(dev):
    """n = 64 * 5 + 16: the last tile has 16 keys, so the second key half of that
    tile is all masked. Kept alone, that half contributes nothing; listed first
    (before other tiles), its -inf reference forces the exact-maximum retry. And
    keys that grow from tile to tile overflow the first tile's reference."""
    vd = vdm()
    n, ht, d = 64 * 5 + 16, 2, 128
    q, k, v = inputs(n, ht, d, 3040)
    attn = vd.Attention(n, n, ht, d)
    tq, tk = attn.q_tiles, attn.k_tiles
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    alone = np.full((ht, tq, 1), tk - 1, dtype=np.int32)
    first = np.tile(np.array([tk - 1, 0, 2], dtype=np.int32), (ht, tq, 1))
    for name, tl in (("ragged tile alone", alone), ("ragged tile listed first", first)):
        note(f"vsa {name}")
        out = attn.vsa_attend(qd, kd, vd_, tiles=torch.from_numpy(tl).to(dev))
        torch.cuda.synchronize()
        ref, _ = oracle.vsa_reference(q, k, v, tiles=tl)
        check(as_f64(out), ref, f"vsa {name}")
    # growing keys: tile t scaled by 1 + 8 t (scores far above the first tile's)
    kf = si.bf16_bits_to_f32(k).copy()
    for t in range(tk):
        kf[t * 64:(t + 1) * 64] *= 1 + 8 * t
    kg = si.f32_to_bf16_bits(kf)
    kgd = up(kg, dev)
    tiles = attn.vsa_select(qd, kgd, keep=3)
    out = attn.vsa_attend(qd, kgd, vd_, tiles=tiles)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, kg, keep=3)
    assert np.array_equal(tiles.cpu().numpy(), want)
    ref, _ = oracle.vsa_reference(q, kg, v, tiles=want)
    check(as_f64(out), ref, "vsa growing keys")


def test_packed_layout_and_batch_equal_single_calls(dev):
    vd = vdm()
    B, n, ht, d, keep = 2, 64 * 20 + 5, 2, 128, 4
    note(f"vsa packed B={B} n={n} keep={keep}")
    qkv = [si.normal_bf16((n, 3, ht, d), 3020 + i, si.STREAM_Q) for i in range(B)]
    attn = vd.Attention(n, n, ht, d, layout="N3HD", batch=B)
    both = up(np.stack(qkv), dev)
    tiles = attn.vsa_select(both, keep=keep)
    out = attn.vsa_forward(both, keep=keep)
    torch.cuda.synchronize()
    assert tuple(tiles.shape) == (B, ht, attn.q_tiles, keep)
    one = vd.Attention(n, n, ht, d, layout="N3HD")
    for i in range(B):
        t1 = one.vsa_select(up(qkv[i], dev), keep=keep)
        o1 = one.vsa_forward(up(qkv[i], dev), keep=keep)
        torch.cuda.synchronize()
        assert torch.equal(tiles[i], t1)
        assert np.array_equal(down(out[i]), down(o1)), f"entry {i}"
        want = oracle.vsa_select(qkv[i], layout="N3HD", keep=keep)
        assert np.array_equal(t1.cpu().numpy(), want)
        ref, _ = oracle.vsa_reference(qkv[i], layout="N3HD", tiles=want)
        check(as_f64(o1), ref, f"packed entry {i}")


@pytest.mark.timeout(900)
def test_ulysses_share_n75600_sparsity_08(dev):
    vd = vdm()
    n, ht, h0, hc, d = 21 * 45 * 80, 40, 0, 10, 128
    q, k, v = inputs(n, ht, d, 1003)
    attn = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc)
    keep = attn.vsa_keep(0.8)
    note(f"vsa N={n} heads 0-9 of 40 sparsity 0.8 keep={keep}")
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    tiles = attn.vsa_select(qd, kd, keep=keep)
    out = attn.vsa_attend(qd, kd, vd_, tiles=tiles)
    torch.cuda.synchronize()
    want = oracle.vsa_select(q, k, head_begin=h0, head_count=hc, keep=keep)
    got = tiles.cpu().numpy()
    bad = np.argwhere((got != want).any(axis=2))
    assert bad.size == 0, f"selection differs at (head, query tile) {bad[:5].tolist()}"
    # rows of 48 query tiles: the first, the last (ragged) and 46 drawn at random
    tq = attn.q_tiles
    rng = np.random.default_rng(1003)
    qt = np.unique(np.concatenate([[0, tq - 1], rng.choice(tq, 46, replace=False)]))
    rows = np.unique(np.concatenate([np.minimum(t * 64 + np.array([0, 1, 31, 32, 63]), n - 1) for t in qt] +
                                    [rng.integers(t * 64, min(t * 64 + 64, n), 11) for t in qt]))
    ref, _ = oracle.vsa_reference(q, k, v, head_begin=h0, head_count=hc, rows=rows, tiles=want)
    check(as_f64(out[torch.from_numpy(rows).to(dev)]), ref, f"vsa N={n} ({len(rows)} rows x {hc} heads)")


def test_out_of_range_tiles_are_clamped(dev):
    vd = vdm()
    n, ht, d, keep = 64 * 6 + 10, 1, 64, 2
    q, k, v = inputs(n, ht, d, 3030)
    attn = vd.Attention(n, n, ht, d)
    tq, tk = attn.q_tiles, attn.k_tiles
    wild = torch.tensor([[-5, 3]] + [[1, 10 ** 6]] * (tq - 1), dtype=torch.int32).reshape(1, tq, keep).to(dev)
    tame = torch.tensor([[0, 3]] + [[1, tk - 1]] * (tq - 1), dtype=torch.int32).reshape(1, tq, keep).to(dev)
    qd, kd, vd_ = up(q, dev), up(k, dev), up(v, dev)
    a = attn.vsa_attend(qd, kd, vd_, tiles=wild)
    b = attn.vsa_attend(qd, kd, vd_, tiles=tame)
    torch.cuda.synchronize()
    assert np.array_equal(down(a), down(b))


def test_vsa_call_errors(dev):
    vd = vdm()
    from long_sequence_attention_amd import _lib
    lib = _lib.load()
    INVALID, UNSUPPORTED, WORKSPACE = 1, 2, 6
    n, ht, d = 64 * 4, 2, 64
    q = torch.zeros((n, ht, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros_like(q)
    masked = vd.Attention(n, n, ht, d, use_key_mask=True)
    with pytest.raises(vd.VditError) as e:
        masked.vsa_select(q, k, keep=1)
    assert e.value.code == UNSUPPORTED
    attn = vd.Attention(n, n, ht, d)
    for keep, code in ((0, INVALID), (5, INVALID)):
        with pytest.raises(vd.VditError) as e:
            attn.vsa_workspace_bytes(keep)
        assert e.value.code == code, keep
    big = vd.Attention(64 * 4097, 64 * 4097, 1, 64)
    assert big.vsa_workspace_bytes(4096) > 0
    with pytest.raises(vd.VditError) as e:
        big.vsa_workspace_bytes(4097)
    assert e.value.code == UNSUPPORTED
    huge = vd.Attention(64 * 8193, 64 * 8193, 1, 64)
    with pytest.raises(vd.VditError) as e:
        huge.vsa_keep(0.8) and huge.vsa_workspace_bytes(1)
    assert e.value.code == UNSUPPORTED
    small_ws = torch.empty(attn.workspace_bytes, dtype=torch.uint8, device=dev)
    with pytest.raises(vd.VditError) as e:
        attn.vsa_select(q, k, keep=2, workspace=small_ws)
    assert e.value.code == WORKSPACE
    tiles = torch.zeros((ht, attn.q_tiles, 2), dtype=torch.int32, device=dev)
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_vsa_workspace(2, dev)
    st = lib.vdit_vsa_attend(attn._h, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                             ctypes.c_void_p(k.data_ptr()), 2, ctypes.c_void_p(out.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == INVALID, "tiles overlapping out must be rejected"
    st = lib.vdit_vsa_select(attn._h, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()), 2,
                             ctypes.c_void_p(ws.data_ptr()), ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == INVALID, "tiles inside the workspace must be rejected"
    torch.cuda.synchronize()
    assert tiles.shape[-1] == 2
