"""GPU: several sequences per call (the batch axis, e.g. the positive and negative
conditioning of classifier-free guidance).

Every batch entry must equal, bit for bit, the same problem run alone (B = 1),
and match the float64 oracle to the parity tolerances; per-entry key lengths
must mask exactly their own keys.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from test_gpu_parity import as_f64, check, down, note, up, workspace_layout

pytestmark = pytest.mark.gpu


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


def entries(b, n, nk, ht, d, seed, sigma=1.0):
    """B independent (q, k, v) problems, entry i drawn from seed + i."""
    return [(si.normal_bf16((n, ht, d), seed + i, si.STREAM_Q, sigma),
             si.normal_bf16((nk, ht, d), seed + i, si.STREAM_K, sigma),
             si.normal_bf16((nk, ht, d), seed + i, si.STREAM_V, sigma)) for i in range(b)]


def stack(dev, arrs):
    return up(np.stack(arrs), dev)


@pytest.mark.parametrize("d", [64, 128])
def test_batch_self_attention_equals_single_calls(dev, d):
    vd = vdm()
    B, n, ht, h0, hc = 3, 700, 4, 1, 2
    note(f"batch self-attention B={B} n={n} Ht={ht} heads {h0}-{h0 + hc - 1} d={d}")
    es = entries(B, n, n, ht, d, 4100 + d)
    attn = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc, batch=B)
    out = attn.forward(stack(dev, [e[0] for e in es]), stack(dev, [e[1] for e in es]),
                       stack(dev, [e[2] for e in es]))
    torch.cuda.synchronize()
    assert tuple(out.shape) == (B, n, hc, d)
    for i, (q, k, v) in enumerate(es):
        single = vd.Attention(n, n, ht, d, head_begin=h0, head_count=hc).forward(up(q, dev), up(k, dev), up(v, dev))
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(single)), f"entry {i} differs from its single call"
        check(as_f64(out[i]), oracle.mha_reference(q, k, v, head_begin=h0, head_count=hc), f"batch entry {i}")


def test_batch_cross_attention_per_entry_key_lengths(dev):
    vd = vdm()
    B, nq, nk, ht, d = 2, 600, 512, 4, 128
    lens = [512, 77]
    note(f"batch cross-attention B={B} nq={nq} nk={nk} key_lens={lens}")
    es = entries(B, nq, nk, ht, d, 4200)
    # keys past an entry's length hold NaN: they must not reach any output
    dirty = []
    for (q, k, v), L in zip(es, lens):
        k2, v2 = k.copy(), v.copy()
        k2[L:] = 0x7FC0
        v2[L:] = 0x7FC0
        dirty.append((q, k2, v2))
    attn = vd.Attention(nq, nk, ht, d, use_key_mask=True, batch=B)
    qb, kb, vb = (stack(dev, [e[j] for e in dirty]) for j in range(3))
    out = attn.forward(qb, kb, vb, key_lens=lens)
    ws = attn.prepare(qb, kb, vb, key_lens=lens)
    out2 = attn.attend(qb, kb, vb, key_lens=lens, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(down(out), down(out2)), "prepare_lens + attend_lens differ from fwd_lens"
    for i, ((q, k, v), L) in enumerate(zip(es, lens)):
        single = vd.Attention(nq, nk, ht, d, use_key_mask=True).forward(up(q, dev), up(k, dev), up(v, dev),
                                                                        key_len=L)
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(single)), f"entry {i} (key_len {L}) differs from its single call"
        check(as_f64(out[i]), oracle.mha_reference(q, k, v, key_len=L), f"cross entry {i} L={L}")
    # one key_len for every entry
    out3 = attn.forward(qb, kb, vb, key_len=77)
    torch.cuda.synchronize()
    single = vd.Attention(nq, nk, ht, d, use_key_mask=True).forward(up(es[0][0], dev), up(es[0][1], dev),
                                                                    up(es[0][2], dev), key_len=77)
    torch.cuda.synchronize()
    assert np.array_equal(down(out3[0]), down(single))
    assert np.array_equal(down(out3[1]), down(out[1]))


def test_batch_packed_rope_equals_single_calls(dev):
    vd = vdm()
    B, grid, ht, d = 2, (2, 8, 16), 2, 128
    n = grid[0] * grid[1] * grid[2]
    rope = {"grid": grid, "dims": (44, 42, 42), "base": 10000.0}
    note(f"batch packed RoPE B={B} grid={grid} Ht={ht}")
    qkv = [si.normal_bf16((n, 3, ht, d), 4300 + i, si.STREAM_Q, 0.5) for i in range(B)]
    out = vd.Attention(n, n, ht, d, layout="N3HD", rope=rope, batch=B).forward(stack(dev, qkv))
    torch.cuda.synchronize()
    for i in range(B):
        single = vd.Attention(n, n, ht, d, layout="N3HD", rope=rope).forward(up(qkv[i], dev))
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(single)), f"entry {i} differs from its single call"
        check(as_f64(out[i]), oracle.mha_reference(qkv[i], layout="N3HD", rope=rope), f"packed RoPE entry {i}")


def test_batch_call_errors(dev):
    vd = vdm()
    from long_sequence_attention_amd import _lib
    B, nq, nk, ht, d = 2, 64, 128, 2, 64
    attn = vd.Attention(nq, nk, ht, d, use_key_mask=True, batch=B)
    q = torch.zeros((B, nq, ht, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, nk, ht, d), dtype=torch.bfloat16, device=dev)
    v = torch.zeros_like(k)
    for bad in ([0, 5], [5, nk + 1], [-1, 3]):
        with pytest.raises(vd.VditError) as e:
            attn.forward(q, k, v, key_lens=bad)
        assert e.value.code == 1, bad
    with pytest.raises(ValueError):
        attn.forward(q, k, v, key_lens=[5])
    out = torch.empty(attn.out_shape, dtype=torch.bfloat16, device=dev)
    ws = attn.new_workspace(dev)
    lib = _lib.load()
    st = lib.vdit_attn_fwd_lens(attn._h, ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(k.data_ptr()),
                                ctypes.c_void_p(v.data_ptr()), None, ctypes.c_void_p(out.data_ptr()),
                                ctypes.c_void_p(ws.data_ptr()), ws.numel(), None)
    assert st == 1, "NULL key_lens with the key mask must be rejected"
    with pytest.raises(ValueError):
        attn.forward(q[0], k[0], v[0], key_lens=[5, 5])  # missing batch dimension
    # the workspace grows with the batch, as the header lays it out
    assert attn.workspace_bytes == workspace_layout(B, ht, nq, nk, d)["end"]


@pytest.mark.parametrize("lens", [(512, 200), (100, 512, 300)])
def test_batch_mixed_key_lengths_resident_and_streaming(dev, lens):
    # 16384 queries x 4 heads give every CU a 256-query tile, so entries whose key
    # length fits the LDS array (<= 256 at d = 128) take the keys-resident kernel and
    # the others the streaming one, each launched on its own; every entry must still
    # equal its single call bit for bit
    vd = vdm()
    B, nq, nk, ht, d = len(lens), 16384, 512, 4, 128
    note(f"batch mixed key lengths B={B} nq={nq} key_lens={lens}")
    es = entries(B, nq, nk, ht, d, 4300)
    attn = vd.Attention(nq, nk, ht, d, use_key_mask=True, batch=B)
    out = attn.forward(stack(dev, [e[0] for e in es]), stack(dev, [e[1] for e in es]),
                       stack(dev, [e[2] for e in es]), key_lens=lens)
    torch.cuda.synchronize()
    single = vd.Attention(nq, nk, ht, d, use_key_mask=True)
    rows = si.sample_rows(nq, 512, 4300, si.tile_edge_rows(nq))
    for i, (q, k, v) in enumerate(es):
        o1 = single.forward(up(q, dev), up(k, dev), up(v, dev), key_len=lens[i])
        torch.cuda.synchronize()
        assert np.array_equal(down(out[i]), down(o1)), f"entry {i} (key length {lens[i]})"
        got = as_f64(out[i][torch.from_numpy(rows).to(dev)])
        check(got, oracle.mha_reference(q, k, v, key_len=lens[i], rows=rows), f"entry {i} L={lens[i]}")
