"""GPU: one Ulysses sequence-parallel attention layer simulated on one device.

P virtual ranks each hold a shard of N / P tokens with all Ht heads (the layout
of sequence parallelism). Each packs its shard into P head groups
(`vdit_pack_heads`); the all-to-all is simulated with device copies (rank r
receives head group r of every rank's shard, i.e. all N tokens of its Ht / P
heads); each rank runs the attention over its heads; the reverse exchange sends
token block s of each rank's output back to rank s, which unpacks it
(`vdit_unpack_heads`) into [N / P, Ht, d]. The layer must equal, bit for bit, one
all-heads attention call on the unsharded tensors (the pages: sequence
parallelism is numerically equivalent to a single GPU), and match the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synthetic_inputs as si
from test_gpu_parity import as_f64, check, down, note, up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this environment")
    import long_sequence_attention_amd as vd
    vd.load_library()
    return torch.device("cuda:0")


def ulysses_layer(vd, q, k, v, degree, key_len=None):
    """Sequence-parallel attention over `degree` virtual ranks; returns [N, Ht, d]."""
    n, ht, d = q.shape
    nk = k.shape[0]
    tq, tk = n // degree, nk // degree
    # per rank: token shards packed into head groups, [P, tokens/P, Ht/P, d]
    packed = [[vd.pack_heads(x[r * t:(r + 1) * t].contiguous(), degree) for r in range(degree)]
              for x, t in ((q, tq), (k, tk), (v, tk))]
    outs = []
    for r in range(degree):
        # all-to-all: rank r gathers head group r of every rank's shard, in token order
        qr, kr, vr = (torch.cat([p[s][r] for s in range(degree)], dim=0) for p in packed)
        hb, hc = vd.ulysses_heads(ht, degree, r)
        assert hc == ht // degree and hb == r * hc
        attn = vd.Attention(n, nk, hc, d, use_key_mask=key_len is not None)
        outs.append(attn.forward(qr, kr, vr, key_len=key_len or 0))  # [N, Ht/P, d]
    # reverse all-to-all: rank s collects token block s of every rank's output
    shards = []
    for s in range(degree):
        back = torch.stack([outs[r][s * tq:(s + 1) * tq] for r in range(degree)])  # [P, N/P, Ht/P, d]
        shards.append(vd.unpack_heads(back))                                       # [N/P, Ht, d]
    torch.cuda.synchronize()
    return torch.cat(shards, dim=0)


@pytest.mark.parametrize("degree", [2, 4, 8])
def test_ulysses_layer_equals_single_device(dev, degree):
    import long_sequence_attention_amd as vd
    n, ht, d = 8192, 40, 128
    note(f"Ulysses layer on {degree} virtual ranks, N={n} Ht={ht} d={d}")
    qb = si.normal_bf16((n, ht, d), 7800, si.STREAM_Q)
    kb = si.normal_bf16((n, ht, d), 7800, si.STREAM_K)
    vb = si.normal_bf16((n, ht, d), 7800, si.STREAM_V)
    q, k, v = up(qb, dev), up(kb, dev), up(vb, dev)
    layer = ulysses_layer(vd, q, k, v, degree)
    single = vd.Attention(n, n, ht, d).forward(q, k, v)
    torch.cuda.synchronize()
    assert np.array_equal(down(layer), down(single)), "sequence-parallel layer differs from the single-device call"
    rows = si.sample_rows(n, 128, 7800, si.tile_edge_rows(n))
    got = as_f64(layer[torch.from_numpy(rows).to(dev)])
    check(got, oracle.mha_reference(qb, kb, vb, rows=rows), f"Ulysses layer P={degree}")


def test_ulysses_layer_text_cross_attention(dev):
    # query tokens sharded, text keys and values sharded too (every rank gathers them
    # all with its head group), one key length
    import long_sequence_attention_amd as vd
    n, nk, ht, d, L, degree = 12000, 512, 40, 128, 300, 4
    note(f"Ulysses cross-attention layer on {degree} virtual ranks, N={n} Nk={nk} L={L}")
    q = up(si.normal_bf16((n, ht, d), 7900, si.STREAM_Q), dev)
    k = up(si.normal_bf16((nk, ht, d), 7900, si.STREAM_K), dev)
    v = up(si.normal_bf16((nk, ht, d), 7900, si.STREAM_V), dev)
    layer = ulysses_layer(vd, q, k, v, degree, key_len=L)
    single = vd.Attention(n, nk, ht, d, use_key_mask=True).forward(q, k, v, key_len=L)
    torch.cuda.synchronize()
    assert np.array_equal(down(layer), down(single))
